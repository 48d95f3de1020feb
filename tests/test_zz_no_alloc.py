"""qmoe_forward_noalloc: the QMoE layer with its workspace in the library's
static per-GPU array, for callers that cannot allocate device memory.

Checked through the C ABI against qmoe_forward on the same inputs (the same
kernels, so the outputs must be bit-identical), on two calls in a row of which
the second is smaller, so that it runs on whatever the first left in the
shared array; the size limit is checked on the host before any device call.
"""
import ctypes
import sys

import numpy as np
import pytest

import synth
import block_quantized_weight_03_amd as mnb

WS_TOO_SMALL = -5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _host_plans(E, H, I, bs):
    keep = []

    def prep(desc, W, s):
        dst = np.zeros(mnb.mnb_prepacked_size(desc) + 512, np.uint8)
        off = (-dst.ctypes.data) % 256
        keep.append(dst)
        return mnb.mnb_prepare_host(desc, W, s, None, dst[off:off + mnb.mnb_prepacked_size(desc)])

    p1 = prep(mnb.qmoe_proj_desc(H, 2 * I, E, bs), synth.int3_rows(1, E * 2 * I, H),
              synth.scales_f16(2, (E * 2 * I, H // bs)))
    p2 = prep(mnb.qmoe_proj_desc(I, H, E, bs), synth.int3_rows(3, E * H, I),
              synth.scales_f16(4, (E * H, I // bs)))
    return p1, p2, keep


def test_noalloc_size_limit_checked_on_the_host():
    """A request whose workspace exceeds the static array is refused before
    any device call (host plans suffice); T = 0 is a no-op."""
    E, H, I, bs, k = 2, 16384, 64, 64, 2
    p1, p2, _keep = _host_plans(E, H, I, bs)
    q = mnb.make_qmoe_desc(k)
    lib = mnb.lib()
    need = mnb.qmoe_workspace_size(p1, p2, q, 4096)
    assert need > mnb.MNB_NOALLOC_SCRATCH_BYTES
    rc = lib.qmoe_forward_noalloc(ctypes.byref(p1), ctypes.byref(p2), ctypes.byref(q), 4096, 16, 16,
                                  16, None)
    assert rc == WS_TOO_SMALL
    assert lib.qmoe_forward_noalloc(ctypes.byref(p1), ctypes.byref(p2), ctypes.byref(q), 0, None,
                                    None, None, None) == 0


def _layer(seed, E, H, I, bs, bits1=3, bits2=3):
    W1 = synth.packed_rows(synth.seed_for(seed, 3), E * 2 * I, H, bits1)
    s1 = synth.scales_f16(synth.seed_for(seed, 4), (E * 2 * I, H // bs))
    W2 = synth.packed_rows(synth.seed_for(seed, 5), E * H, I, bits2)
    s2 = synth.scales_f16(synth.seed_for(seed, 6), (E * H, I // bs))
    p1 = mnb.PreparedWeight(mnb.qmoe_proj_desc(H, 2 * I, E, bs, bits1), W1, s1)
    p2 = mnb.PreparedWeight(mnb.qmoe_proj_desc(I, H, E, bs, bits2), W2, s2)
    return p1, p2


@pytest.mark.gpu
@pytest.mark.parametrize("E,H,I,k,T0,T1", [(128, 2048, 768, 8, 512, 1), (16, 512, 192, 4, 300, 7)])
def test_noalloc_matches_qmoe_forward(E, H, I, k, T0, T1):
    torch = pytest.importorskip("torch")
    say(f"qmoe noalloc E={E} H={H} I={I} k={k} T={T0} then T={T1}")
    bs = 64
    p1, p2 = _layer(E + H, E, H, I, bs)
    q = mnb.make_qmoe_desc(k)
    assert mnb.qmoe_workspace_size(p1.plan, p2.plan, q, max(T0, T1)) <= mnb.MNB_NOALLOC_SCRATCH_BYTES
    for T in (T0, T1):
        x = torch.from_numpy(synth.activations_f16(synth.seed_for(T, 1), T, H)).cuda()
        lg = torch.from_numpy(synth.router_logits(synth.seed_for(T, 2), T, E)).cuda()
        need = mnb.qmoe_workspace_size(p1.plan, p2.plan, q, T)
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        ref = torch.empty((T, H), dtype=torch.float16, device="cuda")
        mnb.qmoe_forward(p1.plan, p2.plan, q, T, x, lg, ref, ws, ws.numel())
        guard = 64
        og = torch.full((T * H + 2 * guard,), float("nan"), dtype=torch.float16, device="cuda")
        out = og[guard:guard + T * H]
        mnb.qmoe_forward_noalloc(p1.plan, p2.plan, q, T, x, lg, out)
        torch.cuda.synchronize()
        g = og.cpu().numpy()
        assert np.isnan(g[:guard]).all() and np.isnan(g[guard + T * H:]).all()
        assert np.array_equal(g[guard:guard + T * H].view(np.uint16),
                              ref.cpu().numpy().reshape(-1).view(np.uint16)), f"T={T}"
