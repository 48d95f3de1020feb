"""The library's compute calls enqueue only kernels on the caller's stream (no
host synchronisation, no memset nodes), so they can be captured in a HIP graph.
Each test replays a captured graph several times, with eager work and
synchronisations in between, and checks every replay bit for bit against the
eager result."""
import sys

import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import block_quantized_weight_03_amd as mnb  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def replay_and_check(g, out, ref, eager):
    for _ in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        eager()  # unrelated eager work between replays
        torch.cuda.synchronize()


def test_graph_gemv_and_gemm():
    say("graph gemv + gemm")
    K, N, M = 2050, 700, 37
    nb = -(-K // 32)
    w = mnb.PreparedWeight(mnb.dense_desc(K, N, 32, True), synth.int4_blocked_weights(1, N, K, 32),
                           synth.scales_f32(2, (N, nb)), synth.int4_zero_points(3, N, nb))
    a1 = torch.from_numpy(synth.activations_f32(4, 1, K)[0]).cuda()
    aM = torch.from_numpy(synth.activations_f32(5, M, K)).cuda()
    y1 = torch.empty(N, device="cuda")
    yM = torch.empty((M, N), device="cuda")
    need = max(mnb.mnb_gemv_workspace_size(w.plan), mnb.mnb_gemm_workspace_size(w.plan, M), 256)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def run():
        mnb.mnb_gemv(w.plan, a1, y1, ws, need)
        mnb.mnb_gemm(w.plan, M, aM, yM, ws, need)

    run()
    torch.cuda.synchronize()
    ref1, refM = y1.clone(), yM.clone()
    g = capture(run)
    for _ in range(3):
        y1.fill_(float("nan"))
        yM.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y1, ref1) and torch.equal(yM, refM)
        (aM * 2).sum().item()
        torch.cuda.synchronize()


def test_graph_gemv_multi():
    say("graph gemv multi")
    K = 2048
    ws_ = [mnb.PreparedWeight(mnb.dense_desc(K, N), synth.int4_blocked_weights(10 + i, N, K, 32),
                              synth.scales_f32(20 + i, (N, K // 32))) for i, N in enumerate((700, 1300))]
    a = torch.from_numpy(synth.activations_f32(30, 1, K)[0]).cuda()
    ys = [torch.empty(w.desc.N, device="cuda") for w in ws_]
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")

    def run():
        mnb.mnb_gemv_multi([w.plan for w in ws_], a, ys, ws, 256)

    run()
    torch.cuda.synchronize()
    refs = [y.clone() for y in ys]
    g = capture(run)
    for _ in range(4):
        for y in ys:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(y, r) for y, r in zip(ys, refs))
        (a * 2).sum().item()
        torch.cuda.synchronize()


@pytest.mark.parametrize("T", [48, 2, 7])  # grouped path; decode with fused routing; decode
def test_graph_qmoe(T):
    say(f"graph qmoe T={T}")
    H, I, E, k, bs = 256, 128, 16, 4, 64
    W1 = synth.int3_rows(1, E * 2 * I, H)
    s1 = synth.scales_f16(2, (E * 2 * I, H // bs))
    W2 = synth.int3_rows(3, E * H, I)
    s2 = synth.scales_f16(4, (E * H, I // bs))
    p1 = mnb.PreparedWeight(mnb.qmoe_proj_desc(H, 2 * I, E, bs), W1, s1)
    p2 = mnb.PreparedWeight(mnb.qmoe_proj_desc(I, H, E, bs), W2, s2)
    q = mnb.make_qmoe_desc(k)
    x = torch.from_numpy(synth.activations_f16(5, T, H)).cuda()
    lg = torch.from_numpy(synth.router_logits(6, T, E)).cuda()
    out = torch.empty((T, H), dtype=torch.float16, device="cuda")
    ws = torch.empty(mnb.qmoe_workspace_size(p1.plan, p2.plan, q, T), dtype=torch.uint8, device="cuda")

    def run():
        mnb.qmoe_forward(p1.plan, p2.plan, q, T, x, lg, out, ws, ws.numel())

    run()
    torch.cuda.synchronize()
    ref = out.clone()
    g = capture(run)
    replay_and_check(g, out, ref, lambda: (x.float() * 3).sum().item())


@pytest.mark.parametrize("T,bits1,bits2,bf16", [(48, 4, 3, False), (2, 3, 4, True), (40, 4, 4, True),
                                                (7, 3, 3, False)])
def test_graph_qmoe_biased_widths_dtypes(T, bits1, bits2, bf16):
    """qmoe_forward_biased with mixed widths and fp16 or bf16 layers."""
    say(f"graph qmoe biased T={T} widths ({bits1},{bits2}) bf16={bf16}")
    H, I, E, k, bs = 256, 128, 16, 4, 64
    sd = mnb.MNB_DTYPE_BF16 if bf16 else mnb.MNB_DTYPE_F16
    scales = synth.scales_bf16 if bf16 else synth.scales_f16
    W1 = synth.packed_rows(1, E * 2 * I, H, bits1)
    W2 = synth.packed_rows(3, E * H, I, bits2)
    p1 = mnb.PreparedWeight(mnb.qmoe_proj_desc(H, 2 * I, E, bs, bits1, sd), W1,
                            scales(2, (E * 2 * I, H // bs)))
    p2 = mnb.PreparedWeight(mnb.qmoe_proj_desc(I, H, E, bs, bits2, sd), W2, scales(4, (E * H, I // bs)))
    q = mnb.make_qmoe_desc(k)

    def dev16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()

    if bf16:
        x = dev16(synth.activations_bf16(5, T, H))
        b1 = dev16(synth.activations_bf16(7, E, 2 * I))
        b2 = dev16(synth.activations_bf16(8, E, H))
    else:
        x = dev16(synth.activations_f16(5, T, H))
        b1 = dev16(synth.activations_f16(7, E, 2 * I))
        b2 = dev16(synth.activations_f16(8, E, H))
    lg = torch.from_numpy(synth.router_logits(6, T, E)).cuda()
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ws = torch.empty(mnb.qmoe_workspace_size(p1.plan, p2.plan, q, T), dtype=torch.uint8, device="cuda")

    def run():
        mnb.qmoe_forward_biased(p1.plan, p2.plan, q, T, x, lg, b1, b2, out, ws, ws.numel())

    run()
    torch.cuda.synchronize()
    ref = out.clone()
    g = capture(run)
    for _ in range(4):
        out.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        (lg * 3).sum().item()
        torch.cuda.synchronize()


@pytest.mark.parametrize("bf16", [False, True])
def test_graph_rtn_quantizer(bf16):
    say(f"graph rtn quantizer bf16={bf16}")
    rows, K, bs = 300, 256, 32
    W = torch.from_numpy((synth.normal(9, rows * K) * 0.1).astype(np.float32).reshape(rows, K)).cuda()
    B = torch.empty((rows, 3 * K // 8), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows, K // bs), dtype=torch.float16, device="cuda")
    st = torch.empty((rows, K // bs), dtype=torch.uint8, device="cuda")
    sd = mnb.MNB_DTYPE_BF16 if bf16 else mnb.MNB_DTYPE_F16

    def run():
        mnb.mnb_quantize_int3_rtn(W, rows, K, bs, B, s, st, None, sd)

    run()
    torch.cuda.synchronize()
    refs = (B.clone(), s.clone(), st.clone())
    g = capture(run)
    for _ in range(4):
        B.fill_(0x5A)
        s.fill_(7.0)
        st.fill_(9)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(B, refs[0]) and torch.equal(s, refs[1]) and torch.equal(st, refs[2])
        (W * 2).sum().item()
        torch.cuda.synchronize()


@pytest.mark.parametrize("M,N", [(4, 300), (16, 4096)])
def test_graph_single_launch_small_m_gemm(M, N):
    """The single-launch small-M GEMM (no workspace) replayed from a graph."""
    say(f"graph small-M gemm M={M} N={N}")
    K = 1024
    nb = K // 32
    w = mnb.PreparedWeight(mnb.dense_desc(K, N, 32, True), synth.int4_blocked_weights(7, N, K, 32),
                           synth.scales_f32(8, (N, nb)), synth.int4_zero_points(9, N, nb))
    a = torch.from_numpy(synth.activations_f32(10, M, K)).cuda()
    y = torch.empty((M, N), device="cuda")
    ws = torch.empty(max(mnb.mnb_gemm_workspace_size(w.plan, M), 256), dtype=torch.uint8,
                     device="cuda")

    def run():
        mnb.mnb_gemm(w.plan, M, a, y, ws, ws.numel())

    run()
    torch.cuda.synchronize()
    ref = y.clone()
    g = capture(run)
    replay_and_check(g, y, ref, lambda: (a * 3).sum().item())
