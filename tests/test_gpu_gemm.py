"""GPU parity of the small-M / prefill GEMM against the fp64 oracle, through
the C ABI.

Operation: "Qwen3 Missing-Kernel Implementation Plan", section "PR sequence",
step K03 (small-M and prefill GEMM on the same compressed weights; partial
blocks and output tails).  Bar: |y - y_oracle| <= 4e-3 * sum_k |a_k w_k| per
element (fp16 matrix-core inputs, fp32 accumulation); exact cases bit-exact.
"""
import sys

import numpy as np
import pytest

import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import block_quantized_weight_03_amd as mnb  # noqa: E402

TOL = 4e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def prepare(K, N, bs=32, zp=False, seed=0):
    nb = -(-K // bs)
    B = synth.int4_blocked_weights(synth.seed_for(seed, 1), N, K, bs)
    s = synth.scales_f32(synth.seed_for(seed, 2), (N, nb))
    Z = synth.int4_zero_points(synth.seed_for(seed, 3), N, nb) if zp else None
    return mnb.PreparedWeight(mnb.dense_desc(K, N, bs, zp), B, s, Z), B, s, Z


def run_gemm(w, a_np, guard=256):
    M, N = a_np.shape[0], w.desc.N
    A = torch.from_numpy(np.ascontiguousarray(a_np)).cuda()
    Yg = torch.full((M * N + 2 * guard,), float("nan"), dtype=torch.float32, device="cuda")
    Y = Yg[guard:guard + M * N]
    need = mnb.mnb_gemm_workspace_size(w.plan, M)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    mnb.mnb_gemm(w.plan, M, A, Y, ws, ws.numel())
    torch.cuda.synchronize()
    g = Yg.cpu().numpy()
    assert np.isnan(g[:guard]).all() and np.isnan(g[guard + M * N:]).all(), "guard band written"
    return g[guard:guard + M * N].reshape(M, N).copy()


def check(orc, y, a, B, s, Z, K, N, bs):
    _, y64, S = orc.mnb_gemm(a, B, s, Z, K, N, bs=bs, nthreads=8)
    err = np.abs(y.astype(np.float64) - y64)
    ratio = err / np.maximum(S, 1e-300)
    assert (err <= TOL * S).all(), f"{(err > TOL * S).sum()} over 4e-3*S, worst {ratio.max():.3e}"
    return ratio.max()


@pytest.mark.parametrize("M,K,N,bs,zp", [
    (1, 32, 1, 32, False), (3, 34, 7, 32, False), (17, 100, 127, 32, True),
    (33, 2050, 300, 32, False), (64, 4096, 256, 128, True), (65, 64, 129, 64, False),
    (130, 6144, 129, 64, False), (257, 96, 513, 32, True), (5, 33, 1000, 32, True),
    (300, 2048, 260, 32, False), (2, 1, 3, 32, False),
    # M <= 32 with K % 32 == 0
    (1, 2048, 300, 32, False), (16, 2048, 1000, 64, True), (17, 4096, 129, 128, False),
    (32, 96, 33, 32, True), (5, 6144, 64, 32, False), (31, 160, 257, 32, True),
    # the register-staged kernels between the small-M and the LDS-streaming
    # ranges (M < 64, or M < 40 with K <= 2048, or K not a multiple of 64),
    # and the LDS-streaming kernel from M = 64 (from 40 with K <= 2048)
    (48, 4096, 300, 32, False), (39, 2048, 300, 32, True), (100, 2080, 500, 32, True),
    (64, 128, 1000, 64, True), (127, 192, 333, 32, False), (40, 2048, 333, 32, False),
    (57, 1024, 500, 64, True)])
def test_gemm_small_shapes_elementwise(orc, M, K, N, bs, zp):
    say(f"gemm small M={M} K={K} N={N} bs={bs} zp={zp}")
    w, B, s, Z = prepare(K, N, bs, zp, seed=M * 31 + K + N)
    a = synth.activations_f32(synth.seed_for(M + K, N % 255), M, K)
    y = run_gemm(w, a)
    check(orc, y, a, B, s, Z, K, N, bs)


@pytest.mark.parametrize("K,N", [(2048, 6144), (6144, 2048)])
@pytest.mark.parametrize("M", [16, 128, 512, 2048, 4096])
def test_gemm_prefill_configs_sampled_rows(orc, M, K, N):
    """The prefill configurations at full size; the oracle recomputes a sample
    of output rows (every column of each)."""
    say(f"gemm prefill M={M} K={K} N={N}")
    w, B, s, Z = prepare(K, N, seed=4 * 1000 + K % 997)
    a = synth.activations_f32(synth.seed_for(4, M % 251), M, K)
    y = run_gemm(w, a)
    assert np.isfinite(y).all()
    rng = np.random.default_rng(M)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(M, 14), replace=False)]))
    check(orc, y[rows], a[rows], B, s, Z, K, N, 32)


def test_gemm_exact_integer_case_bit_exact(orc):
    say("gemm exact integer")
    M, K, N = 70, 1024, 300
    _, B, _, _ = prepare(K, N, seed=21)
    s = np.full((N, K // 32), 0.25, np.float32)
    w = mnb.PreparedWeight(mnb.dense_desc(K, N), B, s, None)
    a = synth.small_int_activations(22, M, K)
    y = run_gemm(w, a)
    _, y64, _ = orc.mnb_gemm(a, B, s, None, K, N)
    assert np.array_equal(y.astype(np.float64), y64)


def test_gemm_all_codes_at_zero_point_give_zero():
    say("gemm zero invariant")
    M, K, N = 40, 256, 256
    nb = K // 32
    B = np.full((N, nb, 16), 0x88, np.uint8)
    s = synth.scales_f32(23, (N, nb))
    w = mnb.PreparedWeight(mnb.dense_desc(K, N), B, s, None)
    assert (run_gemm(w, synth.activations_f32(24, M, K)) == 0).all()


def test_gemm_deterministic():
    say("gemm determinism")
    M, K, N = 512, 2048, 1024
    w, *_ = prepare(K, N, seed=25)
    a = synth.activations_f32(26, M, K)
    y1, y2 = run_gemm(w, a), run_gemm(w, a)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("M,lo,hi", [(32, 3, 20), (100, 20, 90), (700, 100, 400)])
def test_gemm_rows_are_independent(M, lo, hi):
    """Row m of the output depends only on row m of A (no cross-row mixing in
    the tiling): a sub-batch that takes the same kernel (the register-staged
    one below 64 rows, here the 128 x 128 LDS-streaming one from 64, with K
    unsplit) gives the same bits.  Different kernels sum K in different
    orders."""
    say(f"gemm row independence M={M}")
    K, N = 512, 384
    w, *_ = prepare(K, N, seed=27)
    a = synth.activations_f32(28, M, K)
    y = run_gemm(w, a)
    y_sub = run_gemm(w, a[lo:hi])
    assert np.array_equal(y[lo:hi], y_sub)


# M >= 128 with K a multiple of 64 takes the LDS-streaming kernel (128 x 128
# tiles while there are at most 384 of them, else 256 x 256, or 256 x 128
# over the whole of K where too few 256 x 256 tiles would need split K):
# ragged M and N tails, one-stage K, every block size, zero points, split K,
# on every tile shape (the last four cases have more than 384 tiles of
# 128 x 128 and take the 256 x 128 tiles).
@pytest.mark.parametrize("M,K,N,bs,zp", [
    (1100, 320, 700, 64, True), (1025, 64, 33, 32, False), (1030, 384, 257, 128, True),
    (1300, 192, 1000, 32, False), (1040, 4096, 300, 128, True), (600, 320, 700, 64, True),
    (2048, 4096, 130, 128, False), (2100, 64, 3000, 32, True), (2600, 128, 2500, 64, False),
    (4100, 320, 1600, 128, True), (4000, 320, 1900, 64, True),
    # 256 x 256 tiles alone would need between one and two rounds: one launch of
    # 256 x 256 tiles up to a column split and 256 x 128 tiles beyond it, here
    # with zero points, a ragged last row block and (N = 4000) a partial last
    # narrow column tile
    (4100, 192, 4000, 64, True), (4500, 128, 4096, 32, True),
    # too few 256 x 256 tiles for one per CU while 256 x 128 ones alone would
    # need a second round: both widths in one round (36 wide, 216 narrow tiles)
    (1400, 192, 6100, 64, False), (1536, 128, 6144, 32, True),
    # 128 x 128 tiles would exceed one per CU (384) while 192 tiles of 256 x 128
    # cover the output in one round: those
    (1000, 192, 6100, 64, True),
    # 256 x 256 tiles just over one per CU (264): 128 x 128 tiles (1008, two
    # workgroups per CU) instead
    (2688, 128, 6100, 32, True)])
def test_gemm_large_m_ragged_elementwise(orc, M, K, N, bs, zp):
    say(f"gemm large-M M={M} K={K} N={N} bs={bs} zp={zp}")
    w, B, s, Z = prepare(K, N, bs, zp, seed=M * 7 + K + N)
    a = synth.activations_f32(synth.seed_for(M + K, N % 251), M, K)
    y = run_gemm(w, a)
    check(orc, y, a, B, s, Z, K, N, bs)


@pytest.mark.parametrize("M,K,N,zp", [(128, 6144, 2048, False), (512, 6144, 2048, True),
                                       (1024, 6144, 2048, False)])
def test_gemm_split_k_reuses_a_dirty_workspace(orc, M, K, N, zp):
    """Split K on the LDS-streaming kernel (12, 4 and 2 splits here): one
    workspace, filled with 0xFF before the first call, serves three calls;
    every call gives the same bits (nothing depends on what the workspace
    held), and sampled rows match the oracle."""
    say(f"gemm split-K dirty workspace M={M} K={K} N={N} zp={zp}")
    w, B, s, Z = prepare(K, N, 32, zp, seed=M + K + 3)
    a = synth.activations_f32(synth.seed_for(31, M), M, K)
    A = torch.from_numpy(a).cuda()
    need = mnb.mnb_gemm_workspace_size(w.plan, M)
    ws = torch.full((max(need, 256),), 0xFF, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(3):
        Y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        mnb.mnb_gemm(w.plan, M, A, Y, ws, ws.numel())
        torch.cuda.synchronize()
        outs.append(Y.cpu().numpy())
    assert np.isfinite(outs[0]).all()
    for y in outs[1:]:
        assert np.array_equal(y.view(np.uint32), outs[0].view(np.uint32))
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(M).choice(M, 6)]))
    check(orc, outs[0][rows], a[rows], B, s, Z, K, N, 32)


def test_gemm_large_m_rows_are_independent():
    say("gemm large-M row independence")
    M, K, N = 4500, 512, 4096  # 256 x 256 tiles for the batch and the sub-batch
    w, *_ = prepare(K, N, seed=29)
    a = synth.activations_f32(30, M, K)
    y = run_gemm(w, a)
    y_sub = run_gemm(w, a[100:2300])
    assert np.array_equal(y[100:2300], y_sub)


# The single-launch small-M kernel (M <= 4, or M <= 32 with N >= 4096; K a
# multiple of 128 up to 8192): one 16-row weight tile per workgroup, K chunks
# split over 4 or 8 waves (with waves that get no chunk when K is short),
# rows of N past the last whole tile, every block size, zero points, one
# 16-token tile up to M = 16 and two above (a partial second one at M = 17,
# 25); then the limits beside it (K = 8320, M = 17 with N = 70, M = 8 with
# N = 2048, M = 33) that take the other kernels.
@pytest.mark.parametrize("M,K,N,bs,zp", [
    (1, 128, 17, 32, True), (16, 8192, 4112, 128, True), (7, 384, 4100, 64, False),
    (16, 1024, 4144, 64, True), (5, 2048, 6160, 32, False), (9, 128, 8200, 128, True),
    (16, 2176, 4096, 32, True), (12, 6272, 4128, 64, False), (2, 256, 5, 128, True),
    (16, 2048, 6144, 32, False), (4, 6144, 2048, 64, True), (3, 8192, 33, 32, False),
    (16, 8320, 40, 32, False), (17, 2048, 70, 32, True), (8, 2048, 2048, 32, False),
    (17, 4096, 4112, 128, True), (20, 2048, 6144, 32, False), (25, 8192, 4096, 32, True),
    (32, 1024, 4144, 64, False), (32, 6272, 4128, 64, True), (33, 2048, 4096, 32, False)])
def test_gemm_single_launch_small_m(orc, M, K, N, bs, zp):
    say(f"gemm single-launch small M={M} K={K} N={N} bs={bs} zp={zp}")
    w, B, s, Z = prepare(K, N, bs, zp, seed=M * 7 + K + N)
    a = synth.activations_f32(synth.seed_for(M + K, 3), M, K)
    y = run_gemm(w, a)
    check(orc, y, a, B, s, Z, K, N, bs)
    assert np.array_equal(run_gemm(w, a).view(np.uint32), y.view(np.uint32))  # deterministic


def test_gemm_small_m_exact_integer_and_zero_cases(orc):
    say("gemm small-M exact cases")
    M, K, N = 9, 1024, 4096
    _, B, _, _ = prepare(K, N, seed=31)
    s = np.full((N, K // 32), 0.25, np.float32)
    w = mnb.PreparedWeight(mnb.dense_desc(K, N), B, s, None)
    a = synth.small_int_activations(32, M, K)
    _, y64, _ = orc.mnb_gemm(a, B, s, None, K, N)
    assert np.array_equal(run_gemm(w, a).astype(np.float64), y64)
    Bz = np.full((N, K // 32, 16), 0x88, np.uint8)
    wz = mnb.PreparedWeight(mnb.dense_desc(K, N), Bz, synth.scales_f32(33, (N, K // 32)), None)
    assert (run_gemm(wz, synth.activations_f32(34, M, K)) == 0).all()


@pytest.mark.parametrize("M,K,N", [(2, 256, 64), (20, 256, 96), (160, 256, 160)])
def test_gemm_fp16_input_range(orc, M, K, N):
    """The documented range of the fp16-input GEMM, on each kernel regime
    (single-launch small M, register-staged, LDS-streaming): an |A| past the
    fp16 range turns its output row non-finite while the other rows stay
    within the bound; |A| just inside it stays finite and within the bound;
    scales small enough that every weight is an fp16 subnormal add at most
    2^-25 |a| per product to the bound."""
    say(f"gemm fp16 range M={M} K={K} N={N}")
    bs = 32
    w, B, s, Z = prepare(K, N, bs, False, seed=M + 7)
    a = synth.activations_f32(synth.seed_for(M, 77), M, K)
    a[0, 5] = 1.0e5          # rounds to +Inf in fp16
    a[1, 9] = -65000.0       # finite in fp16 (max 65504)
    y = run_gemm(w, a)
    assert not np.isfinite(y[0]).any()
    check(orc, y[1:], a[1:], B, s, Z, K, N, bs)
    # subnormal weights: |(q - 8) s| <= 8 * 2^-20 = 2^-17 < 2^-14
    s_tiny = np.full_like(s, 2.0 ** -20)
    wt = mnb.PreparedWeight(mnb.dense_desc(K, N, bs, False), B, s_tiny, None)
    a2 = synth.activations_f32(synth.seed_for(M, 78), M, K)
    y2 = run_gemm(wt, a2)
    _, y64, S = orc.mnb_gemm(a2, B, s_tiny, None, K, N, bs=bs, nthreads=8)
    extra = 2.0 ** -25 * np.abs(a2.astype(np.float64)).sum(axis=1, keepdims=True) * 1.001
    err = np.abs(y2.astype(np.float64) - y64)
    assert np.isfinite(y2).all()
    assert (err <= TOL * S + extra).all()


@pytest.mark.parametrize("zp", [False, True])
def test_gemm_mixed_tile_widths_every_element(orc, zp):
    """Shapes whose 256 x 256 tiles would need between one and two rounds run
    256-wide tiles on the first columns and 256 x 128 tiles on the rest, in
    one launch; ragged M and N put partial tiles at the end of both widths."""
    M, K, N, bs = 2011, 256, 10163, 32
    say(f"gemm mixed tile widths M={M} K={K} N={N} zp={zp}")
    w, B, s, Z = prepare(K, N, bs, zp, seed=91 + zp)
    a = synth.activations_f32(synth.seed_for(M, 5), M, K)
    y = run_gemm(w, a)
    check(orc, y, a, B, s, Z, K, N, bs)
