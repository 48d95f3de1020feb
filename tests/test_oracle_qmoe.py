"""Pins of the oracle's routing and INT3 QMoE layer (CPU only).

Sources: onnxruntime PR "INT3 QMoE CUDA correctness baseline and Qwen
experimental results" (embedded P0/P1 body: sections "P0" for the format and
the tiny predetermined-route SwiGLU MoE, "P1" for fused interleaved gate/up
and swiglu; embedded Olive body for the (code - 4) * scale decode) and the
pegainfer PR "component kernels extracted from the brick PRs" (fp32 softmax,
top-k, renormalized routing weights).
"""
import numpy as np
import pytest

import synth
from tests.golden import fixtures
from tests.np_brute import qmoe_all_experts, softmax


def _const_rows(code, rows, K):
    """Rows of K identical INT3 codes, built from the hand-derived byte
    vectors (64 x code c) of int3_byte_vectors.txt."""
    vecs = {tuple(c): b for c, b in fixtures.byte_vectors("int3_byte_vectors.txt")}
    row = np.frombuffer(vecs[tuple([code] * 64)], np.uint8)
    assert K % 64 == 0
    return np.tile(row, (rows, K // 64))


def test_worked_tiny_moe(orc):
    f = fixtures.tiny_moe()
    H = I = 64
    E, k, bs = 4, 2, 64
    fc1 = [int(c) for c in f["fc1_codes"].split(",")]
    fc2 = [int(c) for c in f["fc2_codes"].split(",")]
    W1 = np.stack([_const_rows(fc1[e], 2 * I, H) for e in range(E)])
    W2 = np.stack([_const_rows(fc2[e], H, I) for e in range(E)])
    s = np.float16(float(f["scale"]))
    s1 = np.full((E, 2 * I, H // bs), s, np.float16)
    s2 = np.full((E, H, I // bs), s, np.float16)
    x = np.ones((2, H), np.float16)
    logits = np.array([[float(v) for v in f["logits_t0"].split(",")],
                       [float(v) for v in f["logits_t1"].split(",")]], np.float32)
    o = orc.qmoe(x, logits, W1, s1, W2, s2, k=k, bs=bs)
    assert o["ids"][0].tolist() == [int(v) for v in f["ids_t0"].split(",")]
    assert o["ids"][1].tolist() == [int(v) for v in f["ids_t1"].split(",")]
    np.testing.assert_allclose(o["r"][0], [float(v) for v in f["r_t0"].split(",")], rtol=0, atol=1e-7)
    np.testing.assert_allclose(o["out64"][0], float(f["out_t0"]), rtol=0, atol=1e-7)
    assert (o["out16"][0] == int(f["out16_t0"], 16)).all()
    assert (o["out64"][1] == 0.0).all() and (o["out16"][1] == 0).all()
    # stage values: expert 0 has g = u = 1, expert 1 has g = u = -1
    np.testing.assert_allclose(o["g"][0, 0], 1.0, atol=1e-12)
    np.testing.assert_allclose(o["u"][0, 1], -1.0, atol=1e-12)
    np.testing.assert_allclose(o["h"][0, 1], 1.0 / (1.0 + np.e), atol=1e-12)


def test_route_against_numpy_and_full_softmax(orc):
    T, E = 64, 16
    logits = synth.router_logits(5, T, E)
    for k in (1, 2, 8, E):
        ids, w = orc.route(logits, k)
        ref = np.argsort(-logits, axis=1, kind="stable")[:, :k]
        assert np.array_equal(ids, ref)
        p = softmax(logits)
        sel = np.take_along_axis(p, ref, axis=1)
        np.testing.assert_allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13)
        if k == E:
            # with k = E the renormalized weights are the full softmax
            np.testing.assert_allclose(np.take_along_axis(p, ids, axis=1), w, rtol=1e-13)
        assert np.all(np.diff(w, axis=1) <= 0)


def test_route_ties_go_to_lower_index(orc):
    logits = np.array([[0.5, 1.0, 1.0, 0.25, 1.0, -2.0]], np.float32)
    ids, w = orc.route(logits, 3)
    assert ids[0].tolist() == [1, 2, 4]
    np.testing.assert_allclose(w[0], [1 / 3] * 3, rtol=1e-15)


def _random_moe(seed, T, H, I, E, bs):
    x = synth.activations_f16(seed, T, H)
    logits = synth.router_logits(seed + 1, T, E)
    W1 = synth.int3_rows(seed + 2, E * 2 * I, H).reshape(E, 2 * I, -1)
    s1 = synth.scales_f16(seed + 3, (E, 2 * I, H // bs))
    W2 = synth.int3_rows(seed + 4, E * H, I).reshape(E, H, -1)
    s2 = synth.scales_f16(seed + 5, (E, H, I // bs))
    return x, logits, W1, s1, W2, s2


@pytest.mark.parametrize("T,H,I,E,k,bs", [(5, 64, 64, 4, 2, 64), (3, 128, 64, 8, 3, 32),
                                          (8, 64, 128, 6, 6, 64), (1, 128, 128, 5, 1, 128)])
def test_qmoe_brute_force_over_all_experts(orc, T, H, I, E, k, bs):
    x, logits, W1, s1, W2, s2 = _random_moe(T * 100 + E, T, H, I, E, bs)
    o = orc.qmoe(x, logits, W1, s1, W2, s2, k=k, bs=bs)
    ref, order, rw = qmoe_all_experts(x, logits, W1, s1, W2, s2, k, bs)
    assert np.array_equal(o["ids"], order)
    np.testing.assert_allclose(o["r"], rw, rtol=1e-12)
    scale = np.abs(ref).max() + 1e-300
    np.testing.assert_allclose(o["out64"], ref, rtol=1e-10, atol=1e-12 * scale)
    assert np.array_equal(o["out16"], orc.f64_to_f16(o["out64"]))
    # the combine is the route-weighted sum of per-expert FC2 outputs
    y, yS = orc.qmoe_fc2(o["ids"], o["h"], W2, s2, H, I, E, bs=bs)
    np.testing.assert_allclose((o["r"][:, :, None] * y).sum(axis=1), o["out64"], rtol=1e-12,
                               atol=1e-14 * scale)


def test_qmoe_invariants(orc):
    T, H, I, E, k, bs = 6, 64, 64, 8, 3, 64
    x, logits, W1, s1, W2, s2 = _random_moe(901, T, H, I, E, bs)
    base = orc.qmoe(x, logits, W1, s1, W2, s2, k=k, bs=bs)
    # permuting tokens permutes the outputs
    perm = np.array([3, 0, 5, 1, 4, 2])
    o = orc.qmoe(x[perm], logits[perm], W1, s1, W2, s2, k=k, bs=bs)
    assert np.array_equal(o["out64"], base["out64"][perm])
    # relabelling experts together with the logit columns changes nothing
    rel = np.array([2, 7, 0, 1, 6, 3, 5, 4])
    o = orc.qmoe(x, logits[:, rel], W1[rel], s1[rel], W2[rel], s2[rel], k=k, bs=bs)
    assert np.array_equal(o["out64"], base["out64"])
    # T tokens at once equal T single-token calls
    for t in range(T):
        o = orc.qmoe(x[t:t + 1], logits[t:t + 1], W1, s1, W2, s2, k=k, bs=bs)
        assert np.array_equal(o["out64"][0], base["out64"][t])
    # all codes equal to the zero point 4 give exactly zero
    z1 = _const_rows(4, E * 2 * I, H).reshape(E, 2 * I, -1)
    z2 = _const_rows(4, E * H, I).reshape(E, H, -1)
    o = orc.qmoe(x, logits, z1, s1, z2, s2, k=k, bs=bs)
    assert (o["out64"] == 0).all() and (o["S"] == 0).all()


def test_qmoe_tolerance_sum_covers_fp16_rounding_chain(orc):
    """An fp16/fp32 emulation of the GPU rounding chain (weights and h in fp16,
    fp32 accumulation) must land inside 4e-3 * S + half an fp16 ulp."""
    T, H, I, E, k, bs = 4, 128, 64, 4, 2, 64
    x, logits, W1, s1, W2, s2 = _random_moe(555, T, H, I, E, bs)
    o = orc.qmoe(x, logits, W1, s1, W2, s2, k=k, bs=bs)
    from tests.np_brute import int3_weights
    w1 = int3_weights(W1, s1, H, bs).astype(np.float16).astype(np.float32)
    w2 = int3_weights(W2, s2, I, bs).astype(np.float16).astype(np.float32)
    out = np.zeros((T, H), np.float32)
    for t in range(T):
        for j in range(k):
            e = o["ids"][t, j]
            G = x[t].astype(np.float32) @ w1[e, 0::2].T
            U = x[t].astype(np.float32) @ w1[e, 1::2].T
            h = (G / (1 + np.exp(-G)) * U).astype(np.float16).astype(np.float32)
            out[t] += np.float32(o["r"][t, j]) * (h @ w2[e].T)
    out16 = out.astype(np.float16).astype(np.float64)
    ulp = np.spacing(np.abs(o["out"]).astype(np.float16)).astype(np.float64)
    err = np.abs(out16 - o["out64"])
    assert (err <= 4e-3 * o["S"] + 0.5 * ulp + ulp).all()
    assert (o["S"] > 0).all()


# ---------------------------------------------------------------------------
# INT4 and mixed-width projections.  The P1 section of the INT3 QMoE page lets
# each projection carry its own width, (FC1, FC2) in {(3,3), (3,4), (4,3)};
# the same page's results table runs the all-INT4 (4,4) layer next to (3,3).
# A 4-bit row-local LSB-first row puts even positions in the low nibble, and
# the implicit zero point is 2^(bits - 1) = 8.
# ---------------------------------------------------------------------------

def _random_moe_bits(seed, T, H, I, E, bs, bits1, bits2):
    x = synth.activations_f16(seed, T, H)
    logits = synth.router_logits(seed + 1, T, E)
    W1 = synth.packed_rows(seed + 2, E * 2 * I, H, bits1).reshape(E, 2 * I, -1)
    s1 = synth.scales_f16(seed + 3, (E, 2 * I, H // bs))
    W2 = synth.packed_rows(seed + 4, E * H, I, bits2).reshape(E, H, -1)
    s2 = synth.scales_f16(seed + 5, (E, H, I // bs))
    return x, logits, W1, s1, W2, s2


@pytest.mark.parametrize("bits1,bits2,T,H,I,E,k,bs", [(4, 4, 5, 64, 64, 4, 2, 64),
                                                      (4, 4, 3, 128, 64, 8, 3, 32),
                                                      (3, 4, 4, 64, 128, 6, 2, 64),
                                                      (4, 3, 2, 128, 128, 5, 1, 128)])
def test_qmoe_mixed_width_brute_force(orc, bits1, bits2, T, H, I, E, k, bs):
    x, logits, W1, s1, W2, s2 = _random_moe_bits(T * 31 + E, T, H, I, E, bs, bits1, bits2)
    o = orc.qmoe(x, logits, W1, s1, W2, s2, k=k, bits1=bits1, bits2=bits2, bs=bs)
    ref, order, rw = qmoe_all_experts(x, logits, W1, s1, W2, s2, k, bs, bits1, bits2)
    assert np.array_equal(o["ids"], order)
    scale = np.abs(ref).max() + 1e-300
    np.testing.assert_allclose(o["out64"], ref, rtol=1e-10, atol=1e-12 * scale)
    if bits2 == 4:
        # reading the 4-bit FC2 rows as 3-bit streams changes the result
        wrong = qmoe_all_experts(x, logits, W1, s1, W2, s2, k, bs, bits1, 3)[0]
        assert np.abs(wrong - ref).max() > 1e-3 * scale


def test_qmoe_int4_rows_are_low_nibble_first_dense_blocks(orc):
    """A 4-bit row-local row with block-aligned K is byte for byte a dense
    MatMulNBits row [nb, bs/2] (low nibble = even position, zero point 8), so
    the stage values of one expert must equal products with the dense nibble
    decode of the same bytes."""
    from tests.np_brute import dense_weights
    T, H, I, E, k, bs = 3, 128, 64, 1, 1, 32
    x, logits, W1, s1, W2, s2 = _random_moe_bits(77, T, H, I, E, bs, 4, 4)
    o = orc.qmoe(x, logits, W1, s1, W2, s2, k=k, bits1=4, bits2=4, bs=bs)
    w1 = dense_weights(W1[0].reshape(2 * I, H // bs, bs // 2), s1[0].astype(np.float32), None, H, bs)
    w2 = dense_weights(W2[0].reshape(H, I // bs, bs // 2), s2[0].astype(np.float32), None, I, bs)
    xx = x.astype(np.float64)
    G, U = xx @ w1[0::2].T, xx @ w1[1::2].T
    np.testing.assert_allclose(o["g"][:, 0], G, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o["u"][:, 0], U, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(o["r"], np.ones((T, 1)))
    Y = (G / (1 + np.exp(-G)) * U) @ w2.T
    np.testing.assert_allclose(o["out64"], Y, rtol=1e-11, atol=1e-12 * np.abs(Y).max())


def test_qmoe_int4_codes_at_zero_point_give_zero(orc):
    T, H, I, E, k, bs = 4, 64, 64, 4, 2, 64
    x, logits, W1, s1, W2, s2 = _random_moe_bits(313, T, H, I, E, bs, 4, 4)
    z1 = np.full_like(W1, 0x88)
    z2 = np.full_like(W2, 0x88)
    o = orc.qmoe(x, logits, z1, s1, z2, s2, k=k, bits1=4, bits2=4, bs=bs)
    assert (o["out64"] == 0).all() and (o["S"] == 0).all() and (o["g"] == 0).all()
    # codes 8 + 1 in FC1 and the x = 1 row: g = u = sum of the scales
    o = orc.qmoe(np.ones((1, H), np.float16), logits[:1], np.full_like(W1, 0x99), s1,
                 W2, s2, k=k, bits1=4, bits2=4, bs=bs)
    for j in range(k):
        e = o["ids"][0, j]
        np.testing.assert_allclose(o["g"][0, j], s1[e, 0::2].astype(np.float64).sum(axis=1) * bs,
                                   rtol=1e-14)


# ---------------------------------------------------------------------------
# Optional biases (P1 section of the INT3 QMoE page: optional biases).  FC1's
# bias is added to the gate and up rows before SwiGLU, FC2's to each expert's
# output before its routing weight.
# ---------------------------------------------------------------------------

def _biases(seed, E, I, H):
    b1 = synth.activations_f16(seed, E, 2 * I) * np.float16(0.5)
    b2 = synth.activations_f16(seed + 1, E, H) * np.float16(0.25)
    return b1, b2


@pytest.mark.parametrize("bits1,bits2", [(3, 3), (4, 4), (3, 4)])
def test_qmoe_biases_brute_force(orc, bits1, bits2):
    T, H, I, E, k, bs = 5, 64, 64, 6, 2, 32
    x, logits, W1, s1, W2, s2 = _random_moe_bits(71 + bits1, T, H, I, E, bs, bits1, bits2)
    b1, b2 = _biases(5, E, I, H)
    o = orc.qmoe(x, logits, W1, s1, W2, s2, k=k, bits1=bits1, bits2=bits2, bs=bs, b1=b1, b2=b2)
    ref, _, _ = qmoe_all_experts(x, logits, W1, s1, W2, s2, k, bs, bits1, bits2, b1, b2)
    np.testing.assert_allclose(o["out64"], ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())
    plain = orc.qmoe(x, logits, W1, s1, W2, s2, k=k, bits1=bits1, bits2=bits2, bs=bs)
    assert np.abs(plain["out64"] - o["out64"]).max() > 1e-2  # the biases matter
    # the tolerance sums grow by exactly the bias magnitudes (one more term each)
    ids = o["ids"]
    np.testing.assert_allclose(o["gs"] - plain["gs"],
                               np.abs(b1[ids][:, :, 0::2].astype(np.float64)), rtol=1e-12, atol=1e-15)


def test_qmoe_biases_closed_forms(orc):
    """With every code at the zero point the weights vanish: g and u are the
    FC1 biases, and the layer output is sum_j r_j b2[e_j]."""
    T, H, I, E, k, bs = 3, 64, 32, 4, 2, 32
    x, logits, W1, s1, W2, s2 = _random_moe_bits(91, T, H, I, E, bs, 4, 4)
    b1, b2 = _biases(9, E, I, H)
    z1, z2 = np.full_like(W1, 0x88), np.full_like(W2, 0x88)
    o = orc.qmoe(x, logits, z1, s1, z2, s2, k=k, bits1=4, bits2=4, bs=bs, b1=b1, b2=b2)
    ids = o["ids"]
    np.testing.assert_array_equal(o["g"], b1[ids][:, :, 0::2].astype(np.float64))
    np.testing.assert_array_equal(o["u"], b1[ids][:, :, 1::2].astype(np.float64))
    want = (o["r"][:, :, None] * b2[ids].astype(np.float64)).sum(axis=1)
    np.testing.assert_allclose(o["out64"], want, rtol=1e-15, atol=1e-18)
    # FC1 weights at the zero point, FC2 real: h = silu(b_g) b_u enters FC2
    o = orc.qmoe(x, logits, z1, s1, W2, s2, k=k, bits1=4, bits2=4, bs=bs, b1=b1, b2=b2)
    g, u = o["g"], o["u"]
    np.testing.assert_allclose(o["h"], g / (1 + np.exp(-g)) * u, rtol=1e-14)
    y, _ = orc.qmoe_fc2(ids, o["h"], W2, s2, H, I, E, bits2=4, bs=bs, b2=b2)
    np.testing.assert_allclose((o["r"][:, :, None] * y).sum(axis=1), o["out64"], rtol=1e-12,
                               atol=1e-15)


# ---------------------------------------------------------------------------
# bfloat16 layers (P1 section of the INT3 QMoE page: FP16 or BF16, with the
# activation and scale types matching).  Inputs are bfloat16 patterns; the
# brute force widens them with torch's bfloat16 (independent of the oracle).
# ---------------------------------------------------------------------------

def _bf16_f64(bits):
    torch = pytest.importorskip("torch")
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(
        torch.float64).numpy()


@pytest.mark.parametrize("bits1,bits2,bs", [(3, 3, 64), (4, 4, 32), (4, 3, 128)])
def test_qmoe_bf16_brute_force(orc, bits1, bits2, bs):
    T, H, I, E, k = 4, 128, 128, 5, 2
    x = synth.activations_bf16(31, T, H)
    logits = synth.router_logits(32, T, E)
    W1 = synth.packed_rows(33, E * 2 * I, H, bits1).reshape(E, 2 * I, -1)
    s1 = synth.scales_bf16(34, (E, 2 * I, H // bs))
    W2 = synth.packed_rows(35, E * H, I, bits2).reshape(E, H, -1)
    s2 = synth.scales_bf16(36, (E, H, I // bs))
    b1 = synth.activations_bf16(37, E, 2 * I)
    b2 = synth.activations_bf16(38, E, H)
    o = orc.qmoe(x, logits, W1, s1, W2, s2, k=k, bits1=bits1, bits2=bits2, bs=bs, b1=b1, b2=b2,
                 dtype="bf16")
    ref, order, _ = qmoe_all_experts(_bf16_f64(x), logits, W1, _bf16_f64(s1), W2, _bf16_f64(s2),
                                     k, bs, bits1, bits2, _bf16_f64(b1), _bf16_f64(b2))
    assert np.array_equal(o["ids"], order)
    np.testing.assert_allclose(o["out64"], ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())
    # out is the bfloat16 rounding of out64: within half a bf16 step, and the
    # widened pattern matches torch's reading of it
    np.testing.assert_array_equal(o["out"], _bf16_f64(o["out16"]))
    assert (np.abs(o["out"] - o["out64"]) <= np.abs(o["out64"]) * 2.0 ** -8 + 1e-38).all()
    # the same bytes read as fp16 give a different layer (the dtype is honoured)
    o16 = orc.qmoe(x.view(np.float16), logits, W1, s1.view(np.float16), W2, s2.view(np.float16),
                   k=k, bits1=bits1, bits2=bits2, bs=bs)
    assert not np.allclose(o16["out64"], o["out64"])
    # FC2 alone with the bf16 dtype reproduces the combine
    y, _ = orc.qmoe_fc2(o["ids"], o["h"], W2, s2, H, I, E, bits2=bits2, bs=bs, b2=b2, dtype="bf16")
    np.testing.assert_allclose((o["r"][:, :, None] * y).sum(axis=1), o["out64"], rtol=1e-12,
                               atol=1e-14 * np.abs(ref).max())


# ---------------------------------------------------------------------------
# The tolerance sums.  Every QMoE bound on the GPU is 4e-3 times a sum the
# oracle returns (gs, us for FC1; yS for FC2 fed the GPU's h; S for the layer),
# so each sum is pinned here to an independent whole-tensor numpy form: every
# expert evaluated, a masked routing-weight matrix, |x| @ |w|^T products and
# the SwiGLU derivative by complex-step differentiation (INT3 QMoE page, P0
# section: independent scalar references; the first-order propagation of a
# per-product bound through h = silu(g) * u).
# ---------------------------------------------------------------------------

def _bf16_moe(seed, T, H, I, E, bs, bits1, bits2):
    x = synth.activations_bf16(seed, T, H)
    logits = synth.router_logits(seed + 1, T, E)
    W1 = synth.packed_rows(seed + 2, E * 2 * I, H, bits1).reshape(E, 2 * I, -1)
    s1 = synth.scales_bf16(seed + 3, (E, 2 * I, H // bs))
    W2 = synth.packed_rows(seed + 4, E * H, I, bits2).reshape(E, H, -1)
    s2 = synth.scales_bf16(seed + 5, (E, H, I // bs))
    return x, logits, W1, s1, W2, s2


@pytest.mark.parametrize("bits1,bits2", [(3, 3), (4, 4), (3, 4), (4, 3)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("biased", [False, True])
def test_qmoe_tolerance_sums_independent(orc, bits1, bits2, dtype, biased):
    from tests.np_brute import fc2_tolerance_sum, qmoe_tolerance_sums
    T, H, I, E, k, bs = 5, 128, 64, 6, 3, 32
    seed = 400 + 10 * bits1 + bits2
    if dtype == "bf16":
        x, logits, W1, s1, W2, s2 = _bf16_moe(seed, T, H, I, E, bs, bits1, bits2)
        b1 = synth.activations_bf16(seed + 7, E, 2 * I) if biased else None
        b2 = synth.activations_bf16(seed + 8, E, H) if biased else None
        wid = _bf16_f64
    else:
        x, logits, W1, s1, W2, s2 = _random_moe_bits(seed, T, H, I, E, bs, bits1, bits2)
        b1, b2 = _biases(seed + 7, E, I, H) if biased else (None, None)
        wid = lambda a: a.astype(np.float64)  # noqa: E731
    o = orc.qmoe(x, logits, W1, s1, W2, s2, k=k, bits1=bits1, bits2=bits2, bs=bs, b1=b1, b2=b2,
                 dtype=dtype)
    nb = lambda a: None if a is None else wid(a)  # noqa: E731
    gs, us, S = qmoe_tolerance_sums(wid(x), logits, W1, wid(s1), W2, wid(s2), k, bs, bits1, bits2,
                                    nb(b1), nb(b2))
    ids = o["ids"].astype(np.int64)
    np.testing.assert_allclose(o["gs"], np.take_along_axis(gs, ids[:, :, None], axis=1), rtol=1e-12)
    np.testing.assert_allclose(o["us"], np.take_along_axis(us, ids[:, :, None], axis=1), rtol=1e-12)
    np.testing.assert_allclose(o["S"], S, rtol=1e-12)
    # FC2 fed an arbitrary h (here the oracle's, with signs flipped on half of
    # it: the sum takes magnitudes) and the expert ids of the routing
    h = o["h"] * np.where(np.arange(I) % 2, -1.0, 1.0)
    _, yS = orc.qmoe_fc2(o["ids"], h, W2, s2, H, I, E, bits2=bits2, bs=bs, b2=b2, dtype=dtype)
    np.testing.assert_allclose(yS, fc2_tolerance_sum(o["ids"], h, W2, wid(s2), I, bs, bits2, nb(b2)),
                               rtol=1e-12)


def test_silu_derivative_complex_step_matches_finite_differences():
    """The complex-step derivative used above, against a central difference
    (error O(step^2)) at points spanning both signs and the minimum of silu."""
    from tests.np_brute import silu_derivative
    g = np.array([-8.0, -3.0, -1.2784645, -0.5, 0.0, 0.25, 1.0, 4.0, 12.0])
    d = 1e-5
    silu = lambda v: v / (1.0 + np.exp(-v))  # noqa: E731
    fd = (silu(g + d) - silu(g - d)) / (2 * d)
    np.testing.assert_allclose(silu_derivative(g), fd, rtol=0, atol=1e-9)
    assert abs(silu_derivative(np.array([0.0]))[0] - 0.5) < 1e-15
