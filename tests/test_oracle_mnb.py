"""Pins of the oracle's MatMulNBits (CPU only).

Contract: "Qwen3 Missing-Kernel Implementation Plan", section "PR sequence",
steps K01 (FP32 A, UINT8 packed B, FP32 scales, bits=4, block_size=32,
implicit zero points, scale indexing, padding), K02 (M=1 GEMV, exact packing
and tail tests) and K03 (small-M/prefill on the same compressed weights,
partial blocks and output tails).
"""
import numpy as np
import pytest

import synth
from tests.golden import fixtures
from tests.np_brute import dense_gemm, dense_weights


def pack_int4_blocks(codes_2d: np.ndarray, bs: int) -> np.ndarray:
    """Test-side packer for hand-built cases: codes [N, nb*bs] -> [N, nb, bs/2]."""
    N, L = codes_2d.shape
    c = codes_2d.astype(np.uint8).reshape(N, L // bs, bs)
    return (c[:, :, 0::2] | (c[:, :, 1::2] << 4)).astype(np.uint8)


def test_closed_forms(orc):
    cf = fixtures.gemv_closed_forms()
    q = np.arange(32) % 16
    B = pack_int4_blocks(q[None, :], 32)
    s = np.array([[0.5]], np.float32)
    K, y = cf["one_block_ones"]
    Y, Y64, _ = orc.mnb_gemm(np.ones((1, K), np.float32), B, s, None, K, 1)
    assert Y64[0, 0] == y and Y[0, 0] == y
    K, y = cf["one_block_ramp"]
    Y, Y64, _ = orc.mnb_gemm(np.arange(K, dtype=np.float32)[None, :], B, s, None, K, 1)
    assert Y64[0, 0] == y


@pytest.mark.parametrize("pad_value", [0, 5, 15])
def test_k_tail_closed_form_ignores_pad_codes(orc, pad_value):
    K, y = fixtures.gemv_closed_forms()["k_tail"]
    codes = np.full((1, 64), pad_value, np.int64)
    codes[0, :32] = 8
    codes[0, 32:34] = [9, 10]
    B = pack_int4_blocks(codes, 32)
    s = np.array([[0.25, 0.5]], np.float32)
    Y, Y64, S = orc.mnb_gemm(np.ones((1, K), np.float32), B, s, None, K, 1)
    assert Y64[0, 0] == y
    assert S[0, 0] == 1.5


@pytest.mark.parametrize("M,N,K,bs,zp", [
    (1, 7, 32, 32, False), (3, 13, 64, 32, True), (2, 5, 96, 64, False),
    (4, 9, 128, 128, True), (1, 16, 34, 32, False), (5, 11, 50, 32, True),
    (2, 3, 130, 64, True), (64, 64, 64, 32, True), (1, 1, 1, 32, False)])
def test_brute_force_against_numpy(orc, M, N, K, bs, zp):
    seed = M * 1000 + N * 10 + K
    nb = -(-K // bs)
    A = synth.activations_f32(seed, M, K)
    B = synth.int4_blocked_weights(seed + 1, N, K, bs, pad="random")
    s = synth.scales_f32(seed + 2, (N, nb))
    Z = synth.int4_zero_points(seed + 3, N, nb) if zp else None
    Y, Y64, S = orc.mnb_gemm(A, B, s, Z, K, N, bs=bs)
    ref, refS = dense_gemm(A, B, s, Z, K, bs)
    np.testing.assert_allclose(Y64, ref, rtol=1e-12, atol=1e-12 * refS.max())
    np.testing.assert_allclose(S, refS, rtol=1e-12)
    assert np.array_equal(Y, Y64.astype(np.float32))
    W = orc.mnb_dequant(B, s, Z, K, N, bs=bs)
    assert np.array_equal(W, dense_weights(B, s, Z, K, bs))


def test_codes_and_zero_points_match_numpy_unpacking(orc):
    N, K, bs = 6, 200, 64
    nb = -(-K // bs)
    B = synth.int4_blocked_weights(5, N, K, bs)
    Z = synth.int4_zero_points(6, N, nb)
    codes, zeros = orc.mnb_codes(B, Z, K, N, bs=bs)
    from tests.np_brute import int4_codes, int4_zeros
    assert np.array_equal(codes, int4_codes(B, K))
    assert np.array_equal(zeros, int4_zeros(Z, N, nb))
    _, zeros8 = orc.mnb_codes(B, None, K, N, bs=bs)
    assert (zeros8 == 8).all()


def test_all_codes_equal_zero_point_gives_exact_zero(orc):
    N, K, bs = 9, 96, 32
    nb = K // bs
    A = synth.activations_f32(11, 3, K)
    s = synth.scales_f32(12, (N, nb))
    B = np.full((N, nb, bs // 2), 0x88, np.uint8)
    Y, Y64, S = orc.mnb_gemm(A, B, s, None, K, N)
    assert (Y64 == 0).all() and (S == 0).all()
    # explicit zero points: every code equals its block's zero point
    Z = synth.int4_zero_points(13, N, nb)
    zfull = np.empty((N, 2 * Z.shape[1]), np.uint8)
    zfull[:, 0::2] = Z & 15
    zfull[:, 1::2] = Z >> 4
    codes = np.repeat(zfull[:, :nb], bs, axis=1)
    B2 = pack_int4_blocks(codes, bs)
    Y, Y64, S = orc.mnb_gemm(A, B2, s, Z, K, N)
    assert (Y64 == 0).all() and (S == 0).all()


def test_power_of_two_scaling_is_exact(orc):
    N, K, bs = 8, 64, 32
    A = synth.activations_f32(21, 2, K)
    B = synth.int4_blocked_weights(22, N, K, bs)
    s = synth.scales_f32(23, (N, K // bs))
    _, y0, _ = orc.mnb_gemm(A, B, s, None, K, N)
    for p in (-7, 3):
        _, ya, _ = orc.mnb_gemm(A * np.float32(2.0 ** p), B, s, None, K, N)
        _, ys, _ = orc.mnb_gemm(A, B, s * np.float32(2.0 ** p), None, K, N)
        assert np.array_equal(ya, y0 * 2.0 ** p)
        assert np.array_equal(ys, y0 * 2.0 ** p)


def test_exact_integer_case_equals_integer_matmul(orc):
    M, N, K, bs = 4, 12, 96, 32
    A = synth.small_int_activations(31, M, K)
    B = synth.int4_blocked_weights(32, N, K, bs)
    s = np.ones((N, K // bs), np.float32)
    Y, Y64, _ = orc.mnb_gemm(A, B, s, None, K, N)
    from tests.np_brute import int4_codes
    ref = A.astype(np.int64) @ (int4_codes(B, K) - 8).T
    assert np.array_equal(Y64, ref.astype(np.float64))


def test_transposed_or_misindexed_weights_would_be_caught(orc):
    """Sanity of the pins themselves: a wrong nibble order or a wrong scale
    index changes the result that the brute-force pin compares against."""
    N, K, bs = 4, 64, 32
    A = synth.activations_f32(41, 1, K)
    B = synth.int4_blocked_weights(42, N, K, bs)
    s = synth.scales_f32(43, (N, K // bs))
    _, y, _ = orc.mnb_gemm(A, B, s, None, K, N)
    swapped = ((B >> 4) | (B << 4)).astype(np.uint8)
    _, y_sw, _ = orc.mnb_gemm(A, swapped, s, None, K, N)
    _, y_st, _ = orc.mnb_gemm(A, B, s[:, ::-1].copy(), None, K, N)
    assert not np.allclose(y, y_sw) and not np.allclose(y, y_st)
