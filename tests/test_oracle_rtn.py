"""Pins of the oracle's INT3 round-to-nearest producer quantizer (CPU only).

Sources: onnxruntime PR "INT3 QMoE CUDA correctness baseline and Qwen
experimental results": embedded Olive body ("Summary": scale max|w| / 3.5,
zero point 4, all-zero group scale 1 / 3.5 with code 4, rejection of
non-finite weights and of scales that round to zero, subnormal stored scales
allowed) and embedded P0/P1 body, section "P0" (stored-scale rounding,
row-local LSB-first packing, golden-bytes regressions).
"""
import numpy as np
import pytest

import synth
from tests.golden import fixtures
from tests.np_brute import unpack_le


@pytest.mark.parametrize("case", fixtures.rtn_int3(), ids=lambda c: c[0])
def test_hand_derived_groups(orc, case):
    name, w, scale_bits, status, want = case
    B, s, st = orc.rtn_int3(np.array([w], np.float32), 32)
    assert B[0].tobytes() == want, name
    assert int(s.view(np.uint16)[0, 0]) == scale_bits, name
    assert int(st[0, 0]) == status, name


def test_groups_are_independent_and_rows_concatenate(orc):
    """A row of several groups equals its groups quantized one by one; group
    bytes are 3 bs / 8 and line up with the group boundaries."""
    cases = [c for c in fixtures.rtn_int3()]
    W = np.array([sum((c[1] for c in cases), [])], np.float32)
    B, s, st = orc.rtn_int3(W, 32)
    assert B[0].tobytes() == b"".join(c[4] for c in cases)
    assert s.view(np.uint16)[0].tolist() == [c[2] for c in cases]
    assert st[0].tolist() == [c[3] for c in cases]
    # the same weights as 64-wide groups pair the lines up
    B64, s64, st64 = orc.rtn_int3(W, 64)
    assert B64[0].tobytes() != b"" and st64.shape == (1, len(cases) // 2)


def _neighbours_f16(s16):
    b = s16.view(np.uint16).astype(np.int64)
    lo = np.maximum(b - 1, 0).astype(np.uint16).view(np.float16)
    hi = (b + 1).astype(np.uint16).view(np.float16)
    return lo.astype(np.float64), hi.astype(np.float64)


@pytest.mark.parametrize("bs", [32, 64, 128])
def test_random_weights_nearest_scale_and_nearest_code(orc, bs):
    """Properties that fix the result without its formula: the stored scale is
    the fp16 value nearest to amax / 3.5; every code is the nearest of the
    eight levels (q - 4) s to its weight (up to rounding-order ties); the
    decode error is at most half a step except at the clamped top level."""
    rows, K = 48, 4 * bs
    sigma = np.exp(synth.normal(7, rows * K // bs) * 3).reshape(rows, K // bs)  # spread of magnitudes
    W = (synth.normal(8, rows * K).reshape(rows, K // bs, bs) * sigma[:, :, None] * 0.01)
    W = W.astype(np.float32)
    W[3, 1] = 0.0  # an all-zero group
    B, s, st = orc.rtn_int3(W.reshape(rows, K), bs)
    assert (st == 0).all()
    q = np.stack([unpack_le(B[r], K, 3) for r in range(rows)]).reshape(rows, K // bs, bs)
    s64 = s.astype(np.float64)
    amax = np.abs(W.astype(np.float64)).max(axis=2)
    target = np.where(amax > 0, amax / 3.5, 1 / 3.5)
    lo, hi = _neighbours_f16(s)
    assert (np.abs(s64 - target) <= np.abs(lo - target) + 1e-300).all()
    assert (np.abs(s64 - target) <= np.abs(hi - target)).all()
    assert s.view(np.uint16)[3, 1] == 0x3492 and (q[3, 1] == 4).all()
    w = W.astype(np.float64)
    levels = (np.arange(8) - 4.0)[None, None, None, :] * s64[:, :, None, None]
    dist = np.abs(w[..., None] - levels)
    mine = np.take_along_axis(dist, q[..., None], axis=3)[..., 0]
    best = dist.min(axis=3)
    assert (mine <= best + 1e-6 * s64[:, :, None]).all()
    top = q == 7
    err = np.abs(w - (q - 4) * s64[:, :, None])
    assert (err[~top] <= 0.5 * s64[:, :, None].repeat(bs, 2)[~top] * (1 + 1e-6)).all()
    # the top level also covers the slice (3.5 s, amax]: with a normal fp16
    # scale amax <= 3.5 s (1 + 2^-11); subnormal scales round more coarsely
    normal = np.broadcast_to((s64 >= 2.0 ** -14)[:, :, None], err.shape)
    assert normal.any() and (~normal).any()
    assert (err[normal] <= (0.5 * 1.004 * np.broadcast_to(s64[:, :, None], err.shape))[normal]).all()
    assert q.min() == 0 or q.max() == 7  # the extreme weight of some group hits an end level


def test_status_groups_do_not_affect_their_neighbours(orc):
    W = np.array(synth.normal(3, 4 * 64), np.float32).reshape(1, 256)
    ref_B, ref_s, _ = orc.rtn_int3(W, 64)
    bad = W.copy()
    bad[0, 64 + 5] = np.nan
    B, s, st = orc.rtn_int3(bad, 64)
    assert st[0].tolist() == [0, 1, 0, 0]
    assert s.view(np.uint16)[0, 1] == 0
    for g in (0, 2, 3):
        assert B[0, 24 * g:24 * g + 24].tobytes() == ref_B[0, 24 * g:24 * g + 24].tobytes()
    assert B[0, 24:48].tobytes() == bytes.fromhex("244992" * 8)


def test_argument_errors(orc):
    with pytest.raises(ValueError):
        orc.rtn_int3(np.zeros((2, 48), np.float32), 32)  # K not a multiple of bs


# bfloat16 stored scales (P1 section of the INT3 QMoE page: FP16 or BF16
# scales; the Olive body's dtype-specific subnormal-scale regressions)
@pytest.mark.parametrize("case", fixtures.rtn_int3("rtn_int3_bf16.txt"), ids=lambda c: c[0])
def test_hand_derived_groups_bf16(orc, case):
    name, w, scale_bits, status, want = case
    B, s, st = orc.rtn_int3(np.array([w], np.float32), 32, "bf16")
    assert B[0].tobytes() == want, name
    assert int(s[0, 0]) == scale_bits, name
    assert int(st[0, 0]) == status, name


def test_bf16_scales_are_the_nearest_bfloat16(orc):
    """The stored bf16 scale is the bfloat16 value nearest amax / 3.5 (torch's
    bfloat16 rounding of the fp32 quotient, an independent implementation),
    and every code is the nearest of the eight levels of that scale."""
    torch = pytest.importorskip("torch")
    rows, K, bs = 40, 256, 64
    mag = np.exp(synth.normal(11, rows * K // bs) * 4).reshape(rows, K // bs)
    W = (synth.normal(12, rows * K).reshape(rows, K // bs, bs) * mag[:, :, None]).astype(np.float32)
    B, s, st = orc.rtn_int3(W.reshape(rows, K), bs, "bf16")
    assert (st == 0).all()
    amax = np.abs(W).max(axis=2)
    want = torch.from_numpy(amax / np.float32(3.5)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(s.view(np.int16), want)
    sd = torch.from_numpy(s.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    q = np.stack([unpack_le(B[r], K, 3) for r in range(rows)]).reshape(rows, K // bs, bs)
    w = W.astype(np.float64)
    levels = (np.arange(8) - 4.0)[None, None, None, :] * sd[:, :, None, None]
    dist = np.abs(w[..., None] - levels)
    mine = np.take_along_axis(dist, q[..., None], axis=3)[..., 0]
    assert (mine <= dist.min(axis=3) + 1e-6 * sd[:, :, None]).all()
