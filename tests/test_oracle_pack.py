"""Pins of the oracle's bit packing and binary16 conversions (CPU only).

Packing rule: onnxruntime PR "INT3 QMoE CUDA correctness baseline and Qwen
experimental results", embedded P0/P1 body, section "P0: Portable Format and
Numerical References" (row-local LSB-first UINT8 packing, widths 1..8,
canonical padding).
"""
import numpy as np
import pytest

import synth
from tests.golden import fixtures
from tests.np_brute import unpack_le


@pytest.mark.parametrize("name,bits", [("int3_byte_vectors.txt", 3), ("int4_byte_vectors.txt", 4)])
def test_hand_derived_byte_vectors(orc, name, bits):
    vecs = fixtures.byte_vectors(name)
    assert len(vecs) >= 5
    for codes, expect in vecs:
        got = orc.pack_bits(np.array(codes), bits).tobytes()
        assert got == expect, (codes, got.hex(), expect.hex())
        back = orc.unpack_bits(np.frombuffer(expect, np.uint8), len(codes), bits)
        assert back.tolist() == codes
        assert orc.padding_is_canonical(np.frombuffer(expect, np.uint8), len(codes), bits)


@pytest.mark.parametrize("bits", range(1, 9))
def test_round_trips_all_widths(orc, bits):
    for n in list(range(1, 40)) + [63, 64, 65, 127, 128, 200, 257]:
        raw = synth.random_bytes(synth.seed_for(bits, n), n)
        codes = (raw & ((1 << bits) - 1)).astype(np.uint8)
        packed = orc.pack_bits(codes, bits)
        assert packed.size == (n * bits + 7) // 8
        assert orc.padding_is_canonical(packed, n, bits)
        assert np.array_equal(orc.unpack_bits(packed, n, bits), codes)
        # independent unpacking through numpy.unpackbits
        assert np.array_equal(unpack_le(packed, n, bits), codes.astype(np.int64))
        # pack(unpack(b)) == b for canonical b
        assert np.array_equal(orc.pack_bits(orc.unpack_bits(packed, n, bits), bits), packed)


def test_non_canonical_padding_detected(orc):
    # 11 codes at width 3 use 33 bits: byte 4 holds one valid bit.
    row = np.frombuffer(bytes.fromhex("88c6faff01"), np.uint8).copy()
    assert orc.padding_is_canonical(row, 11, 3)
    for bit in range(1, 8):
        bad = row.copy()
        bad[4] |= 1 << bit
        assert not orc.padding_is_canonical(bad, 11, 3)
        # the valid codes themselves are unchanged by pad bits
        assert np.array_equal(orc.unpack_bits(bad, 11, 3), orc.unpack_bits(row, 11, 3))
    # block-aligned rows have no pad bits at all
    assert orc.padding_is_canonical(np.full(24, 0xFF, np.uint8), 64, 3)


def test_pack_rejects_codes_wider_than_width(orc):
    with pytest.raises(ValueError):
        orc.pack_bits(np.array([8]), 3)
    with pytest.raises(ValueError):
        orc.pack_bits(np.array([16]), 4)


def test_f16_decode_matches_numpy_on_every_pattern(orc):
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_to_f64(pats)
    ref = pats.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_f16_encode_matches_numpy(orc):
    # random magnitudes over the whole binary16 range, plus every exact halfway
    # point between neighbouring binary16 values (ties to even)
    u = synth.uniform01(77, 200000)
    sgn = np.where(synth.uniform01(78, 200000) < 0.5, -1.0, 1.0)
    x = sgn * np.exp2(u * 44.0 - 28.0)
    fin = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (fin[:-1] + fin[1:]) / 2.0
    specials = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6, np.inf, -np.inf,
                         2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -14, 6.1e-5])
    for vals in (x, mids, -mids, specials):
        got = orc.f64_to_f16(vals)
        with np.errstate(over="ignore"):
            ref = vals.astype(np.float16).view(np.uint16)
        assert np.array_equal(got, ref)
    assert orc.f64_to_f16(np.array([np.nan]))[0] & 0x7C00 == 0x7C00


# ---------------------------------------------------------------------------
# bfloat16 conversions, against torch's CPU bfloat16 (an independent
# implementation): every pattern widens exactly; narrowing of binary32
# values rounds to nearest even, including exact halfway points, overflow
# and subnormals.
# ---------------------------------------------------------------------------

def test_bf16_widening_all_patterns(orc):
    torch = pytest.importorskip("torch")
    pats = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = orc.bf16_to_f64(pats)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_narrowing_round_to_nearest_even(orc):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    finite = np.arange(65536, dtype=np.uint16)
    finite = finite[(finite & 0x7F80) != 0x7F80]
    base = torch.from_numpy(finite.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    # halfway between neighbours (exact in binary32), quarter points, randoms
    nxt = torch.from_numpy((finite + 1).astype(np.uint16).view(np.int16)).view(torch.bfloat16)
    nxt = nxt.to(torch.float32).numpy()
    ok = np.isfinite(nxt) & (np.sign(nxt) == np.sign(base))
    half = (base[ok].astype(np.float64) + nxt[ok].astype(np.float64)) / 2
    quarter = base[ok].astype(np.float64) * 0.75 + nxt[ok].astype(np.float64) * 0.25
    rand = (rng.standard_normal(20000) * np.exp(rng.uniform(-87, 87, 20000))).astype(np.float32)
    x = np.concatenate([base, half.astype(np.float32), quarter.astype(np.float32), rand,
                        np.float32([3.4e38, -3.4e38, 1e-40, -1e-45, 0.0, -0.0])])
    assert np.array_equal(x.astype(np.float64).astype(np.float32), x)  # all exact in binary32
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.f64_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)
