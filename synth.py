"""Seeded synthetic inputs shared by the tests, the benchmark and smoke().

This module only draws random numbers and lays them out in the storage formats
of the operator contracts.  It holds none of the method's arithmetic: nothing
here unpacks a code, applies a scale or multiplies anything.  Both the oracle
and the HIP path receive exactly the bytes produced here.

Generator: splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), one independent stream per tensor with
seed = (config_id << 8) | tensor_id.  Uniforms take the top 53 bits times
2**-53; normals use Box-Muller in float64 and are then rounded once to the
storage dtype.  Packed code tensors are uniform random bytes: every nibble of
a uniform byte is a uniform 4-bit code, and every 3-bit field of a uniform bit
stream is a uniform 3-bit code, so no per-code packing is needed.  Padding
positions that the formats require to be zero are cleared.
"""
from __future__ import annotations

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def seed_for(config_id: int, tensor_id: int) -> int:
    return ((int(config_id) & 0xFFFFFFFFFFFFFF) << 8) | (int(tensor_id) & 0xFF)


def splitmix64(seed: int, n: int) -> np.ndarray:
    """The first n outputs of splitmix64 started from state `seed`."""
    n = int(n)
    with np.errstate(over="ignore"):
        idx = np.arange(1, n + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + idx * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform01(seed: int, n: int) -> np.ndarray:
    """float64 in [0, 1): top 53 bits of each draw times 2**-53."""
    return (splitmix64(seed, n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def normal(seed: int, n: int) -> np.ndarray:
    """float64 N(0, 1) by Box-Muller over consecutive uniform pairs."""
    m = (int(n) + 1) // 2
    u = uniform01(seed, 2 * m)
    u1 = 1.0 - u[0::2]  # (0, 1]
    u2 = u[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    z = np.empty(2 * m, dtype=np.float64)
    z[0::2] = r * np.cos(2.0 * np.pi * u2)
    z[1::2] = r * np.sin(2.0 * np.pi * u2)
    return z[: int(n)]


def random_bytes(seed: int, n: int) -> np.ndarray:
    words = splitmix64(seed, (int(n) + 7) // 8)
    return words.view(np.uint8)[: int(n)].copy()


# ----------------------------------------------------------------------------
# Dense MatMulNBits inputs (A fp32 [M,K]; B uint8 [N, nb, bs*bits/8];
# scales fp32 [N, nb]; optional packed 4-bit zero points [N, ceil(nb/2)]).
# ----------------------------------------------------------------------------

def activations_f32(seed: int, M: int, K: int) -> np.ndarray:
    return normal(seed, M * K).astype(np.float32).reshape(M, K)


def int4_blocked_weights(seed: int, N: int, K: int, bs: int, pad: str = "zero") -> np.ndarray:
    """uint8 [N, ceil(K/bs), bs/2], two 4-bit codes per byte.

    pad="zero" clears the nibbles of positions k >= K in the last block;
    pad="random" leaves them random (their value must not matter).
    """
    nb = -(-K // bs)
    B = random_bytes(seed, N * nb * (bs // 2)).reshape(N, nb, bs // 2)
    valid = K - (nb - 1) * bs
    if pad == "zero" and valid < bs:
        last = B[:, nb - 1, :]
        full_bytes = valid // 2
        if valid % 2:
            last[:, full_bytes] &= 0x0F
            last[:, full_bytes + 1:] = 0
        else:
            last[:, full_bytes:] = 0
    elif pad not in ("zero", "random"):
        raise ValueError(pad)
    return B


def scales_f32(seed: int, shape, lo: float = 0.005, hi: float = 0.02) -> np.ndarray:
    n = int(np.prod(shape))
    return (lo + (hi - lo) * uniform01(seed, n)).astype(np.float32).reshape(shape)


def int4_zero_points(seed: int, N: int, nb: int) -> np.ndarray:
    """uint8 [N, ceil(nb/2)] of uniform 4-bit zero points; a final unused
    high nibble (odd nb) is cleared."""
    zb = (nb + 1) // 2
    Z = random_bytes(seed, N * zb).reshape(N, zb)
    if nb % 2:
        Z[:, zb - 1] &= 0x0F
    return Z


# ----------------------------------------------------------------------------
# QMoE inputs (INT3 or INT4 row-local projections, fp16 scales).
# ----------------------------------------------------------------------------

def packed_rows(seed: int, rows: int, K: int, bits: int) -> np.ndarray:
    """uint8 [rows, ceil(bits*K/8)] of a uniform bit stream per row with the
    pad bits beyond bits*K cleared (canonical padding)."""
    rb = (bits * K + 7) // 8
    W = random_bytes(seed, rows * rb).reshape(rows, rb)
    used = (bits * K) % 8
    if used:
        W[:, rb - 1] &= np.uint8((1 << used) - 1)
    return W


def int3_rows(seed: int, rows: int, K: int) -> np.ndarray:
    return packed_rows(seed, rows, K, 3)


def scales_f16(seed: int, shape, lo: float = 0.005, hi: float = 0.02) -> np.ndarray:
    n = int(np.prod(shape))
    return (lo + (hi - lo) * uniform01(seed, n)).astype(np.float16).reshape(shape)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 patterns of float32 values, rounded to nearest even
    (the storage rounding of a bfloat16 tensor; inputs here are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def scales_bf16(seed: int, shape, lo: float = 0.005, hi: float = 0.02) -> np.ndarray:
    """uint16 bfloat16 patterns of uniform scales."""
    n = int(np.prod(shape))
    return to_bf16_bits((lo + (hi - lo) * uniform01(seed, n)).astype(np.float32)).reshape(shape)


def activations_bf16(seed: int, T: int, H: int) -> np.ndarray:
    """uint16 bfloat16 patterns of N(0,1) activations."""
    return to_bf16_bits(normal(seed, T * H).astype(np.float32)).reshape(T, H)


def activations_f16(seed: int, T: int, H: int) -> np.ndarray:
    return normal(seed, T * H).astype(np.float16).reshape(T, H)


def router_logits(seed: int, T: int, E: int) -> np.ndarray:
    """fp32 [T, E] holding fp16-representable N(0,1) values."""
    return normal(seed, T * E).astype(np.float16).astype(np.float32).reshape(T, E)


def small_int_activations(seed: int, M: int, K: int, lo: int = -8, hi: int = 7) -> np.ndarray:
    """fp32 [M, K] of integers uniform in [lo, hi] (exact-arithmetic cases)."""
    u = uniform01(seed, M * K)
    v = np.floor(u * (hi - lo + 1)) + lo
    return v.astype(np.float32).reshape(M, K)
