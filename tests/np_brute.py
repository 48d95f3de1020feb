"""Brute-force numpy formulations used only to pin the oracle.

They are deliberately written differently from oracle.cpp: bit unpacking goes
through numpy.unpackbits(bitorder="little"), dequantization is whole-tensor
broadcasting, products are numpy float64 matmuls, and the MoE loops over every
expert with a k-hot mask instead of visiting only the selected ones.
"""
import numpy as np


def unpack_le(row_bytes: np.ndarray, n_codes: int, bits: int) -> np.ndarray:
    """Row-local LSB-first codes via numpy.unpackbits."""
    b = np.unpackbits(np.asarray(row_bytes, dtype=np.uint8), bitorder="little")
    b = b[: n_codes * bits].reshape(n_codes, bits).astype(np.int64)
    return b @ (1 << np.arange(bits, dtype=np.int64))


def int4_codes(B: np.ndarray, K: int) -> np.ndarray:
    """B [N, nb, bs/2] -> codes [N, K] (low nibble = even position)."""
    N, nb, half = B.shape
    c = np.empty((N, nb, 2 * half), dtype=np.int64)
    c[:, :, 0::2] = B & 0x0F
    c[:, :, 1::2] = B >> 4
    return c.reshape(N, nb * 2 * half)[:, :K]


def int4_zeros(zp, N: int, nb: int) -> np.ndarray:
    if zp is None:
        return np.full((N, nb), 8, dtype=np.int64)
    z = np.empty((N, zp.shape[1] * 2), dtype=np.int64)
    z[:, 0::2] = zp & 0x0F
    z[:, 1::2] = zp >> 4
    return z[:, :nb]


def dense_weights(B, scales, zp, K: int, bs: int) -> np.ndarray:
    N, nb, _ = B.shape
    q = int4_codes(B, K)
    z = np.repeat(int4_zeros(zp, N, nb), bs, axis=1)[:, :K]
    s = np.repeat(scales.astype(np.float64), bs, axis=1)[:, :K]
    return (q - z).astype(np.float64) * s


def dense_gemm(A, B, scales, zp, K: int, bs: int):
    W = dense_weights(B, scales, zp, K, bs)
    A64 = A.astype(np.float64)
    return A64 @ W.T, np.abs(A64) @ np.abs(W).T


def moe_weights(W: np.ndarray, s16: np.ndarray, K: int, bs: int, bits: int = 3) -> np.ndarray:
    """W uint8 [..., rows, rb] (row-local LSB-first codes of the given width),
    s16 float16 [..., rows, K/bs]; implicit zero point 2**(bits-1)."""
    lead = W.shape[:-1]
    flat = W.reshape(-1, W.shape[-1])
    q = np.stack([unpack_le(r, K, bits) for r in flat]).reshape(*lead, K)
    s = np.repeat(s16.astype(np.float64), bs, axis=-1)
    return (q - (1 << (bits - 1))).astype(np.float64) * s


def int3_weights(W: np.ndarray, s16: np.ndarray, K: int, bs: int) -> np.ndarray:
    return moe_weights(W, s16, K, bs, 3)


def softmax(v):
    v = np.asarray(v, dtype=np.float64)
    e = np.exp(v - v.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def qmoe_all_experts(x16, logits, W1, s1, W2, s2, k: int, bs: int, bits1: int = 3, bits2: int = 3,
                     b1=None, b2=None):
    """Every expert evaluated for every token, then a k-hot mask of the
    renormalized top-k probabilities selects the mixture."""
    T, H = x16.shape
    E, twoI, _ = W1.shape
    I = twoI // 2
    w1 = moe_weights(W1, s1, H, bs, bits1)    # [E, 2I, H]
    w2 = moe_weights(W2, s2, I, bs, bits2)    # [E, H, I]
    x = x16.astype(np.float64)
    p = softmax(logits.astype(np.float64))    # [T, E]
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    mask = np.zeros((T, E))
    np.put_along_axis(mask, order, 1.0, axis=1)
    pm = p * mask
    rw = pm / pm.sum(axis=1, keepdims=True)   # [T, E], zero off the top-k
    out = np.zeros((T, H))
    for e in range(E):
        G = x @ w1[e, 0::2].T                 # [T, I]
        U = x @ w1[e, 1::2].T
        if b1 is not None:
            G = G + b1[e, 0::2].astype(np.float64)
            U = U + b1[e, 1::2].astype(np.float64)
        Hh = G / (1.0 + np.exp(-G)) * U
        Y = Hh @ w2[e].T                      # [T, H]
        if b2 is not None:
            Y = Y + b2[e].astype(np.float64)
        out += rw[:, e:e + 1] * Y
    return out, order, np.take_along_axis(rw, order, axis=1)
