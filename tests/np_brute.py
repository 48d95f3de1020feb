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


def silu_derivative(g):
    """d/dg [g * sigmoid(g)] by complex-step differentiation, Im f(g + i*h) / h
    with h = 1e-30: accurate to rounding and obtained without writing the
    closed-form derivative, so a wrong closed form elsewhere cannot hide."""
    step = 1e-30
    z = np.asarray(g, dtype=np.float64) + 1j * step
    return (z / (1.0 + np.exp(-z))).imag / step


def qmoe_tolerance_sums(x16, logits, W1, s1, W2, s2, k: int, bs: int, bits1: int = 3,
                        bits2: int = 3, b1=None, b2=None):
    """The QMoE tolerance sums for every expert, as whole-tensor products.

    gs[t, e, i] = sum_c |x[t, c] w1[e, 2i, c]| (+ |b1[e, 2i]|), us likewise on
    row 2i + 1, and the end-to-end sum
    S[t, n] = sum_e rw[t, e] sum_i |w2[e, n, i]| (|h| + |dh/dg| gs + |dh/du| us),
    with rw the renormalized top-k weights masked to the selected experts (zero
    elsewhere), dh/dg = u silu'(g) and dh/du = silu(g).  Returns (gs, us, S)
    with gs and us shaped [T, E, I]."""
    T, H = x16.shape
    E, twoI, _ = W1.shape
    I = twoI // 2
    w1 = moe_weights(W1, s1, H, bs, bits1)
    w2 = moe_weights(W2, s2, I, bs, bits2)
    x = x16.astype(np.float64)
    p = softmax(logits.astype(np.float64))
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    mask = np.zeros((T, E))
    np.put_along_axis(mask, order, 1.0, axis=1)
    rw = p * mask
    rw = rw / rw.sum(axis=1, keepdims=True)
    gs = np.zeros((T, E, I))
    us = np.zeros((T, E, I))
    S = np.zeros((T, H))
    for e in range(E):
        G = x @ w1[e, 0::2].T
        U = x @ w1[e, 1::2].T
        gs[:, e] = np.abs(x) @ np.abs(w1[e, 0::2]).T
        us[:, e] = np.abs(x) @ np.abs(w1[e, 1::2]).T
        if b1 is not None:
            bg = b1[e, 0::2].astype(np.float64)
            bu = b1[e, 1::2].astype(np.float64)
            G, U = G + bg, U + bu
            gs[:, e] += np.abs(bg)
            us[:, e] += np.abs(bu)
        silu = G / (1.0 + np.exp(-G))
        V = np.abs(silu * U) + np.abs(U * silu_derivative(G)) * gs[:, e] + np.abs(silu) * us[:, e]
        Ye = V @ np.abs(w2[e]).T
        if b2 is not None:
            Ye = Ye + np.abs(b2[e].astype(np.float64))
        S += rw[:, e:e + 1] * Ye
    return gs, us, S


def fc2_tolerance_sum(ids, h, W2, s2, I: int, bs: int, bits2: int = 3, b2=None):
    """yS[t, j, n] = sum_i |h[t, j, i] w2[ids[t, j], n, i]| (+ |b2[ids[t, j], n]|)."""
    w2 = moe_weights(W2, s2, I, bs, bits2)
    T, k = ids.shape
    yS = np.zeros((T, k, w2.shape[1]))
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            yS[t, j] = np.abs(w2[e]) @ np.abs(h[t, j])
            if b2 is not None:
                yS[t, j] += np.abs(b2[e].astype(np.float64))
    return yS
