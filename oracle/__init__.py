"""TEST INFRASTRUCTURE ONLY: ctypes binding of the fp64 CPU oracle.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  The product library (block_quantized_weight_03_amd)
never imports or links it, and it never imports the product library.

The oracle is plain C++17 (oracle.cpp), compiled with g++ -O2 and
-ffp-contract=off.  Function-level documentation and the page citations are
in oracle.h.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so next to its source."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
               "-pthread", "-Wall", "-Wextra", "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = ctypes.CDLL(_LIB)
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with status {rc}")


I64 = ctypes.c_int64
INT = ctypes.c_int


def unpack_bits(row: np.ndarray, n_codes: int, bits: int) -> np.ndarray:
    row = np.ascontiguousarray(row, dtype=np.uint8)
    out = np.zeros(n_codes, dtype=np.uint8)
    _check(lib().orc_unpack_bits(_p(row), I64(n_codes), INT(bits), _p(out)), "unpack")
    return out


def pack_bits(codes: np.ndarray, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.zeros((codes.size * bits + 7) // 8, dtype=np.uint8)
    _check(lib().orc_pack_bits(_p(codes), I64(codes.size), INT(bits), _p(out)), "pack")
    return out


def padding_is_canonical(row: np.ndarray, n_codes: int, bits: int) -> bool:
    row = np.ascontiguousarray(row, dtype=np.uint8)
    rc = lib().orc_padding_is_canonical(_p(row), I64(n_codes), INT(bits))
    if rc < 0:
        raise ValueError("bad arguments")
    return rc == 1


def f16_to_f64(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.zeros(h.shape, dtype=np.float64)
    lib().orc_f16_to_f64_array(_p(h), I64(h.size), _p(out))
    return out


def f64_to_f16(x: np.ndarray) -> np.ndarray:
    """Returns the binary16 bit patterns (uint16)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    lib().orc_f64_to_f16_array(_p(x), I64(x.size), _p(out))
    return out


def mnb_gemm(A, B, scales, zp, K, N, bits=4, bs=32, nthreads=1):
    """Returns (Y fp32 [M,N], Y64, S)."""
    A = np.ascontiguousarray(A, dtype=np.float32)
    M = A.shape[0]
    B = np.ascontiguousarray(B, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    zp = None if zp is None else np.ascontiguousarray(zp, dtype=np.uint8)
    Y = np.zeros((M, N), dtype=np.float32)
    Y64 = np.zeros((M, N), dtype=np.float64)
    S = np.zeros((M, N), dtype=np.float64)
    _check(lib().orc_mnb_gemm(I64(M), I64(K), I64(N), INT(bits), INT(bs), _p(A), _p(B),
                              _p(scales), _p(zp), _p(Y), _p(Y64), _p(S), INT(nthreads)),
           "mnb_gemm")
    return Y, Y64, S


def mnb_dequant(B, scales, zp, K, N, bits=4, bs=32):
    B = np.ascontiguousarray(B, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    zp = None if zp is None else np.ascontiguousarray(zp, dtype=np.uint8)
    W = np.zeros((N, K), dtype=np.float64)
    _check(lib().orc_mnb_dequant(I64(K), I64(N), INT(bits), INT(bs), _p(B), _p(scales),
                                 _p(zp), _p(W)), "mnb_dequant")
    return W


def mnb_codes(B, zp, K, N, bits=4, bs=32):
    """Returns (codes uint8 [N,K], zero points uint8 [N,nb])."""
    B = np.ascontiguousarray(B, dtype=np.uint8)
    zp = None if zp is None else np.ascontiguousarray(zp, dtype=np.uint8)
    nb = -(-K // bs)
    codes = np.zeros((N, K), dtype=np.uint8)
    zeros = np.zeros((N, nb), dtype=np.uint8)
    _check(lib().orc_mnb_codes(I64(K), I64(N), INT(bits), INT(bs), _p(B), _p(zp),
                               _p(codes), _p(zeros)), "mnb_codes")
    return codes, zeros


def route(logits, k):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    _check(lib().orc_route(I64(T), INT(E), INT(k), _p(logits), _p(ids), _p(w)), "route")
    return ids, w


def _bits16(a, dtype):
    """16-bit patterns of fp16 values (dtype "f16": a float16 array) or of
    bfloat16 values (dtype "bf16": a uint16 array of bfloat16 patterns)."""
    if a is None:
        return None
    if dtype == "bf16":
        a = np.ascontiguousarray(a)
        assert a.dtype == np.uint16, "bf16 values are passed as uint16 patterns"
        return a
    return np.ascontiguousarray(a, dtype=np.float16).view(np.uint16)


def bf16_to_f64(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.zeros(h.shape, np.float64)
    _check(lib().orc_bf16_to_f64_array(_p(h), I64(h.size), _p(out)), "bf16_to_f64")
    return out


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.zeros(x.shape, np.uint16)
    _check(lib().orc_f64_to_bf16_array(_p(x), I64(x.size), _p(out)), "f64_to_bf16")
    return out


def qmoe(x_f16, logits, W1, s1, W2, s2, k=8, bits1=3, bits2=3, bs=64, nthreads=1, b1=None, b2=None,
         dtype="f16"):
    """x: [T,H]; s1, s2; optional biases b1 [E,2I] and b2 [E,H]; all float16
    (dtype "f16") or uint16 bfloat16 patterns (dtype "bf16").  Returns a dict
    of every output; "out16" holds the 16-bit patterns of out."""
    dt = 1 if dtype == "bf16" else 0
    x = _bits16(x_f16, dtype)
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    W1 = np.ascontiguousarray(W1, dtype=np.uint8)
    W2 = np.ascontiguousarray(W2, dtype=np.uint8)
    s1, s2 = _bits16(s1, dtype), _bits16(s2, dtype)
    b1, b2 = _bits16(b1, dtype), _bits16(b2, dtype)
    T, H = x.shape
    E = W1.shape[0]
    I = W1.shape[1] // 2
    o = dict(out16=np.zeros((T, H), np.uint16), out64=np.zeros((T, H)), S=np.zeros((T, H)),
             ids=np.zeros((T, k), np.int32), r=np.zeros((T, k)),
             g=np.zeros((T, k, I)), u=np.zeros((T, k, I)), h=np.zeros((T, k, I)),
             gs=np.zeros((T, k, I)), us=np.zeros((T, k, I)))
    _check(lib().orc_qmoe(I64(T), I64(H), I64(I), INT(E), INT(k), INT(bits1), INT(bits2),
                          INT(bs), INT(dt), _p(x), _p(logits), _p(W1), _p(s1), _p(W2), _p(s2),
                          _p(b1), _p(b2), _p(o["out16"]), _p(o["out64"]), _p(o["S"]), _p(o["ids"]), _p(o["r"]),
                          _p(o["g"]), _p(o["u"]), _p(o["h"]), _p(o["gs"]), _p(o["us"]),
                          INT(nthreads)), "qmoe")
    o["out"] = o["out16"].view(np.float16) if dt == 0 else bf16_to_f64(o["out16"])
    return o


def qmoe_fc2(ids, h, W2, s2, H, I, E, bits2=3, bs=64, nthreads=1, b2=None, dtype="f16"):
    """h: fp64 [T,k,I].  Returns (y [T,k,H], yS [T,k,H])."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    h = np.ascontiguousarray(h, dtype=np.float64)
    W2 = np.ascontiguousarray(W2, dtype=np.uint8)
    s2, b2 = _bits16(s2, dtype), _bits16(b2, dtype)
    T, k = ids.shape
    y = np.zeros((T, k, H))
    yS = np.zeros((T, k, H))
    _check(lib().orc_qmoe_fc2(I64(T), I64(H), I64(I), INT(E), INT(k), INT(bits2), INT(bs),
                              INT(1 if dtype == "bf16" else 0), _p(ids), _p(h), _p(W2), _p(s2), _p(b2), _p(y), _p(yS),
                              INT(nthreads)),
           "qmoe_fc2")
    return y, yS


def rtn_int3(W, bs, dtype="f16"):
    """W: float32 [rows, K].  Returns (B uint8 [rows, ceil(3K/8)], scales
    [rows, K/bs] (float16, or uint16 bfloat16 patterns for dtype "bf16"),
    status uint8 [rows, K/bs])."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    rows, K = W.shape
    B = np.zeros((rows, (3 * K + 7) // 8), np.uint8)
    s = np.zeros((rows, K // bs), np.uint16)
    st = np.zeros((rows, K // bs), np.uint8)
    _check(lib().orc_rtn_int3(I64(rows), I64(K), INT(bs), INT(1 if dtype == "bf16" else 0), _p(W),
                              _p(B), _p(s), _p(st)), "rtn_int3")
    return B, (s if dtype == "bf16" else s.view(np.float16)), st
