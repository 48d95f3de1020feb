"""Python binding of libmnb.so, the block-quantized weight-only matmul library
for AMD Instinct MI355X (gfx950).

Argument marshalling only: every function below forwards to the C entry point
of the same name in include/mnb.h (or include/mnb_debug.h).  All arithmetic
runs in the library's HIP kernels; torch is used by callers for device memory
and streams.  There is no fallback: if libmnb.so is missing or a call fails,
an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmnb.so")

MNB_ABI_VERSION = 1
MNB_DTYPE_F32, MNB_DTYPE_F16, MNB_DTYPE_BF16 = 0, 1, 2
MNB_ROWS_BLOCKED, MNB_ROWS_ROW_LOCAL = 0, 1
QMOE_ACT_SWIGLU = 1
QMOE_GATE_UP_INTERLEAVED = 1
QMOE_QUANT_INT = 0
MNB_NOALLOC_SCRATCH_BYTES = 64 << 20  # the static workspace of qmoe_forward_noalloc

STATUS = {0: "MNB_OK", -1: "MNB_ERR_INVALID_ARG", -2: "MNB_ERR_UNSUPPORTED",
          -3: "MNB_ERR_SIZE_OVERFLOW", -4: "MNB_ERR_CONTENT", -5: "MNB_ERR_WORKSPACE_TOO_SMALL",
          -6: "MNB_ERR_DEVICE", -7: "MNB_ERR_STALE_PLAN", -8: "MNB_ERR_HOST_MEMORY"}


class MnbError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status})")
        self.status = status


class mnb_desc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("accuracy_level", ctypes.c_int32),
                ("K", ctypes.c_int64), ("N", ctypes.c_int64),
                ("scale_dtype", ctypes.c_int32), ("has_zero_points", ctypes.c_int32),
                ("row_layout", ctypes.c_int32), ("num_experts", ctypes.c_int32)]


class mnb_plan(ctypes.Structure):
    _fields_ = [("desc", mnb_desc), ("magic", ctypes.c_uint32), ("layout_version", ctypes.c_uint32),
                ("n_blocks", ctypes.c_int64), ("row_bytes", ctypes.c_int64),
                ("codes_bytes", ctypes.c_uint64), ("scales_bytes", ctypes.c_uint64),
                ("zeros_bytes", ctypes.c_uint64), ("total_bytes", ctypes.c_uint64),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p),
                ("device", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class qmoe_desc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("normalize_routing_weights", ctypes.c_int32), ("activation", ctypes.c_int32),
                ("gate_up", ctypes.c_int32), ("weights_prepacked", ctypes.c_int32),
                ("quant_type", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_P = ctypes.c_void_p
_I32, _I64, _U64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
_PD, _PPLAN, _PQ = ctypes.POINTER(mnb_desc), ctypes.POINTER(mnb_plan), ctypes.POINTER(qmoe_desc)
_PU64 = ctypes.POINTER(ctypes.c_uint64)

# name -> argtypes; every function returns int32 except mnb_status_string
SIGNATURES = {
    # include/mnb.h
    "mnb_status_string": [_I32],
    "mnb_prepacked_size": [_PD, _PU64],
    "mnb_prepare": [_PD, _P, _P, _P, _P, _U64, _P, _PPLAN],
    "mnb_gemv_workspace_size": [_PPLAN, _PU64],
    "mnb_gemv": [_PPLAN, _P, _P, _P, _U64, _P],
    "mnb_gemv_multi": [_P, _I32, _P, _P, _P, _U64, _P],
    "mnb_gemm_workspace_size": [_PPLAN, _I64, _PU64],
    "mnb_gemm": [_PPLAN, _I64, _P, _P, _P, _U64, _P],
    "qmoe_workspace_size": [_PPLAN, _PPLAN, _PQ, _I64, _PU64],
    "qmoe_forward": [_PPLAN, _PPLAN, _PQ, _I64, _P, _P, _P, _P, _U64, _P],
    "qmoe_forward_biased": [_PPLAN, _PPLAN, _PQ, _I64, _P, _P, _P, _P, _P, _P, _U64, _P],
    "qmoe_forward_noalloc": [_PPLAN, _PPLAN, _PQ, _I64, _P, _P, _P, _P],
    "mnb_quantize_int3_rtn": [_P, _I64, _I64, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P],
    # include/mnb_debug.h
    "mnb_prepare_host": [_PD, _P, _P, _P, _P, _U64, _PPLAN],
    "mnb_debug_unpack_host": [_PPLAN, _I64, _I64, _I64, _P, _P, _P],
    "mnb_debug_unpack": [_PPLAN, _I64, _I64, _I64, _P, _P],
    "mnb_debug_dequant_f16": [_PPLAN, _I64, _I64, _I64, _P, _P],
    "qmoe_forward_debug": [_PPLAN, _PPLAN, _PQ, _I64, _P, _P, _P, _P, _P, _P, _U64, _P, _P, _P, _P,
                           _P],
    "mnb_debug_stream_read": [_P, _P, _I32, _P, _P],
}

_lib = None


def lib():
    """Loads libmnb.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        # torch ships its own HIP runtime under the same soname; loading torch
        # first makes libmnb.so bind to that one.  Loaded the other way round,
        # the process holds two HIP runtimes and the library cannot use device
        # pointers or streams that torch created (every device call fails).
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p if name == "mnb_status_string" else ctypes.c_int32
        _lib = L
    return _lib


def _check(rc: int, where: str):
    if rc != 0:
        raise MnbError(rc, where)


def _ptr(x):
    """Raw address of a torch tensor, a numpy array, an int or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    return x.data_ptr()  # torch.Tensor


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------------------
# descriptors
# ---------------------------------------------------------------------------

def dense_desc(K: int, N: int, block_size: int = 32, has_zero_points: bool = False,
               accuracy_level: int = 4) -> mnb_desc:
    return mnb_desc(MNB_ABI_VERSION, 4, block_size, accuracy_level, K, N, MNB_DTYPE_F32,
                    int(bool(has_zero_points)), MNB_ROWS_BLOCKED, 1)


def qmoe_proj_desc(K: int, N: int, num_experts: int, block_size: int = 64,
                   bits: int = 3, scale_dtype: int = MNB_DTYPE_F16) -> mnb_desc:
    return mnb_desc(MNB_ABI_VERSION, bits, block_size, 0, K, N, scale_dtype, 0,
                    MNB_ROWS_ROW_LOCAL, num_experts)


def make_qmoe_desc(top_k: int = 8) -> qmoe_desc:
    return qmoe_desc(MNB_ABI_VERSION, top_k, 1, QMOE_ACT_SWIGLU, QMOE_GATE_UP_INTERLEAVED, 0,
                     QMOE_QUANT_INT, 0)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def mnb_status_string(status: int) -> str:
    return lib().mnb_status_string(status).decode()


def mnb_prepacked_size(desc: mnb_desc) -> int:
    out = ctypes.c_uint64()
    _check(lib().mnb_prepacked_size(ctypes.byref(desc), ctypes.byref(out)), "mnb_prepacked_size")
    return out.value


def mnb_prepare(desc: mnb_desc, B_host: np.ndarray, scales_host: np.ndarray, zp_host,
                dst_dev, dst_bytes: int, stream=None) -> mnb_plan:
    plan = mnb_plan()
    B_host = np.ascontiguousarray(B_host)
    scales_host = np.ascontiguousarray(scales_host)
    zp_host = None if zp_host is None else np.ascontiguousarray(zp_host)
    _check(lib().mnb_prepare(ctypes.byref(desc), _ptr(B_host), _ptr(scales_host), _ptr(zp_host),
                             _ptr(dst_dev), dst_bytes, _stream(stream), ctypes.byref(plan)),
           "mnb_prepare")
    return plan


def mnb_prepare_host(desc: mnb_desc, B_host, scales_host, zp_host, dst_host: np.ndarray) -> mnb_plan:
    plan = mnb_plan()
    B_host = np.ascontiguousarray(B_host)
    scales_host = np.ascontiguousarray(scales_host)
    zp_host = None if zp_host is None else np.ascontiguousarray(zp_host)
    _check(lib().mnb_prepare_host(ctypes.byref(desc), _ptr(B_host), _ptr(scales_host),
                                  _ptr(zp_host), _ptr(dst_host), dst_host.nbytes,
                                  ctypes.byref(plan)), "mnb_prepare_host")
    return plan


def mnb_gemv_workspace_size(plan: mnb_plan) -> int:
    out = ctypes.c_uint64()
    _check(lib().mnb_gemv_workspace_size(ctypes.byref(plan), ctypes.byref(out)),
           "mnb_gemv_workspace_size")
    return out.value


def mnb_gemv(plan: mnb_plan, A_dev, Y_dev, ws_dev, ws_bytes: int, stream=None):
    _check(lib().mnb_gemv(ctypes.byref(plan), _ptr(A_dev), _ptr(Y_dev), _ptr(ws_dev), ws_bytes,
                          _stream(stream)), "mnb_gemv")


def mnb_gemv_multi(plans, A_dev, Y_devs, ws_dev, ws_bytes: int, stream=None):
    """plans: sequence of mnb_plan; Y_devs: one output per plan."""
    n = len(plans)
    if n != len(Y_devs):
        raise ValueError("one output per plan")
    parr = (ctypes.POINTER(mnb_plan) * max(n, 1))(*[ctypes.pointer(p) for p in plans])
    yarr = (ctypes.c_void_p * max(n, 1))(*[_ptr(y) for y in Y_devs])
    _check(lib().mnb_gemv_multi(ctypes.cast(parr, ctypes.c_void_p), n, _ptr(A_dev),
                                ctypes.cast(yarr, ctypes.c_void_p), _ptr(ws_dev), ws_bytes,
                                _stream(stream)), "mnb_gemv_multi")


def mnb_gemm_workspace_size(plan: mnb_plan, M: int) -> int:
    out = ctypes.c_uint64()
    _check(lib().mnb_gemm_workspace_size(ctypes.byref(plan), M, ctypes.byref(out)),
           "mnb_gemm_workspace_size")
    return out.value


def mnb_gemm(plan: mnb_plan, M: int, A_dev, Y_dev, ws_dev, ws_bytes: int, stream=None):
    _check(lib().mnb_gemm(ctypes.byref(plan), M, _ptr(A_dev), _ptr(Y_dev), _ptr(ws_dev), ws_bytes,
                          _stream(stream)), "mnb_gemm")


def qmoe_workspace_size(fc1: mnb_plan, fc2: mnb_plan, q: qmoe_desc, T: int) -> int:
    out = ctypes.c_uint64()
    _check(lib().qmoe_workspace_size(ctypes.byref(fc1), ctypes.byref(fc2), ctypes.byref(q), T,
                                     ctypes.byref(out)), "qmoe_workspace_size")
    return out.value


def qmoe_forward(fc1: mnb_plan, fc2: mnb_plan, q: qmoe_desc, T: int, x_dev, logits_dev, out_dev,
                 ws_dev, ws_bytes: int, stream=None):
    _check(lib().qmoe_forward(ctypes.byref(fc1), ctypes.byref(fc2), ctypes.byref(q), T, _ptr(x_dev),
                              _ptr(logits_dev), _ptr(out_dev), _ptr(ws_dev), ws_bytes,
                              _stream(stream)), "qmoe_forward")


def qmoe_forward_noalloc(fc1: mnb_plan, fc2: mnb_plan, q: qmoe_desc, T: int, x_dev, logits_dev,
                         out_dev, stream=None):
    _check(lib().qmoe_forward_noalloc(ctypes.byref(fc1), ctypes.byref(fc2), ctypes.byref(q), T,
                                      _ptr(x_dev), _ptr(logits_dev), _ptr(out_dev),
                                      _stream(stream)), "qmoe_forward_noalloc")


def mnb_quantize_int3_rtn(W_dev, rows: int, K: int, block_size: int, B_dev, scales_dev,
                          status_dev, stream=None, scale_dtype: int = MNB_DTYPE_F16):
    """Enqueues the INT3 RTN quantizer; read status_dev after the stream ends."""
    _check(lib().mnb_quantize_int3_rtn(_ptr(W_dev), rows, K, block_size, scale_dtype, _ptr(B_dev),
                                       _ptr(scales_dev), _ptr(status_dev), _stream(stream)),
           "mnb_quantize_int3_rtn")


def quantize_int3_rtn(W, block_size: int = 64, stream=None, scale_dtype: int = MNB_DTYPE_F16):
    """fp32 device weights [rows, K] -> (B uint8 [rows, 3K/8], scales [rows,
    K/bs]: float16, or bfloat16 patterns in int16 for MNB_DTYPE_BF16) as device
    tensors; raises MnbError(CONTENT) when a group is rejected (non-finite
    weight or a scale the type cannot store)."""
    import torch
    rows, K = W.shape
    B = torch.empty((rows, 3 * K // 8), dtype=torch.uint8, device=W.device)
    s = torch.empty((rows, K // block_size),
                    dtype=torch.int16 if scale_dtype == MNB_DTYPE_BF16 else torch.float16,
                    device=W.device)
    st = torch.empty((rows, K // block_size), dtype=torch.uint8, device=W.device)
    mnb_quantize_int3_rtn(W, rows, K, block_size, B, s, st, stream, scale_dtype)
    if rows and int(st.max().item()) != 0:
        raise MnbError(-4, "quantize_int3_rtn")  # MNB_ERR_CONTENT
    return B, s


def qmoe_forward_biased(fc1: mnb_plan, fc2: mnb_plan, q: qmoe_desc, T: int, x_dev, logits_dev,
                        fc1_bias_dev, fc2_bias_dev, out_dev, ws_dev, ws_bytes: int, stream=None):
    _check(lib().qmoe_forward_biased(ctypes.byref(fc1), ctypes.byref(fc2), ctypes.byref(q), T,
                                     _ptr(x_dev), _ptr(logits_dev), _ptr(fc1_bias_dev),
                                     _ptr(fc2_bias_dev), _ptr(out_dev), _ptr(ws_dev), ws_bytes,
                                     _stream(stream)), "qmoe_forward_biased")


def qmoe_forward_debug(fc1, fc2, q, T, x_dev, logits_dev, out_dev, ws_dev, ws_bytes, stream=None,
                       ids_dev=None, w_dev=None, h_dev=None, slot_dev=None, fc1_bias_dev=None,
                       fc2_bias_dev=None):
    _check(lib().qmoe_forward_debug(ctypes.byref(fc1), ctypes.byref(fc2), ctypes.byref(q), T,
                                    _ptr(x_dev), _ptr(logits_dev), _ptr(fc1_bias_dev),
                                    _ptr(fc2_bias_dev), _ptr(out_dev), _ptr(ws_dev),
                                    ws_bytes, _stream(stream), _ptr(ids_dev), _ptr(w_dev),
                                    _ptr(h_dev), _ptr(slot_dev)), "qmoe_forward_debug")


def mnb_debug_unpack_host(plan: mnb_plan, expert: int, row0: int, nrows: int, want_scales=True):
    """Returns (codes [nrows,K], zeros [nrows,nb], scales [nrows,nb]) from a host plan."""
    K, nb = plan.desc.K, plan.n_blocks
    codes = np.zeros((nrows, K), np.uint8)
    zeros = np.zeros((nrows, nb), np.uint8)
    sdt = np.float32 if plan.desc.scale_dtype == MNB_DTYPE_F32 else np.float16
    scales = np.zeros((nrows, nb), sdt) if want_scales else None
    _check(lib().mnb_debug_unpack_host(ctypes.byref(plan), expert, row0, nrows, _ptr(codes),
                                       _ptr(zeros), _ptr(scales)), "mnb_debug_unpack_host")
    return codes, zeros, scales


def mnb_debug_stream_read(buffers, sink_dev, stream=None):
    """buffers: list of (device pointer or tensor, bytes) pairs, 1 to 4."""
    n = len(buffers)
    ptrs = (ctypes.c_void_p * max(n, 1))(*[_ptr(b) for b, _ in buffers])
    sizes = (ctypes.c_uint64 * max(n, 1))(*[int(nb) for _, nb in buffers])
    _check(lib().mnb_debug_stream_read(ptrs, sizes, n, _ptr(sink_dev), _stream(stream)),
           "mnb_debug_stream_read")


def mnb_debug_unpack(plan: mnb_plan, expert: int, row0: int, nrows: int, codes_dev, stream=None):
    _check(lib().mnb_debug_unpack(ctypes.byref(plan), expert, row0, nrows, _ptr(codes_dev),
                                  _stream(stream)), "mnb_debug_unpack")


def mnb_debug_dequant_f16(plan: mnb_plan, expert: int, row0: int, nrows: int, out_dev, stream=None):
    _check(lib().mnb_debug_dequant_f16(ctypes.byref(plan), expert, row0, nrows, _ptr(out_dev),
                                       _stream(stream)), "mnb_debug_dequant_f16")


# ---------------------------------------------------------------------------
# torch-side convenience: owns the prepacked device buffer of one weight
# ---------------------------------------------------------------------------

class PreparedWeight:
    """Device buffer + plan of one prepared weight (caller-side ownership)."""

    def __init__(self, desc: mnb_desc, B_host, scales_host, zp_host=None, device="cuda"):
        import torch
        self.desc = desc
        nbytes = mnb_prepacked_size(desc)
        self.buffer = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        self.plan = mnb_prepare(desc, B_host, scales_host, zp_host, self.buffer, self.buffer.numel())

    def gemv(self, A, Y=None, ws=None, stream=None):
        import torch
        if Y is None:
            Y = torch.empty(self.desc.N, dtype=torch.float32, device=A.device)
        need = mnb_gemv_workspace_size(self.plan)
        if ws is None:
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device=A.device)
        mnb_gemv(self.plan, A, Y, ws, ws.numel(), stream)
        return Y

    def gemm(self, A, Y=None, ws=None, stream=None):
        import torch
        M = A.shape[0]
        if Y is None:
            Y = torch.empty((M, self.desc.N), dtype=torch.float32, device=A.device)
        need = mnb_gemm_workspace_size(self.plan, M)
        if ws is None and need:
            ws = torch.empty(need, dtype=torch.uint8, device=A.device)
        mnb_gemm(self.plan, M, A, Y, ws, 0 if ws is None else ws.numel(), stream)
        return Y
