// C ABI of the mnb library: argument checks, then launches.  Every entry point
// returns a status and never lets an exception escape (onnxruntime PR "INT3
// QMoE CUDA correctness baseline and Qwen experimental results", embedded
// P0/P1 body, section "Review Fixes and Padding Experiment Follow-up":
// no-exceptions guards).  Unsupported requests are rejected, never routed to
// another kernel ("Qwen3 Missing-Kernel Implementation Plan", section "Common
// implementation and performance gates").

#include <hip/hip_runtime.h>

#include <cstring>
#include <memory>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/mnb.h"
#include "../../include/mnb_debug.h"
#include "contract.h"
#include "kernels.h"

using namespace mnb;

// Workspace array of qmoe_forward_noalloc (see scratch_for_current_device).
constexpr uint64_t kScratchBytes = uint64_t(64) << 20;
static_assert(kScratchBytes == MNB_NOALLOC_SCRATCH_BYTES, "header and library must agree");
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

int32_t check_device(const mnb_plan* p) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MNB_ERR_DEVICE;
  return dev == p->device ? MNB_OK : MNB_ERR_INVALID_ARG;
}

int32_t check_ws(void* ws, uint64_t ws_bytes, uint64_t need) {
  if (need == 0) return MNB_OK;
  if (!ws || ws_bytes < need) return MNB_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned256(ws)) return MNB_ERR_INVALID_ARG;
  return MNB_OK;
}

int32_t prepare_common(const mnb_desc* desc, const uint8_t* B, const void* scales,
                       const uint8_t* zp, void* dst, uint64_t dst_bytes, bool device,
                       hipStream_t st, mnb_plan* plan) {
  if (!plan) return MNB_ERR_INVALID_ARG;
  std::memset(plan, 0, sizeof(*plan));
  Sizes s;
  int32_t rc = check_desc(desc, &s);
  if (rc != MNB_OK) return rc;
  if (!B || !scales || !dst || (desc->has_zero_points && !zp)) return MNB_ERR_INVALID_ARG;
  if (dst_bytes < s.total) return MNB_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned256(dst)) return MNB_ERR_INVALID_ARG;
  rc = validate_content(desc, s, B, scales, zp);
  if (rc != MNB_OK) return rc;
  int dev = -1;
  if (device) {
    // staging for the repacked bytes (left uninitialised: prepack writes
    // every byte)
    std::unique_ptr<uint8_t[]> host(new (std::nothrow) uint8_t[s.total]);
    if (!host) return MNB_ERR_HOST_MEMORY;
    prepack(s, B, scales, zp, host.get());
    if (hipGetDevice(&dev) != hipSuccess) return MNB_ERR_DEVICE;
    if (hipMemcpyAsync(dst, host.get(), s.total, hipMemcpyHostToDevice, st) != hipSuccess)
      return MNB_ERR_DEVICE;
    if (hipStreamSynchronize(st) != hipSuccess) return MNB_ERR_DEVICE;
  } else {
    prepack(s, B, scales, zp, static_cast<uint8_t*>(dst));
  }
  fill_plan(desc, s, dst, dev, plan);
  return MNB_OK;
}

int32_t check_qmoe(const mnb_plan* fc1, const mnb_plan* fc2, const qmoe_desc* q, int64_t T,
                   Sizes* s1, Sizes* s2) {
  if (!fc1 || !fc2 || !q || T < 0) return MNB_ERR_INVALID_ARG;
  int32_t rc = check_plan(fc1, s1);
  if (rc != MNB_OK) return rc;
  rc = check_plan(fc2, s2);
  if (rc != MNB_OK) return rc;
  if (q->abi_version != MNB_ABI_VERSION || q->reserved != 0) return MNB_ERR_INVALID_ARG;
  if (s1->kind != kMoe || s2->kind != kMoe) return MNB_ERR_UNSUPPORTED;
  if (q->normalize_routing_weights != 1 || q->activation != QMOE_ACT_SWIGLU ||
      q->gate_up != QMOE_GATE_UP_INTERLEAVED || q->weights_prepacked != 0 ||
      q->quant_type != QMOE_QUANT_INT)
    return MNB_ERR_UNSUPPORTED;
  // FC1 is [E, 2I, H], FC2 is [E, H, I]: H from FC1's K, I from FC1's rows
  if (s1->E != s2->E || s1->N % 2 || s2->K != s1->N / 2 || s2->N != s1->K)
    return MNB_ERR_INVALID_ARG;
  if (s1->bs != s2->bs) return MNB_ERR_UNSUPPORTED;
  // one 16-bit type for activations and scales across the layer [P1]
  if (fc1->desc.scale_dtype != fc2->desc.scale_dtype) return MNB_ERR_UNSUPPORTED;
  if (q->top_k < 1 || q->top_k > s1->E) return MNB_ERR_INVALID_ARG;
  if (!qmoe_supported(*s1, *s2, q->top_k)) return MNB_ERR_UNSUPPORTED;
  return MNB_OK;
}

// Workspace of qmoe_forward_noalloc: one array per GPU, held from the first
// use on that GPU until the process ends.  Its address is taken once per
// device with hipGetSymbolAddress (host code never passes the array's name
// to a kernel: on the host it is only a stand-in, not the device address).
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

// The device address of the current device's scratch array.
int32_t scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MNB_ERR_DEVICE;
  if (dev < 0 || dev >= kScratchDevices) return MNB_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MNB_ERR_DEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MNB_OK;
}

#define MNB_GUARD(...)           \
  try {                          \
    __VA_ARGS__                  \
  } catch (...) {                \
    return MNB_ERR_INVALID_ARG;  \
  }

}  // namespace

extern "C" {

const char* mnb_status_string(int32_t status) {
  switch (status) {
    case MNB_OK: return "MNB_OK";
    case MNB_ERR_INVALID_ARG: return "MNB_ERR_INVALID_ARG";
    case MNB_ERR_UNSUPPORTED: return "MNB_ERR_UNSUPPORTED";
    case MNB_ERR_SIZE_OVERFLOW: return "MNB_ERR_SIZE_OVERFLOW";
    case MNB_ERR_CONTENT: return "MNB_ERR_CONTENT";
    case MNB_ERR_WORKSPACE_TOO_SMALL: return "MNB_ERR_WORKSPACE_TOO_SMALL";
    case MNB_ERR_DEVICE: return "MNB_ERR_DEVICE";
    case MNB_ERR_STALE_PLAN: return "MNB_ERR_STALE_PLAN";
    case MNB_ERR_HOST_MEMORY: return "MNB_ERR_HOST_MEMORY";
    default: return "MNB_ERR_UNKNOWN";
  }
}

int32_t mnb_prepacked_size(const mnb_desc* desc, uint64_t* bytes) {
  MNB_GUARD({
    if (!bytes) return MNB_ERR_INVALID_ARG;
    Sizes s;
    const int32_t rc = check_desc(desc, &s);
    if (rc != MNB_OK) return rc;
    *bytes = s.total;
    return MNB_OK;
  })
}

int32_t mnb_prepare(const mnb_desc* desc, const uint8_t* B_host, const void* scales_host,
                    const uint8_t* zero_points_host, void* dst_dev, uint64_t dst_bytes,
                    void* stream, mnb_plan* plan) {
  MNB_GUARD({
    return prepare_common(desc, B_host, scales_host, zero_points_host, dst_dev, dst_bytes, true,
                          static_cast<hipStream_t>(stream), plan);
  })
}

int32_t mnb_prepare_host(const mnb_desc* desc, const uint8_t* B_host, const void* scales_host,
                         const uint8_t* zero_points_host, void* dst_host, uint64_t dst_bytes,
                         mnb_plan* plan) {
  MNB_GUARD({
    return prepare_common(desc, B_host, scales_host, zero_points_host, dst_host, dst_bytes, false,
                          nullptr, plan);
  })
}

int32_t mnb_gemv_workspace_size(const mnb_plan* plan, uint64_t* bytes) {
  MNB_GUARD({
    if (!bytes) return MNB_ERR_INVALID_ARG;
    Sizes s;
    const int32_t rc = check_plan(plan, &s);
    if (rc != MNB_OK) return rc;
    if (s.kind != kDenseInt4) return MNB_ERR_UNSUPPORTED;
    *bytes = gemv_ws_bytes(s);
    return MNB_OK;
  })
}

int32_t mnb_gemv(const mnb_plan* plan, const float* A_dev, float* Y_dev, void* ws_dev,
                 uint64_t ws_bytes, void* stream) {
  MNB_GUARD({
    Sizes s;
    int32_t rc = check_plan(plan, &s);
    if (rc != MNB_OK) return rc;
    if (s.kind != kDenseInt4) return MNB_ERR_UNSUPPORTED;
    if (!A_dev || !Y_dev) return MNB_ERR_INVALID_ARG;
    if ((rc = check_ws(ws_dev, ws_bytes, gemv_ws_bytes(s))) != MNB_OK) return rc;
    if ((rc = check_device(plan)) != MNB_OK) return rc;
    if (launch_gemv(s, *plan, A_dev, Y_dev, ws_dev, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
      return MNB_ERR_DEVICE;
    return MNB_OK;
  })
}

int32_t mnb_gemv_multi(const mnb_plan* const* plans, int32_t count, const float* A_dev,
                       float* const* Y_dev, void* ws_dev, uint64_t ws_bytes, void* stream) {
  MNB_GUARD({
    if (!plans || !Y_dev || !A_dev || count < 1 || count > kMaxSegs) return MNB_ERR_INVALID_ARG;
    Sizes s[kMaxSegs];
    uint64_t need = 0;
    for (int i = 0; i < count; ++i) {
      int32_t rc = check_plan(plans[i], &s[i]);
      if (rc != MNB_OK) return rc;
      if (s[i].kind != kDenseInt4) return MNB_ERR_UNSUPPORTED;
      if (!Y_dev[i] || s[i].K != s[0].K) return MNB_ERR_INVALID_ARG;
      const uint64_t w = gemv_ws_bytes(s[i]);
      need = w > need ? w : need;
    }
    int32_t rc = check_ws(ws_dev, ws_bytes, need);
    if (rc != MNB_OK) return rc;
    for (int i = 0; i < count; ++i)
      if ((rc = check_device(plans[i])) != MNB_OK) return rc;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (gemv_multi_fusable(s, count)) {
      if (launch_gemv_multi(s, plans, count, A_dev, Y_dev, st) != hipSuccess) return MNB_ERR_DEVICE;
      return MNB_OK;
    }
    for (int i = 0; i < count; ++i)
      if (launch_gemv(s[i], *plans[i], A_dev, Y_dev[i], ws_dev, st) != hipSuccess)
        return MNB_ERR_DEVICE;
    return MNB_OK;
  })
}

int32_t mnb_gemm_workspace_size(const mnb_plan* plan, int64_t M, uint64_t* bytes) {
  MNB_GUARD({
    if (!bytes || M < 0) return MNB_ERR_INVALID_ARG;
    Sizes s;
    const int32_t rc = check_plan(plan, &s);
    if (rc != MNB_OK) return rc;
    if (s.kind != kDenseInt4) return MNB_ERR_UNSUPPORTED;
    *bytes = gemm_ws_bytes(s, M);
    return MNB_OK;
  })
}

int32_t mnb_gemm(const mnb_plan* plan, int64_t M, const float* A_dev, float* Y_dev,
                 void* ws_dev, uint64_t ws_bytes, void* stream) {
  MNB_GUARD({
    Sizes s;
    int32_t rc = check_plan(plan, &s);
    if (rc != MNB_OK) return rc;
    if (s.kind != kDenseInt4) return MNB_ERR_UNSUPPORTED;
    if (M < 0) return MNB_ERR_INVALID_ARG;
    if (M == 0) return MNB_OK;
    uint64_t mk;
    if (__builtin_mul_overflow((uint64_t)M, (uint64_t)(s.K > s.N ? s.K : s.N), &mk) ||
        mk > (uint64_t)INT64_MAX / 4)
      return MNB_ERR_SIZE_OVERFLOW;
    if (!A_dev || !Y_dev) return MNB_ERR_INVALID_ARG;
    if ((rc = check_ws(ws_dev, ws_bytes, gemm_ws_bytes(s, M))) != MNB_OK) return rc;
    if ((rc = check_device(plan)) != MNB_OK) return rc;
    if (launch_gemm(s, *plan, M, A_dev, Y_dev, ws_dev, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
      return MNB_ERR_DEVICE;
    return MNB_OK;
  })
}

int32_t qmoe_workspace_size(const mnb_plan* fc1, const mnb_plan* fc2, const qmoe_desc* q,
                            int64_t T, uint64_t* bytes) {
  MNB_GUARD({
    if (!bytes) return MNB_ERR_INVALID_ARG;
    Sizes s1, s2;
    const int32_t rc = check_qmoe(fc1, fc2, q, T, &s1, &s2);
    if (rc != MNB_OK) return rc;
    *bytes = qmoe_ws_bytes(s1, s2, q->top_k, T);
    return MNB_OK;
  })
}

static int32_t qmoe_common(const mnb_plan* fc1, const mnb_plan* fc2, const qmoe_desc* q,
                           int64_t T, const uint16_t* x, const float* logits, const uint16_t* b1,
                           const uint16_t* b2, uint16_t* out, void* ws, uint64_t ws_bytes,
                           void* stream, const QmoeDebug* dbg) {
  Sizes s1, s2;
  int32_t rc = check_qmoe(fc1, fc2, q, T, &s1, &s2);
  if (rc != MNB_OK) return rc;
  if (T == 0) return MNB_OK;
  uint64_t th;
  if (__builtin_mul_overflow((uint64_t)T, (uint64_t)(s1.K > s1.E ? s1.K : s1.E), &th) ||
      th > (uint64_t)INT64_MAX / 64)
    return MNB_ERR_SIZE_OVERFLOW;
  if (!x || !logits || !out) return MNB_ERR_INVALID_ARG;
  // the kernels move x rows in 16-byte and outputs in 8-byte pieces
  if ((reinterpret_cast<uintptr_t>(x) & 15) || (reinterpret_cast<uintptr_t>(out) & 7) ||
      (reinterpret_cast<uintptr_t>(logits) & 3) || (reinterpret_cast<uintptr_t>(b1) & 1) ||
      (reinterpret_cast<uintptr_t>(b2) & 1))
    return MNB_ERR_INVALID_ARG;
  if ((rc = check_ws(ws, ws_bytes, qmoe_ws_bytes(s1, s2, q->top_k, T))) != MNB_OK) return rc;
  if ((rc = check_device(fc1)) != MNB_OK) return rc;
  if ((rc = check_device(fc2)) != MNB_OK) return rc;
  if (launch_qmoe(s1, *fc1, s2, *fc2, q->top_k, T, x, logits, b1, b2, out, ws,
                  static_cast<hipStream_t>(stream), dbg) != hipSuccess)
    return MNB_ERR_DEVICE;
  return MNB_OK;
}

int32_t qmoe_forward(const mnb_plan* fc1, const mnb_plan* fc2, const qmoe_desc* q, int64_t T,
                     const uint16_t* x_dev, const float* logits_dev, uint16_t* out_dev,
                     void* ws_dev, uint64_t ws_bytes, void* stream) {
  MNB_GUARD({
    return qmoe_common(fc1, fc2, q, T, x_dev, logits_dev, nullptr, nullptr, out_dev, ws_dev,
                       ws_bytes, stream, nullptr);
  })
}

int32_t qmoe_forward_noalloc(const mnb_plan* fc1, const mnb_plan* fc2, const qmoe_desc* q,
                             int64_t T, const uint16_t* x_dev, const float* logits_dev,
                             uint16_t* out_dev, void* stream) {
  MNB_GUARD({
    Sizes s1, s2;
    int32_t rc = check_qmoe(fc1, fc2, q, T, &s1, &s2);
    if (rc != MNB_OK) return rc;
    if (T == 0) return MNB_OK;
    // the size limit is checked on the host before any HIP call
    if (qmoe_ws_bytes(s1, s2, q->top_k, T) > kScratchBytes) return MNB_ERR_WORKSPACE_TOO_SMALL;
    void* ws = nullptr;
    if ((rc = check_device(fc1)) != MNB_OK) return rc;
    if ((rc = scratch_for_current_device(&ws)) != MNB_OK) return rc;
    // nothing in the workspace needs to start at zero: every kernel writes
    // what a later one reads before it is read
    return qmoe_common(fc1, fc2, q, T, x_dev, logits_dev, nullptr, nullptr, out_dev, ws,
                       kScratchBytes, stream, nullptr);
  })
}

int32_t qmoe_forward_biased(const mnb_plan* fc1, const mnb_plan* fc2, const qmoe_desc* q,
                            int64_t T, const uint16_t* x_dev, const float* logits_dev,
                            const uint16_t* fc1_bias_dev, const uint16_t* fc2_bias_dev,
                            uint16_t* out_dev, void* ws_dev, uint64_t ws_bytes, void* stream) {
  MNB_GUARD({
    return qmoe_common(fc1, fc2, q, T, x_dev, logits_dev, fc1_bias_dev, fc2_bias_dev, out_dev,
                       ws_dev, ws_bytes, stream, nullptr);
  })
}

int32_t qmoe_forward_debug(const mnb_plan* fc1, const mnb_plan* fc2, const qmoe_desc* q,
                           int64_t T, const uint16_t* x_dev, const float* logits_dev,
                           const uint16_t* fc1_bias_dev, const uint16_t* fc2_bias_dev,
                           uint16_t* out_dev, void* ws_dev, uint64_t ws_bytes, void* stream,
                           int32_t* ids_dev, float* w_dev, uint16_t* h_dev, float* slot_dev) {
  MNB_GUARD({
    QmoeDebug dbg{ids_dev, w_dev, h_dev, slot_dev};
    return qmoe_common(fc1, fc2, q, T, x_dev, logits_dev, fc1_bias_dev, fc2_bias_dev, out_dev,
                       ws_dev, ws_bytes, stream, &dbg);
  })
}

int32_t mnb_quantize_int3_rtn(const float* W_dev, int64_t rows, int64_t K, int32_t block_size,
                              int32_t scale_dtype, uint8_t* B_dev, uint16_t* scales_dev,
                              uint8_t* status_dev, void* stream) {
  MNB_GUARD({
    if (rows < 0 || K < 1 || block_size < 1) return MNB_ERR_INVALID_ARG;
    if (scale_dtype != MNB_DTYPE_F16 && scale_dtype != MNB_DTYPE_BF16) {
      return scale_dtype == MNB_DTYPE_F32 ? MNB_ERR_UNSUPPORTED : MNB_ERR_INVALID_ARG;
    }
    if (block_size != 32 && block_size != 64 && block_size != 128) return MNB_ERR_UNSUPPORTED;
    if (K % block_size) return MNB_ERR_UNSUPPORTED;
    uint64_t n;
    if (__builtin_mul_overflow((uint64_t)rows, (uint64_t)K, &n) || n > (uint64_t)INT64_MAX / 4)
      return MNB_ERR_SIZE_OVERFLOW;
    if (rows == 0) return MNB_OK;
    if (n / 8 / 256 >= (uint64_t)UINT32_MAX) return MNB_ERR_UNSUPPORTED;  // grid size
    if (!W_dev || !B_dev || !scales_dev || !status_dev) return MNB_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(W_dev) % 16 || reinterpret_cast<uintptr_t>(B_dev) % 4 ||
        reinterpret_cast<uintptr_t>(scales_dev) % 2)
      return MNB_ERR_INVALID_ARG;
    if (launch_rtn_int3(W_dev, rows, K, block_size, scale_dtype == MNB_DTYPE_BF16, B_dev,
                        scales_dev, status_dev, static_cast<hipStream_t>(stream)) != hipSuccess)
      return MNB_ERR_DEVICE;
    return MNB_OK;
  })
}

int32_t mnb_debug_stream_read(const void* const* src_dev, const uint64_t* bytes, int32_t count,
                              uint32_t* sink_dev, void* stream) {
  MNB_GUARD({
    if (!src_dev || !bytes || !sink_dev || count < 1 || count > kMaxSegs) return MNB_ERR_INVALID_ARG;
    for (int i = 0; i < count; ++i) {
      if (!src_dev[i] || (reinterpret_cast<uintptr_t>(src_dev[i]) & 15) || (bytes[i] & 15))
        return MNB_ERR_INVALID_ARG;
      if (bytes[i] / 16 / 1024 >= (uint64_t)UINT32_MAX / kMaxSegs) return MNB_ERR_UNSUPPORTED;
    }
    if (launch_stream_read(src_dev, bytes, count, sink_dev, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
      return MNB_ERR_DEVICE;
    return MNB_OK;
  })
}

int32_t mnb_debug_unpack_host(const mnb_plan* plan, int64_t expert, int64_t row0, int64_t nrows,
                              uint8_t* codes, uint8_t* zeros, void* scales) {
  MNB_GUARD({
    Sizes s;
    const int32_t rc = check_plan(plan, &s);
    if (rc != MNB_OK) return rc;
    if (plan->device != -1) return MNB_ERR_INVALID_ARG;  // host plans only
    if (expert < 0 || expert >= s.E || row0 < 0 || nrows < 0 || row0 + nrows > s.N)
      return MNB_ERR_INVALID_ARG;
    unpack_host(s, plan, expert, row0, nrows, codes, zeros, scales);
    return MNB_OK;
  })
}

int32_t mnb_debug_unpack(const mnb_plan* plan, int64_t expert, int64_t row0, int64_t nrows,
                         uint8_t* codes_dev, void* stream) {
  MNB_GUARD({
    Sizes s;
    int32_t rc = check_plan(plan, &s);
    if (rc != MNB_OK) return rc;
    if (expert < 0 || expert >= s.E || row0 < 0 || nrows < 0 || row0 + nrows > s.N ||
        (nrows && !codes_dev))
      return MNB_ERR_INVALID_ARG;
    if ((rc = check_device(plan)) != MNB_OK) return rc;
    if (launch_debug_unpack(s, *plan, expert, row0, nrows, codes_dev,
                            static_cast<hipStream_t>(stream)) != hipSuccess)
      return MNB_ERR_DEVICE;
    return MNB_OK;
  })
}

int32_t mnb_debug_dequant_f16(const mnb_plan* plan, int64_t expert, int64_t row0, int64_t nrows,
                              uint16_t* out_dev, void* stream) {
  MNB_GUARD({
    Sizes s;
    int32_t rc = check_plan(plan, &s);
    if (rc != MNB_OK) return rc;
    if (expert < 0 || expert >= s.E || row0 < 0 || nrows < 0 || row0 + nrows > s.N ||
        (nrows && !out_dev))
      return MNB_ERR_INVALID_ARG;
    if ((rc = check_device(plan)) != MNB_OK) return rc;
    if (launch_debug_dequant_f16(s, *plan, expert, row0, nrows, out_dev,
                                 static_cast<hipStream_t>(stream)) != hipSuccess)
      return MNB_ERR_DEVICE;
    return MNB_OK;
  })
}

}  // extern "C"
