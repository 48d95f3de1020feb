// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "contract.h"

namespace mnb {

// ---- M = 1 GEMV on dense INT4 plans (gemv.hip) ----------------------------
uint64_t gemv_ws_bytes(const Sizes& s);
// several dense plans with the same K, block size and zero-point kind times
// one A in one launch (bit-identical to separate launches)
constexpr int kMaxSegs = 4;
bool gemv_multi_fusable(const Sizes* s, int count);
hipError_t launch_gemv_multi(const Sizes* s, const mnb_plan* const* p, int count, const float* A,
                             float* const* Y, hipStream_t st);
hipError_t launch_gemv(const Sizes& s, const mnb_plan& p, const float* A, float* Y,
                       void* ws, hipStream_t st);

// ---- small-M / prefill GEMM on dense INT4 plans (gemm.hip) ----------------
uint64_t gemm_ws_bytes(const Sizes& s, int64_t M);
hipError_t launch_gemm(const Sizes& s, const mnb_plan& p, int64_t M, const float* A,
                       float* Y, void* ws, hipStream_t st);

// single-launch small-M kernel (gemm_small.hip): M <= 4, or M <= 32 with
// N >= 4096; K % 128 == 0, K <= 8192, A 16-byte aligned; needs no workspace
bool gemm_small_supported(const Sizes& s, int64_t M, const void* A);
hipError_t launch_gemm_small(const Sizes& s, const mnb_plan& p, int64_t M, const float* A,
                             float* Y, hipStream_t st);

// large-M kernel streaming fp16 A and the codes through LDS (gemm_lds.hip);
// its workspace starts with an fp16 copy of A, then the split partials
bool gemm_lds_supported(const Sizes& s, int64_t M);
uint64_t gemm_lds_a16_bytes(const Sizes& s, int64_t M);
// (bm x (128 tn) tiles: 128 x 128, 256 x 256 or 256 x 128; with n_split > 0,
// which requires bm = 256 and splits = 1, 256 x 256 tiles over columns
// [0, n_split) and 256 x 128 tiles over the rest, in one launch)
hipError_t launch_gemm_lds(const Sizes& s, const mnb_plan& p, int64_t M, const float* A,
                           void* ws, float* Y, float* part, int32_t splits, int64_t kc, int bm,
                           int tn, int64_t n_split, hipStream_t st);

// ---- QMoE with INT3 / INT4 projections, fp16 or bf16 (qmoe.hip) ----------
struct QmoeDebug {
  int32_t* ids;
  float* w;
  uint16_t* h;
  float* slot;
};
// what the kernels support beyond the contract checks: at most 1024 experts,
// top_k <= 16, each expert's codes addressable with 32-bit offsets
bool qmoe_supported(const Sizes& s1, const Sizes& s2, int top_k);
uint64_t qmoe_ws_bytes(const Sizes& s1, const Sizes& s2, int top_k, int64_t T);
// b1 fp16 [E][2I] and b2 fp16 [E][H]: optional projection biases (nullptr: none)
hipError_t launch_qmoe(const Sizes& s1, const mnb_plan& p1, const Sizes& s2,
                       const mnb_plan& p2, int top_k, int64_t T, const uint16_t* x,
                       const float* logits, const uint16_t* b1, const uint16_t* b2,
                       uint16_t* out, void* ws, hipStream_t st, const QmoeDebug* dbg);

// ---- producer-side INT3 RTN quantizer (quant.hip) ---------------------------
// W fp32 [rows, K] (16-byte aligned), K % bs == 0, bs in {32, 64, 128};
// B [rows, 3K/8] (4-byte aligned), scales fp16 or bf16 (bf16) and status
// uint8 [rows, K/bs]
hipError_t launch_rtn_int3(const float* W, int64_t rows, int64_t K, int bs, bool bf16, uint8_t* B,
                           uint16_t* scales, uint8_t* status, hipStream_t st);

// ---- test-only readers of the device layout (debug.hip) --------------------
hipError_t launch_debug_unpack(const Sizes& s, const mnb_plan& p, int64_t expert,
                               int64_t row0, int64_t nrows, uint8_t* codes, hipStream_t st);
hipError_t launch_debug_dequant_f16(const Sizes& s, const mnb_plan& p, int64_t expert,
                                    int64_t row0, int64_t nrows, uint16_t* out,
                                    hipStream_t st);

// plain 16-byte nontemporal read of count (<= kMaxSegs) buffers in one launch
// (16-byte aligned, bytes multiples of 16); sink is written only for an
// improbable value, so that the loads are not removed
hipError_t launch_stream_read(const void* const* src, const uint64_t* bytes, int count,
                              uint32_t* sink, hipStream_t st);

inline uint64_t align256(uint64_t v) { return (v + 255) / 256 * 256; }

}  // namespace mnb
