/*
 * mnb_debug.h -- test-only entry points of the mnb library.  Production code
 * uses mnb.h; these exist so that the host contract can be tested without a
 * GPU and so that intermediate results can be compared stage by stage.
 *
 * Sources as in mnb.h; the stage checks follow the numerical-reference
 * approach of the onnxruntime PR "INT3 QMoE CUDA correctness baseline and
 * Qwen experimental results" (embedded P0/P1 body, section "P0: Portable
 * Format and Numerical References": independent scalar references and
 * handwritten vectors).
 */
#ifndef MNB_DEBUG_H
#define MNB_DEBUG_H

#include "mnb.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Host-only twin of mnb_prepare: identical checks and repacking, but the
 * prepacked layout is written to the host buffer dst_host (no HIP call is
 * made).  The resulting plan's pointers are host pointers; it may only be
 * passed to mnb_debug_unpack_host. */
int32_t mnb_prepare_host(const mnb_desc* desc, const uint8_t* B_host,
                         const void* scales_host,
                         const uint8_t* zero_points_host, void* dst_host,
                         uint64_t dst_bytes, mnb_plan* plan);

/* Reads a host plan's private layout back into contract terms for rows
 * [row0, row0 + nrows) of expert `expert`:
 *  codes  uint8 [nrows, K]  logical codes q (0 .. 2^bits - 1);
 *  zeros  uint8 [nrows, nb] zero points per block (NULL to skip);
 *  scales same dtype as the plan's, [nrows, nb] (NULL to skip). */
int32_t mnb_debug_unpack_host(const mnb_plan* plan, int64_t expert,
                              int64_t row0, int64_t nrows, uint8_t* codes,
                              uint8_t* zeros, void* scales);

/* Device version: a kernel reads the prepacked device layout of a device
 * plan and writes logical codes uint8 [nrows, K] to codes_dev on `stream`. */
int32_t mnb_debug_unpack(const mnb_plan* plan, int64_t expert, int64_t row0,
                         int64_t nrows, uint8_t* codes_dev, void* stream);

/* Device dequantization of rows [row0, row0 + nrows) of expert `expert` into
 * out_dev [nrows, K] using the exact rounding chain of the matrix-core path:
 * dense INT4: fp16(fma(q, s, -(z * s))) with the fma and z * s in fp32 (for the
 * implicit z = 8 this equals fp16(fp32((q - 8) * s))); QMoE: (q - 2^(bits-1)) * s
 * rounded once to the plan's 16-bit scale type.  out_dev holds binary16
 * patterns (bfloat16 patterns for BF16 QMoE plans). */
int32_t mnb_debug_dequant_f16(const mnb_plan* plan, int64_t expert,
                              int64_t row0, int64_t nrows, uint16_t* out_dev,
                              void* stream);

/* qmoe_forward_biased (biases may be NULL) that also copies out the routing
 * and the intermediates:
 *  ids_dev   int32 [T, top_k] selected experts, rank order;
 *  w_dev     fp32  [T, top_k] renormalized routing weights;
 *  h_dev     fp16  [T, top_k, I] SwiGLU activations fed to FC2;
 *  slot_dev  fp32  [T, top_k, H] r_j * (h_j . W2^T + b2) before the combine.
 * Any of the four may be NULL. */
int32_t qmoe_forward_debug(const mnb_plan* fc1, const mnb_plan* fc2,
                           const qmoe_desc* q, int64_t T,
                           const uint16_t* x_dev, const float* logits_dev,
                           const uint16_t* fc1_bias_dev,
                           const uint16_t* fc2_bias_dev, uint16_t* out_dev,
                           void* ws_dev, uint64_t ws_bytes, void* stream,
                           int32_t* ids_dev, float* w_dev,
                           uint16_t* h_dev, float* slot_dev);

/* Measurement aid: a plain streaming read of count (1..4) device buffers in
 * one launch, the ceiling against which the GEMV's achieved bandwidth is
 * reported.  Each thread issues four 16-byte nontemporal loads (16 KiB per
 * workgroup of 256), so bytes[i] / 16 KiB workgroups per buffer; the loaded
 * words are folded together and sink_dev (one uint32) is written only when the
 * fold equals a fixed improbable value, which keeps the loads from being
 * removed.  src_dev: host array of device pointers, each 16-byte aligned;
 * bytes: host array, multiples of 16 (0 allowed).  Asynchronous on `stream`.
 * Errors: INVALID_ARG (count, NULL or misaligned pointers, sizes), UNSUPPORTED
 * (grid too large), DEVICE. */
int32_t mnb_debug_stream_read(const void* const* src_dev, const uint64_t* bytes,
                              int32_t count, uint32_t* sink_dev, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MNB_DEBUG_H */
