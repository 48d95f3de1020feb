/*
 * TEST INFRASTRUCTURE ONLY.  fp64 CPU reference ("oracle") for block-quantized
 * weight-only matmul (MatMulNBits), the top-k QMoE layer (INT3 / INT4 projections,
 * fp16 or bf16) and the INT3 round-to-nearest producer quantizer.
 *
 * Only the tests, smoke() and the benchmark's CPU-baseline leg may load this
 * library.  It shares no code, header or table with the HIP library: the two
 * are written independently from the same pages so that one can check the
 * other.
 *
 * Sources (page title, then section):
 *  [PLAN]  "Qwen3 Missing-Kernel Implementation Plan" (onnx-light CPU docs),
 *          section "PR sequence", steps K01 (contract: FP32 A, UINT8 packed B,
 *          FP32 scales, bits=4, block_size=32, implicit zero points, scale
 *          indexing, padding), K02 (M=1 decode GEMV) and K03 (small-M/prefill).
 *  [P0]    onnxruntime PR "INT3 QMoE CUDA correctness baseline and Qwen
 *          experimental results", embedded body of the stacked P0/P1 PR,
 *          section "P0: Portable Format and Numerical References" (row-local
 *          LSB-first UINT8 packing for widths 1..8, canonical padding, INT3
 *          offset-4 decoding, deterministic RTN with stored-scale
 *          rounding and subnormal-underflow reporting, tiny
 *          predetermined-route SwiGLU MoE).
 *  [P1]    same body, section "P1: Compatible QMoE v1 Extension" (fused
 *          interleaved gate/up, activation_type swiglu, block sizes 32/64/128,
 *          I inferred from the fused FC1 rows).
 *  [OLIVE] same page, embedded Olive body ("Summary"): INT3 dequantization is
 *          (code - 4) * scale with implicit zero point 4; the symmetric RTN
 *          scale policy max|w| / 3.5, all-zero groups with scale 1 / 3.5 and
 *          code 4, and rejection of non-finite weights and of scales that
 *          round to zero for a nonzero group.
 *  [ROUTE] pegainfer PR "feat(qwen4): component kernels extracted from the
 *          brick PRs", section "Description": MoE routing is an fp32 softmax,
 *          top-k, then renormalization of the selected probabilities
 *          (norm_topk_prob); combine sums the branch outputs.
 *
 * All functions return 0 on success and a negative value on bad arguments.
 */
#ifndef MNB_ORACLE_H
#define MNB_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- bit packing [P0] ---------------------------------------------------- */
int orc_unpack_bits(const uint8_t* row, int64_t n_codes, int bits, uint8_t* codes);
int orc_pack_bits(const uint8_t* codes, int64_t n_codes, int bits, uint8_t* row);
/* 1 if every bit after n_codes*bits in the last byte is zero, else 0. */
int orc_padding_is_canonical(const uint8_t* row, int64_t n_codes, int bits);

/* ---- IEEE binary16 conversions (RN-even) --------------------------------- */
double orc_f16_to_f64(uint16_t h);
uint16_t orc_f64_to_f16(double x);
int orc_f16_to_f64_array(const uint16_t* h, int64_t n, double* out);
int orc_f64_to_f16_array(const double* x, int64_t n, uint16_t* out);

/* ---- bfloat16 conversions (RN-even; bf16 = top half of binary32) --------- */
double orc_bf16_to_f64(uint16_t b);
uint16_t orc_f64_to_bf16(double x);
int orc_bf16_to_f64_array(const uint16_t* h, int64_t n, double* out);
int orc_f64_to_bf16_array(const double* x, int64_t n, uint16_t* out);

/* ---- MatMulNBits [PLAN K01-K03] -------------------------------------------
 * A fp32 [M,K]; B uint8 [N, nb, bs*bits/8] with nb = ceil(K/bs); scales fp32
 * [N, nb]; zp NULL (implicit 2^(bits-1)) or uint8 [N, ceil(nb*bits/8)] of
 * zero points packed like the codes.  Outputs (any may be NULL):
 *   Y   fp32 [M,N] = fp64 result rounded once;
 *   Y64 fp64 [M,N];
 *   S   fp64 [M,N] = sum_k |A[m,k] * w[n,k]|  (the tolerance sum).        */
int orc_mnb_gemm(int64_t M, int64_t K, int64_t N, int bits, int bs,
                 const float* A, const uint8_t* B, const float* scales,
                 const uint8_t* zp, float* Y, double* Y64, double* S,
                 int nthreads);
/* Dequantized weights in fp64, W [N,K] = (q - z) * s. */
int orc_mnb_dequant(int64_t K, int64_t N, int bits, int bs, const uint8_t* B,
                    const float* scales, const uint8_t* zp, double* W);
/* Logical codes [N,K] and zero points [N,nb] as bytes. */
int orc_mnb_codes(int64_t K, int64_t N, int bits, int bs, const uint8_t* B,
                  const uint8_t* zp, uint8_t* codes, uint8_t* zeros);

/* ---- QMoE routing [ROUTE] -------------------------------------------------
 * logits fp32 [T,E] -> ids int32 [T,k] (logit descending, lower index first
 * on ties) and weights fp64 [T,k] = softmax over the selected logits, which
 * equals softmax over all E followed by renormalization of the top k.     */
int orc_route(int64_t T, int E, int k, const float* logits, int32_t* ids,
              double* weights);

/* ---- INT3 QMoE layer [P0][P1][OLIVE] --------------------------------------
 * dtype 0: x, scales, biases and out are IEEE fp16; dtype 1: all bfloat16
 * ([P1]: matching FP16/BF16 activation and scale types).
 * x [T,H]; logits fp32 [T,E];
 * W1 uint8 [E, 2I, ceil(bits1*H/8)], rows 2i = gate_i and 2i+1 = up_i;
 * s1 fp16 [E, 2I, H/bs]; W2 uint8 [E, H, ceil(bits2*I/8)]; s2 fp16 [E, H, I/bs];
 * implicit zero points 2^(bits-1); optional biases ([P1] "optional biases";
 * NULL = none): b1 fp16 [E, 2I] added to the gate/up rows before SwiGLU, b2
 * fp16 [E, H] added to each expert's FC2 output before its routing weight;
 * a bias counts as one more product term (1 * b) in the tolerance sums.
 * Outputs (any may be NULL): out16 fp16 [T,H]; out64 fp64 [T,H]; S fp64 [T,H]
 * (first-order tolerance sum, see orc_qmoe in oracle.cpp); ids int32 [T,k];
 * r fp64 [T,k]; g, u, h fp64 [T,k,I]; gs, us fp64 [T,k,I] (sum_k |x*w1| for
 * the gate and up rows).                                                    */
int orc_qmoe(int64_t T, int64_t H, int64_t I, int E, int k, int bits1,
             int bits2, int bs, int dtype, const uint16_t* x, const float* logits,
             const uint8_t* W1, const uint16_t* s1, const uint8_t* W2,
             const uint16_t* s2, const uint16_t* b1, const uint16_t* b2,
             uint16_t* out16, double* out64, double* S,
             int32_t* ids, double* r, double* g, double* u, double* h,
             double* gs, double* us, int nthreads);

/* FC2 alone on caller-supplied fp64 activations h [T,k,I] for stage checks:
 * y fp64 [T,k,H] = h . w2[ids]^T (+ b2[ids]) and yS = sum_i |h_i * w2[n,i]|
 * (+ |b2|); b2 fp16 [E, H] or NULL.                                        */
int orc_qmoe_fc2(int64_t T, int64_t H, int64_t I, int E, int k, int bits2,
                 int bs, int dtype, const int32_t* ids, const double* h, const uint8_t* W2,
                 const uint16_t* s2, const uint16_t* b2, double* y, double* yS,
                 int nthreads);

/* ---- INT3 round-to-nearest producer quantizer [P0][OLIVE] -----------------
 * W fp32 [rows, K], K a multiple of bs.  Per group of bs consecutive k of a
 * row: amax = max |w|; the scale is amax / 3.5 with the division done in
 * fp32 and the quotient rounded once to the stored type (dtype 0: fp16,
 * 1: bf16 [P1]: FP16/BF16 scales), or the stored fp32(1 / 3.5) for an
 * all-zero group; each code is
 * q = clamp(rint(w / s) + 4, 0, 7) with w / s an fp32 division by the STORED
 * scale (stored-scale rounding) and rint rounding ties to even.
 * Outputs: B uint8 [rows, ceil(3K/8)] row-local LSB-first; scales 16-bit
 * patterns [rows, K/bs]; status uint8 [rows, K/bs]: 0 ok, 1 a weight is NaN
 * or infinite, 2 a nonzero group whose scale rounds to zero, 3 a scale
 * beyond the stored type's range.  A group with a nonzero status gets scale 0 and codes 4.
 * Returns 0 (also when a status is nonzero), negative on bad arguments.    */
int orc_rtn_int3(int64_t rows, int64_t K, int bs, int dtype, const float* W, uint8_t* B,
                 uint16_t* scales, uint8_t* status);

#ifdef __cplusplus
}
#endif
#endif
