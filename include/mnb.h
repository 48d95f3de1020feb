/*
 * mnb.h -- C ABI of the block-quantized weight-only matmul library for AMD
 * Instinct MI355X (gfx950): MatMulNBits GEMV / GEMM on packed INT4 weights and
 * a top-k routed QMoE layer with INT3 or INT4 expert projections.
 *
 * Sources (page title, then section):
 *  [PLAN]  "Qwen3 Missing-Kernel Implementation Plan" (onnx-light CPU docs),
 *          section "PR sequence": K01 defines the MatMulNBits contract (FP32 A,
 *          UINT8 packed B, FP32 scales; bits=4, block_size=32,
 *          accuracy_level=4; implicit zero points; scale indexing; padding;
 *          prepared storage that reuses constant packed weights; explicit
 *          rejection of unsupported variants without expanding the weight
 *          matrix).  K02 is the M=1 decode GEMV (including the vocabulary
 *          head), K03 the small-M/prefill GEMM on the same compressed weights
 *          with a bounded workspace.  Section "Common implementation and
 *          performance gates": unsupported variants never silently run
 *          another kernel.
 *  [P0]    onnxruntime PR "INT3 QMoE CUDA correctness baseline and Qwen
 *          experimental results", embedded body of the stacked P0/P1 PR,
 *          section "P0: Portable Format and Numerical References": row-local
 *          LSB-first UINT8 packing, checked size arithmetic, canonical
 *          padding, INT3 offset-4 decoding, RTN with stored-scale rounding.
 *  [P1]    same body, section "P1: Compatible QMoE v1 Extension": INT3 QMoE
 *          profile (quant_type int, weights_prepacked 0, activation swiglu,
 *          fused interleaved gate/up, block sizes 32/64/128, block-aligned K,
 *          FP16 activations with FP16 scales, H from the activations, I from
 *          the fused FC1 rows; finite nonnegative scales; overflow-checked
 *          byte counts; independent projection widths, (FC1, FC2) in
 *          {(3,3), (3,4), (4,3)}).  Sections "Latest Review Fixes" (N need not be
 *          aligned) and "Review Fixes and Padding Experiment Follow-up"
 *          (errors are status codes, no exceptions).
 *  [RUN]   same page, PR summary: CUDA QMoE execution with routing, fused
 *          gate/up SwiGLU, independent down projection, aggregation and
 *          bounded activation tiling, without materializing floating weights,
 *          for the width pairs (3,3), (3,4), (4,3); its results table runs
 *          the all-INT4 (4,4) layer next to (3,3).
 *  [OLIVE] same page, embedded Olive body ("Summary"): symmetric INT3 RTN
 *          with scale max|w| / 3.5, zero point 4, all-zero groups at scale
 *          1 / 3.5 and code 4; non-finite weights and unrepresentable scales
 *          reported rather than clamped.
 *  [ROUTE] pegainfer PR "feat(qwen4): component kernels extracted from the
 *          brick PRs", section "Description": fp32 softmax, top-k,
 *          renormalized (norm_topk_prob) routing weights; branch combine.
 *
 * Conventions shared by every entry point
 *  - Return value: MNB_OK (0) or a negative mnb_status.  Nothing is thrown
 *    across the ABI.  Argument, descriptor and plan checks run on the host
 *    before any launch; a failed check launches nothing and writes nothing.
 *  - Device pointers ("_dev") are caller-owned device memory on the device
 *    that was current when the plan was prepared.  The library never
 *    allocates device memory and keeps no state between calls, except the
 *    static workspace array of qmoe_forward_noalloc (one per GPU).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every compute call only enqueues work on `stream` and returns; only
 *    mnb_prepare waits (for its own upload).
 *  - Sizes are bytes (uint64_t); shapes are element counts (int64_t) and are
 *    overflow-checked.
 */
#ifndef MNB_H
#define MNB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MNB_ABI_VERSION 1

typedef enum mnb_status {
  MNB_OK = 0,
  MNB_ERR_INVALID_ARG = -1,         /* NULL pointer, bad shape or enum value   */
  MNB_ERR_UNSUPPORTED = -2,         /* valid request outside what is built     */
  MNB_ERR_SIZE_OVERFLOW = -3,       /* a byte count does not fit 64 bits      */
  MNB_ERR_CONTENT = -4,             /* malformed weight content [P1]           */
  MNB_ERR_WORKSPACE_TOO_SMALL = -5, /* ws or dst smaller than required         */
  MNB_ERR_DEVICE = -6,              /* a HIP call or kernel launch failed      */
  MNB_ERR_STALE_PLAN = -7,          /* plan not made by this library version   */
  MNB_ERR_HOST_MEMORY = -8          /* host staging allocation failed          */
} mnb_status;

enum { MNB_DTYPE_F32 = 0, MNB_DTYPE_F16 = 1, MNB_DTYPE_BF16 = 2 };

/* Row layouts of B.  BLOCKED: each row is ceil(K/bs) blocks of bs*bits/8
 * bytes, the K tail padded to a whole block [PLAN K01].  ROW_LOCAL: each row
 * is one LSB-first bit stream of ceil(K*bits/8) bytes [P0].  The two are
 * byte-identical when K is a multiple of the block size. */
enum { MNB_ROWS_BLOCKED = 0, MNB_ROWS_ROW_LOCAL = 1 };

/* Weight descriptor.  Supported profiles (anything else: UNSUPPORTED):
 *  dense MatMulNBits [PLAN K01]: bits 4, block_size 32/64/128, scale_dtype
 *    F32, row_layout BLOCKED, num_experts 1, zero points optional, any
 *    K >= 1 and N >= 1;
 *  QMoE projection [P1]: bits 3 or 4, block_size 32/64/128, scale_dtype
 *    F16 or BF16, row_layout ROW_LOCAL, num_experts >= 1, zero points implicit
 *    (2^(bits-1): 4 or 8) or explicit with every value equal to that
 *    ("all-4 explicit zero points" for INT3), K a multiple of block_size,
 *    any N >= 1 (per-expert matrix [N, K]).
 * accuracy_level must be 0..4; it is recorded, and the numerics are fixed by
 * the kernels (fp32 GEMV, fp16-input MFMA GEMM with fp32 accumulation). */
typedef struct mnb_desc {
  int32_t abi_version;     /* MNB_ABI_VERSION                               */
  int32_t bits;            /* 4 (dense); 3 or 4 (QMoE)                       */
  int32_t block_size;      /* codes per scale along K: 32, 64 or 128         */
  int32_t accuracy_level;  /* 0..4                                            */
  int64_t K;               /* reduction length (columns of the logical W)    */
  int64_t N;               /* output features (rows of W, per expert)        */
  int32_t scale_dtype;     /* MNB_DTYPE_F32 (dense); F16 or BF16 (QMoE)      */
  int32_t has_zero_points; /* 0 = implicit 2^(bits-1), 1 = explicit          */
  int32_t row_layout;      /* MNB_ROWS_BLOCKED / MNB_ROWS_ROW_LOCAL          */
  int32_t num_experts;     /* 1 for dense; E for a stacked QMoE projection   */
} mnb_desc;

/* Prepared constant weights [PLAN K01 "prepared storage", K02 "repeated
 * calls do not repack"].  Caller-owned POD filled by mnb_prepare; read-only
 * afterwards; valid while the dst buffer given to mnb_prepare lives; may be
 * used concurrently from several streams. */
typedef struct mnb_plan {
  mnb_desc desc;
  uint32_t magic;          /* identifies a plan made by this library        */
  uint32_t layout_version; /* version of the private prepacked layout       */
  int64_t n_blocks;        /* ceil(K / block_size)                          */
  int64_t row_bytes;       /* contract bytes of one B row                   */
  uint64_t codes_bytes;    /* prepacked codes                               */
  uint64_t scales_bytes;   /* prepacked scales                              */
  uint64_t zeros_bytes;    /* prepacked zero points (0 if implicit)         */
  uint64_t total_bytes;    /* bytes of dst used (<= dst_bytes)              */
  void* codes;             /* device pointers into dst                      */
  void* scales;
  void* zeros;
  int32_t device;          /* HIP device ordinal the plan lives on          */
  int32_t reserved;
} mnb_plan;

/* Human-readable name of a status code (static storage, never NULL). */
const char* mnb_status_string(int32_t status);

/* Bytes of device memory mnb_prepare needs for `desc`.  The prepacked layout
 * holds as many code and scale bytes as the contract's B and scales; explicit
 * zero points take 4 bytes per (group of 8 rows, block), which is no more
 * than the contract's N * ceil(nb/2) when N is a multiple of 8; on top come
 * at most 768 bytes of section alignment. */
int32_t mnb_prepacked_size(const mnb_desc* desc, uint64_t* bytes);

/* One-time preparation of constant weights [PLAN K01]:
 *  1. checks the descriptor and computes every byte count with overflow
 *     checks [P0];
 *  2. validates content: for QMoE projections, scales must be finite and
 *     >= 0 and the pad bits after K*bits in each row must be zero [P1];
 *     dense INT4 content is not value-checked (non-finite scales propagate
 *     to the outputs);
 *  3. repacks on the host into the private layout and uploads it to dst_dev
 *     with an asynchronous copy on `stream`, then waits for that stream.
 * Host inputs (read only; any alignment):
 *  B_host           uint8, [E*N, nb, bs*bits/8] (BLOCKED) or
 *                   [E*N, ceil(K*bits/8)] (ROW_LOCAL), E = num_experts;
 *  scales_host      fp32, fp16 or bf16 (per scale_dtype), [E*N, nb], index
 *                   n*nb + b;
 *  zero_points_host NULL when has_zero_points == 0, else uint8
 *                   dense: [N, ceil(nb/2)]: block b of row n in byte b/2,
 *                   low nibble for even b;  QMoE: packed per-row block zero
 *                   points [E*N, ceil(nb*bits/8)], row-local LSB-first like
 *                   the codes, every one 2^(bits-1) with canonical padding
 *                   (else CONTENT); they are validated and then implied.
 * dst_dev must hold mnb_prepacked_size(desc) bytes and be 256-byte aligned.
 * On success *plan describes the prepared weights; on failure *plan is
 * zeroed.  Errors: INVALID_ARG, UNSUPPORTED, SIZE_OVERFLOW, CONTENT,
 * WORKSPACE_TOO_SMALL (dst_bytes), HOST_MEMORY, DEVICE. */
int32_t mnb_prepare(const mnb_desc* desc, const uint8_t* B_host,
                    const void* scales_host, const uint8_t* zero_points_host,
                    void* dst_dev, uint64_t dst_bytes, void* stream,
                    mnb_plan* plan);

/* Workspace bytes mnb_gemv needs for this plan (grows with K only). */
int32_t mnb_gemv_workspace_size(const mnb_plan* plan, uint64_t* bytes);

/* M = 1 decode GEMV [PLAN K02], dense INT4 plans only:
 *   Y[n] = sum_{k<K} A[k] * (q[n,k] - z[n,k/bs]) * s[n,k/bs],  n < N.
 * A_dev fp32 [K] (contiguous); Y_dev fp32 [N] (contiguous, written once per
 * element, nothing else is touched); ws_dev >= mnb_gemv_workspace_size bytes,
 * 256-byte aligned, scratch for the call (contents need not be initialised
 * and are clobbered).  Deterministic: the same inputs give the same bits.
 * Errors: INVALID_ARG, UNSUPPORTED (non-dense plan), STALE_PLAN,
 * WORKSPACE_TOO_SMALL, DEVICE. */
int32_t mnb_gemv(const mnb_plan* plan, const float* A_dev, float* Y_dev,
                 void* ws_dev, uint64_t ws_bytes, void* stream);

/* Several M = 1 GEMVs [PLAN K02] sharing one activation vector (e.g. the gate
 * and up projections of a SwiGLU MLP, which read the same input):
 *   for i < count:  Y_dev[i] = mnb_gemv(plans[i], A_dev),
 * bit-identical to the separate calls.  All plans must be dense INT4 with the
 * same K; when they also share the block size and zero-point kind and each
 * takes the short-row fp32 path (N <= 32768, K <= 8192), one kernel launch
 * does them all, otherwise they run one after another on the stream.
 * plans: host array of count plan pointers; Y_dev: host array of count device
 * pointers (fp32 [N_i], contiguous); count in [1, 4]; ws_dev as for mnb_gemv
 * with the largest workspace any of the plans needs (shared, used by one GEMV
 * at a time).  Errors: INVALID_ARG (count out of range, null pointers,
 * different K), otherwise as for mnb_gemv. */
int32_t mnb_gemv_multi(const mnb_plan* const* plans, int32_t count, const float* A_dev,
                       float* const* Y_dev, void* ws_dev, uint64_t ws_bytes, void* stream);

/* Workspace bytes mnb_gemm needs for this plan and M (may be 0). */
int32_t mnb_gemm_workspace_size(const mnb_plan* plan, int64_t M, uint64_t* bytes);

/* Small-M / prefill GEMM on the same compressed weights [PLAN K03]:
 *   Y[m,n] = sum_{k<K} A[m,k] * (q[n,k] - z) * s,  m < M, n < N.
 * A_dev fp32 [M, K] row-major (lda = K); Y_dev fp32 [M, N] row-major.  A and
 * the dequantized weights are rounded to fp16 at the matrix-core inputs and
 * accumulated in fp32.  Valid range, as for any fp16-input product: |A| and
 * |(q - z) * s| must stay below 65520 (larger values round to +-Inf, and the
 * outputs they reach become Inf or NaN), and weights below 2^-14 in magnitude
 * become fp16 subnormals with absolute error up to 2^-25 each, so the error
 * bound 4e-3 * sum|a w| holds only for scales with |(q - z) * s| >= 2^-14 or
 * zero (the GEMV, in fp32, has neither limit).  M = 0 is a no-op.  ws_dev as
 * for mnb_gemv (may be NULL when the required size is 0).  Errors as for
 * mnb_gemv. */
int32_t mnb_gemm(const mnb_plan* plan, int64_t M, const float* A_dev,
                 float* Y_dev, void* ws_dev, uint64_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Top-k routed QMoE layer with INT3 or INT4 projections [P1][RUN][ROUTE].
 */
enum { QMOE_ACT_SWIGLU = 1 };
enum { QMOE_GATE_UP_INTERLEAVED = 1 };
enum { QMOE_QUANT_INT = 0 };

typedef struct qmoe_desc {
  int32_t abi_version;               /* MNB_ABI_VERSION                      */
  int32_t top_k;                     /* 1..num_experts (8 for the configs);
                                        more than 16: UNSUPPORTED            */
  int32_t normalize_routing_weights; /* must be 1 (renormalized top-k)       */
  int32_t activation;                /* must be QMOE_ACT_SWIGLU              */
  int32_t gate_up;                   /* must be QMOE_GATE_UP_INTERLEAVED     */
  int32_t weights_prepacked;         /* must be 0                            */
  int32_t quant_type;                /* must be QMOE_QUANT_INT               */
  int32_t reserved;                  /* must be 0                            */
} qmoe_desc;

/* Limits of the built kernels (beyond them: UNSUPPORTED, from both calls
 * below): num_experts <= 1024, top_k <= 16, and each expert's packed codes
 * below 2 GiB.  Workspace bytes for qmoe_forward with T tokens. */
int32_t qmoe_workspace_size(const mnb_plan* fc1, const mnb_plan* fc2,
                            const qmoe_desc* q, int64_t T, uint64_t* bytes);

/* One QMoE layer on T tokens.
 *  fc1: QMoE plan with N = 2I, K = H (rows 2i = gate_i, 2i+1 = up_i);
 *  fc2: QMoE plan with N = H, K = I; both with the same num_experts E and
 *       block size; each projection has its own width (3 or 4 bits), so the
 *       pairs (3,3), (3,4), (4,3) and (4,4) all run.
 *  x_dev      [T, H] activations, 16-byte aligned, in the plans' 16-bit type:
 *             fp16 for F16 plans, bf16 for BF16 plans ([P1]: matching
 *             FP16/BF16 activation and scale types; both plans must share
 *             scale_dtype, else UNSUPPORTED);
 *  logits_dev fp32 [T, E] router logits;
 *  out_dev    [T, H] in the same 16-bit type, 8-byte aligned (misaligned x or
 *             out: INVALID_ARG).
 * Computes, per token: top_k experts by logit (ties: lower index), weights
 * r_j = softmax over the selected logits (= fp32 softmax over all E then
 * renormalization); weights dequantize as (q - 2^(bits-1)) * s;
 * weights enter the matrix cores rounded once to the layer's type,
 * h = silu(x.W1g^T) * (x.W1u^T) rounded to that type;
 * out = fp16(sum_j r_j * h_j.W2^T) summed in rank order.
 * T = 0 is a no-op.  No host synchronisation (graph-capturable).
 * Errors: INVALID_ARG, UNSUPPORTED, STALE_PLAN, WORKSPACE_TOO_SMALL, DEVICE. */
int32_t qmoe_forward(const mnb_plan* fc1, const mnb_plan* fc2,
                     const qmoe_desc* q, int64_t T, const uint16_t* x_dev,
                     const float* logits_dev, uint16_t* out_dev, void* ws_dev,
                     uint64_t ws_bytes, void* stream);

/* qmoe_forward with the optional projection biases [P1] ("optional
 * biases"):
 *  fc1_bias_dev [E, 2I] in the layer's 16-bit type (row order of FC1: gate_i at 2i, up_i at
 *               2i + 1), added to g and u before SwiGLU; NULL = none;
 *  fc2_bias_dev [E, H] in that type, added to each expert's FC2 output
 *               before its routing weight:
 *               out = round(sum_j r_j (h_j.W2^T + b2[e_j]));
 *               NULL = none.
 * Both 2-byte aligned (else INVALID_ARG); read only.  Everything else as for
 * qmoe_forward, which is this call with two NULL biases. */
int32_t qmoe_forward_biased(const mnb_plan* fc1, const mnb_plan* fc2,
                            const qmoe_desc* q, int64_t T,
                            const uint16_t* x_dev, const float* logits_dev,
                            const uint16_t* fc1_bias_dev,
                            const uint16_t* fc2_bias_dev, uint16_t* out_dev,
                            void* ws_dev, uint64_t ws_bytes, void* stream);

/* qmoe_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The workspace is a static device array of
 * MNB_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, created when the
 * library's code is loaded on that GPU and held until the process ends; its
 * address is looked up on the first call on each device.  No call allocates.
 * Every call on a GPU shares that GPU's array and leaves its contents behind:
 * calls that overlap on one GPU (other streams, other host threads) race and
 * must be serialized by the caller.  Requests whose qmoe_workspace_size
 * exceeds MNB_NOALLOC_SCRATCH_BYTES return WORKSPACE_TOO_SMALL before any
 * device work (the workspace grows with min(T, 512) * top_k * (4H + 2I) bytes
 * plus small tables; the 128-expert, H = 2048, I = 768, top-8 layer needs
 * about 40 MB).  Arguments, results and all other errors as for qmoe_forward. */
#define MNB_NOALLOC_SCRATCH_BYTES (64ull << 20)
int32_t qmoe_forward_noalloc(const mnb_plan* fc1, const mnb_plan* fc2,
                             const qmoe_desc* q, int64_t T, const uint16_t* x_dev,
                             const float* logits_dev, uint16_t* out_dev, void* stream);

/* ---------------------------------------------------------------------------
 * Producer-side INT3 round-to-nearest quantizer [P0][OLIVE]: fp32 weights to
 * the QMoE projection contract (codes and scales ready for mnb_prepare with
 * bits 3, ROW_LOCAL and F16 or BF16 scales [P1]).  Per group of block_size
 * consecutive k of a row: amax = max |w|; stored scale s = amax / 3.5 (fp32
 * quotient, rounded once to the scale type), or the stored fp32(1 / 3.5) for
 * an all-zero group; codes
 * q = clamp(rint(w / s) + 4, 0, 7) divided by the STORED scale in fp32,
 * ties to even (stored-scale rounding).  Decoding is (q - 4) * s.
 *  W_dev      fp32 [rows, K] row-major, 16-byte aligned (rows = E * N for a
 *             stacked projection);
 *  B_dev      uint8 [rows, 3K/8] out, row-local LSB-first 3-bit codes, 4-byte
 *             aligned;
 *  scale_dtype MNB_DTYPE_F16 or MNB_DTYPE_BF16 (F32: UNSUPPORTED);
 *  scales_dev [rows, K/block_size] out in that type, 2-byte aligned;
 *  status_dev uint8 [rows, K/block_size] out: 0 ok, 1 a weight is NaN or
 *             infinite, 2 a nonzero group whose scale rounds to zero, 3 a
 *             scale beyond the type's range.  A group with a nonzero status is
 *             written with scale 0 and codes 4 and must be treated as a
 *             rejected tensor [OLIVE: fail fast, never clamp a scale];
 *             nonzero subnormal scales are status 0.
 * block_size 32, 64 or 128; K a multiple of it.  Asynchronous on `stream`:
 * the caller reads status_dev after the stream has finished.  rows = 0 is a
 * no-op.  Deterministic.  Errors: INVALID_ARG (NULL or misaligned pointers,
 * negative sizes, unknown scale type), UNSUPPORTED (block size, K not block
 * aligned, F32 scales),
 * SIZE_OVERFLOW, DEVICE. */
int32_t mnb_quantize_int3_rtn(const float* W_dev, int64_t rows, int64_t K,
                              int32_t block_size, int32_t scale_dtype,
                              uint8_t* B_dev, uint16_t* scales_dev,
                              uint8_t* status_dev, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MNB_H */
