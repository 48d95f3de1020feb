// Top-k routed QMoE layer with INT3 or INT4 expert projections for gfx950.
//
// Sources: onnxruntime PR "INT3 QMoE CUDA correctness baseline and Qwen
// experimental results" (PR summary: routing, fused gate/up SwiGLU, an
// independent down projection and aggregation, with bounded activation tiling
// and no floating expert weights; embedded P0/P1 body, section "P0" for the
// row-local LSB-first 3-bit format and "P1" for the fused interleaved gate/up
// and swiglu profile, the (3,4) / (4,3) width pairs, FP16/BF16 types and the
// optional biases; embedded Olive body for the (code - 4) * scale decode)
// and pegainfer PR "feat(qwen4): component kernels extracted from the brick
// PRs" (fp32 softmax routing, top-k, renormalized weights, branch combine).
//
// Pipeline per tile of at most kTokTile tokens (all on one stream, no host
// synchronisation):
//  1. route:   one wave per token; top-k by logit (ties: lower expert), then
//              r_j = exp(l_j - l_max) / sum_sel exp(l_i - l_max) in fp32, which
//              equals an fp32 softmax over all experts renormalized over the
//              selected ones.
//  2. group:   one workgroup; per-expert counts, offsets, a permutation of the
//              T*k slots into expert-grouped order, and the list of (expert,
//              row-tile) work items.
//  3. fc1:     per work item, G = X_e W1_e^T on the matrix cores (gathered
//              token rows in LDS; INT3 / INT4 weights dequantized in
//              registers as fp16((q - z) * s), z = 4 / 8, once per item);
//              epilogue
//              h_i = silu(g_i) * u_i from the interleaved gate/up columns,
//              rounded to fp16.
//  4. fc2:     per work item, Y_e = h_e W2_e^T; epilogue multiplies by the
//              slot's routing weight and writes an fp32 slot row.
//  5. combine: out[t] = fp16(sum_j slot[t, j]) in rank order (deterministic).

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <type_traits>

#include "kernels.h"

namespace mnb {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x3 __attribute__((ext_vector_type(3), aligned(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTokTile = 512;   // tokens per pass (bounds the workspace)
constexpr int kDecodeSlots = 32; // T * k up to which the per-slot decode path runs
constexpr int kFusedRouteSlots = 8;  // T * k up to which FC1 also routes (one launch less)
constexpr int kMaxE = 1024;     // experts supported by the grouping kernel
constexpr int kMaxTopK = 16;    // experts per token supported by the routing kernels
constexpr int kGroupThreads = 1024;

// ---------------------------------------------------------------------------
// 1. routing
// ---------------------------------------------------------------------------
// Order-preserving key of a logit: larger logit -> larger unsigned key; NaN
// ranks with -inf; key 0 marks an expert that is taken or absent.
__device__ __forceinline__ uint32_t logit_key(float x) {
  if (x != x) x = -INFINITY;
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_logit(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Wave-wide reductions with DPP moves (no LDS round trips): after the row
// steps every lane of a 16-lane row holds the row result, the two broadcasts
// fold the rows into lane 63, which is read back as a uniform value.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v) {
  // the moved-in value defaults to the identity of the operation, so each
  // step compiles to one v_max_u32_dpp / v_min_u32_dpp
  constexpr int id = MAX ? 0 : -1;
  auto op = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// One wave per token: k rounds of "largest logit, lower expert on ties" over
// the E <= 1024 experts (lane l holds experts 64i + l), then
// r_j = exp(l_j - l_max) / sum_sel exp(l_i - l_max) in fp32, which equals an
// fp32 softmax over all experts renormalized over the selected ones.
// (kPer: experts per lane, E <= 64 kPer; instantiated for 2, 4 and 16)
// Top-k of one token's E logits by one wave (lane l holds experts 64i + l);
// lane 0 writes ids[j] and the renormalized weights wts[j], j < k <= 16.
// (kPer: experts per lane, E <= 64 kPer; instantiated for 2, 4 and 16)
template <int kPer>
__device__ __forceinline__ void route_token(const float* __restrict__ l, int E, int k, int lane,
                                            int32_t* ids, float* wts) {
  const int nper = (E + 63) >> 6;
  uint32_t key[kPer];
  // all logit loads first (clamped to a valid expert, then masked): a
  // guarded load per slot compiled to a branch and a full wait each
  float lv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = i * 64 + lane;
    lv[i] = l[e < E ? e : E - 1];
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = i * 64 + lane;
    key[i] = (i < nper && e < E) ? logit_key(lv[i]) : 0u;
  }
  // lane j keeps the j-th selection (no register array indexed by the round,
  // which compiled to dozens of register moves per round)
  float lmax = 0.0f, den = 0.0f, my_v = 0.0f;
  int my_i = 0;
  for (int j = 0; j < k; ++j) {  // k <= 16 (checked by the launcher)
    // this lane's best: largest key, lowest i on ties (= lowest expert)
    uint32_t bk = 0;
    int bi = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (i < nper && key[i] > bk) {
        bk = key[i];
        bi = i;
      }
    const uint32_t mk = wave_reduce_u32<true>(bk);
    // lowest expert index among the lanes holding the maximum
    const uint32_t cand = (bk == mk) ? (uint32_t)(bi * 64 + lane) : 0xFFFFFFFFu;
    const int win = (int)wave_reduce_u32<false>(cand);
    if ((win & 63) == lane) {
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (i == (win >> 6)) key[i] = 0u;
    }
    const float v = key_logit(mk);
    if (j == 0) lmax = v;
    const float ex = expf(v - lmax);
    den += ex;
    if (lane == j) {
      my_v = ex;
      my_i = win;
    }
  }
  if (lane < k) {
    ids[lane] = my_i;
    wts[lane] = my_v / den;
  }
}

template <int kPer>
__global__ void __launch_bounds__(256) qmoe_route(const float* __restrict__ logits, int64_t T,
                                                  int E, int k, int32_t* __restrict__ ids,
                                                  float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;  // whole waves leave together
  route_token<kPer>(logits + t * E, E, k, lane, ids + t * k, wts + t * k);
}

// ---------------------------------------------------------------------------
// 2. grouping: counts, offsets, permutation, work items
// ---------------------------------------------------------------------------
__device__ __forceinline__ int clamp_id(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

struct GroupOut {
  int32_t* counts;   // [E]
  int32_t* offsets;  // [E + 1]
  int32_t* perm;     // [T*k] grouped position -> slot (t*k + j)
  int32_t* inv;      // [T*k] slot -> grouped position
  int32_t* items;    // [max_items][2] (expert, first row)
  int32_t* nitems;   // [1]
};

// One workgroup of 16 waves; every step is parallel:
//  counts:   LDS atomics, also per wave over a contiguous range of slots;
//  offsets:  block-wide exclusive scans over the experts of the counts and of
//            the work items per expert (ceil(count / bm)); each expert's
//            thread writes its own work items;
//  ranks:    the base of wave w in expert e is offsets[e] plus the counts of
//            waves 0 .. w-1; a wave walks its slots in order, 64 at a time,
//            and takes each slot's position with an LDS fetch-and-add on its
//            expert's base.  Slots of different waves are ordered by wave;
//            within a wave the order of the lanes' atomics is the hardware's.
//            No result depends on this order: each token's rows go through
//            the same per-row arithmetic wherever they sit in a work item,
//            and the combine sums a token's ranks in rank order.
__global__ void __launch_bounds__(kGroupThreads) qmoe_group(const int32_t* __restrict__ ids,
                                                            int64_t T, int k, int E, int64_t max_items,
                                                            int bm, GroupOut o) {
  extern __shared__ __align__(16) int32_t gsm[];
  constexpr int kWaves = kGroupThreads / 64;
  int32_t* cnt = gsm;              // [E]
  int32_t* off = cnt + E;          // [E] exclusive offsets (scanned in place)
  int32_t* ioff = off + E;         // [E] exclusive item offsets
  int32_t* tmp = ioff + E;         // [2 E] exclusive offsets (first E)
  int32_t* hist = tmp + 2 * E;     // [kWaves][E]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t S = T * k;

  for (int e = tid; e < E; e += kGroupThreads) cnt[e] = 0;
  for (int i = tid; i < kWaves * E; i += kGroupThreads) hist[i] = 0;
  __syncthreads();
  const int64_t per = (S + kWaves - 1) / kWaves;
  const int64_t s_lo = wave * per, s_hi = (s_lo + per) < S ? (s_lo + per) : S;
  for (int64_t sl = s_lo + lane; sl < s_hi; sl += 64) {
    const int e = clamp_id(ids[sl], E);
    atomicAdd(&hist[wave * E + e], 1);
    atomicAdd(&cnt[e], 1);
  }
  __syncthreads();

  // inclusive scans of counts and of items per expert, by wave 0: lane l
  // sums experts [P l, P l + P) in order, the lane totals are scanned with
  // DPP row shifts and row broadcasts (no LDS round trips, one barrier)
  if (wave == 0) {
    const int P = (E + 63) >> 6;  // <= kMaxE / 64
    int32_t sc = 0, si = 0;
    for (int j = 0; j < P; ++j) {
      const int e = P * lane + j;
      if (e < E) {
        sc += cnt[e];
        si += (cnt[e] + bm - 1) / bm;
      }
    }
    int32_t ic = sc, ii = si;  // inclusive over lanes
    ic += __builtin_amdgcn_update_dpp(0, ic, 0x111, 0xF, 0xF, true);  // row_shr:1
    ii += __builtin_amdgcn_update_dpp(0, ii, 0x111, 0xF, 0xF, true);
    ic += __builtin_amdgcn_update_dpp(0, ic, 0x112, 0xF, 0xF, true);  // row_shr:2
    ii += __builtin_amdgcn_update_dpp(0, ii, 0x112, 0xF, 0xF, true);
    ic += __builtin_amdgcn_update_dpp(0, ic, 0x114, 0xF, 0xF, true);  // row_shr:4
    ii += __builtin_amdgcn_update_dpp(0, ii, 0x114, 0xF, 0xF, true);
    ic += __builtin_amdgcn_update_dpp(0, ic, 0x118, 0xF, 0xF, true);  // row_shr:8
    ii += __builtin_amdgcn_update_dpp(0, ii, 0x118, 0xF, 0xF, true);
    ic += __builtin_amdgcn_update_dpp(0, ic, 0x142, 0xA, 0xF, false);  // row_bcast:15
    ii += __builtin_amdgcn_update_dpp(0, ii, 0x142, 0xA, 0xF, false);
    ic += __builtin_amdgcn_update_dpp(0, ic, 0x143, 0xC, 0xF, false);  // row_bcast:31
    ii += __builtin_amdgcn_update_dpp(0, ii, 0x143, 0xC, 0xF, false);
    int32_t rc = ic - sc, ri = ii - si;  // exclusive: totals of the earlier lanes
    for (int j = 0; j < P; ++j) {
      const int e = P * lane + j;
      if (e < E) {
        rc += cnt[e];
        ri += (cnt[e] + bm - 1) / bm;
        off[e] = rc;
        ioff[e] = ri;
      }
    }
  }
  __syncthreads();
  // to exclusive, outputs, work items
  for (int e = tid; e < E; e += kGroupThreads) {
    const int32_t c = cnt[e];
    const int32_t ex = off[e] - c;
    const int32_t iex = ioff[e] - (c + bm - 1) / bm;
    o.counts[e] = c;
    o.offsets[e] = ex;
    if (e == E - 1) {
      o.offsets[E] = off[e];
      *o.nitems = (int32_t)(ioff[e] < max_items ? ioff[e] : max_items);
    }
    for (int32_t m0 = 0, it = iex; m0 < c && it < max_items; m0 += bm, ++it) {
      o.items[2 * it] = e;
      o.items[2 * it + 1] = m0;
    }
    tmp[e] = ex;  // keep the exclusive offset for the bases below
  }
  __syncthreads();
  // per-wave bases: offsets[e] + counts of the earlier waves
  for (int e = tid; e < E; e += kGroupThreads) {
    int32_t run = tmp[e];
    for (int w = 0; w < kWaves; ++w) {
      const int32_t v = hist[w * E + e];
      hist[w * E + e] = run;
      run += v;
    }
  }
  __syncthreads();
  int32_t* base = hist + wave * E;
  for (int64_t sl = s_lo + lane; sl < s_hi; sl += 64) {
    const int e = clamp_id(ids[sl], E);
    const int32_t pos = atomicAdd(&base[e], 1);
    o.perm[pos] = (int32_t)sl;
    o.inv[sl] = pos;
  }
}

// ---------------------------------------------------------------------------
// 3./4. grouped INT3 / INT4 GEMM (FC1 with SwiGLU epilogue, FC2 with route
// weights); each projection takes its own width (pairs (3,3), (3,4), (4,3)
// and (4,4))
// ---------------------------------------------------------------------------
//
// A workgroup takes one work item (expert e, up to BM of its tokens) and 64
// weight rows; wave w owns rows [16w, 16w + 16) and computes them for all of
// the item's tokens with v_mfma_f32_16x16x32_f16 (C tiles of 16 tokens x 16
// rows).  The weights never go through LDS: lane (n, g) = (lane & 15,
// lane >> 4) loads the 12-byte (INT3) or 16-byte (INT4) group g (32 codes,
// k = 32g .. 32g + 31 of a 128-wide K chunk) of its row straight into
// registers and dequantizes it once
// for every token of the item.  K order inside an MFMA is free when both
// operands share it: MFMA t of a chunk takes k = 32g + 8t + [0, 8) in lane
// group g, on both sides.  The token rows of the chunk (gathered by route for
// FC1, contiguous grouped rows for FC2) are staged in LDS (pitch 136 halves:
// the 16 rows of an operand read fall on distinct banks), double-buffered.
//
// Dequantization of a pair of codes from the private layout: one shift and one
// and-or give the fp16 values 1024 + q in both halves, v_pk_add_f16 makes the
// exact q - z, v_pk_mul_f16 by the fp16 scale rounds once: fp16((q - z) * s),
// the same value as the exact fp32 product rounded to fp16.

typedef _Float16 half2t __attribute__((ext_vector_type(2)));

// (a & m) | (b & ~m): one v_bfi_b32
__device__ __forceinline__ uint32_t bfi(uint32_t m, uint32_t a, uint32_t b) { return (a & m) | (b & ~m); }

// A group of 32 codes in the private layout: 4 * BITS bytes (three words
// for INT3, four for INT4).
template <int BITS> struct Group;
template <> struct Group<3> { typedef u32x3 W; };
template <> struct Group<4> { typedef u32x4 W; };

// 16-bit activation / scale / output type of a layer: IEEE fp16 (BF = false)
// or bfloat16 (BF = true); the INT3 QMoE profile takes either, with the
// activation and scale types matching.  kMagic is the base B (1024 or 128)
// in both 16-bit halves: B + c is exact for every code c in either format.
template <bool BF> struct Dt;
template <> struct Dt<false> {
  static constexpr uint32_t kMagic = 0x64006400u;
  static constexpr float kBase = 1024.0f;
  __device__ static float to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
  __device__ static uint16_t from_f32(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }
};
template <> struct Dt<true> {
  static constexpr uint32_t kMagic = 0x43004300u;
  static constexpr float kBase = 128.0f;
  __device__ static float to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
  __device__ static uint16_t from_f32(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }
};

// fp16 bias that turns 1024 + q into the exact q - z, z = 2^(BITS-1)
template <int BITS>
__device__ __forceinline__ half2t zero_bias() {
  constexpr float b = -(Dt<false>::kBase + (float)(1 << (BITS - 1)));
  return half2t{(_Float16)b, (_Float16)b};
}

// the two 16-bit halves of a bfloat16 pair word as fp32 (exact)
__device__ __forceinline__ float bf_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf_hi(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t bf_pack(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)lo, (__bf16)hi});  // v_cvt_pk_bf16_f32, RNE
}

// v_mfma_f32_16x16x32 on fp16 or bfloat16 operands held as raw words
template <bool BF>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (BF)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                  __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

// The 16 code pairs (c[2i], c[2i+1]) of a group as B + c in the two 16-bit
// halves of p[i] (B = 1024 in fp16, 128 in bfloat16): the pattern of B + c is
// that of B with c in its low mantissa bits, so each pair is one v_bfi_b32
// into magic (B in both halves, kept in a register the compiler cannot fold,
// so that the insert stays a single v_bfi_b32).  Words are copied into
// scalars before use.
__device__ __forceinline__ void raw_pairs(const u32x3 w, uint32_t magic, uint32_t (&p)[16]) {
#pragma unroll
  for (int m = 0; m < 3; ++m) {
    const uint32_t x = m == 0 ? w.x : (m == 1 ? w.y : w.z);
#pragma unroll
    for (int q = 0; q < 5; ++q) p[5 * m + q] = bfi(0x00070007u, x >> (3 * q), magic);
  }
  p[15] = bfi(0x00010001u, w.x >> 15, bfi(0x00020002u, w.y >> 14, bfi(0x00040004u, w.z >> 13, magic)));
}
__device__ __forceinline__ void raw_pairs(const u32x4 w, uint32_t magic, uint32_t (&p)[16]) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint32_t x = m == 0 ? w.x : (m == 1 ? w.y : (m == 2 ? w.z : w.w));
#pragma unroll
    for (int q = 0; q < 4; ++q) p[4 * m + q] = bfi(0x000F000Fu, x >> (4 * q), magic);
  }
}

// the 32 codes of one group as four MFMA operands (8 consecutive k each),
// each weight rounded once, fp16((q - z) * s) or bf16((q - z) * s):
// fp16: v_pk_add_f16 makes the exact q - z, v_pk_mul_f16 by the scale rounds;
// bf16: (B + q) s - (B + z) s in one fp32 fma is exact, v_cvt_pk_bf16_f32
// rounds.
template <int BITS, bool BF>
__device__ __forceinline__ void dequant_group(const typename Group<BITS>::W w, uint16_t sbits,
                                              uint32_t magic, u32x4 (&out)[4]) {
  uint32_t p[16];
  raw_pairs(w, magic, p);
  if constexpr (BF) {
    const float s = Dt<true>::to_f32(sbits);
    const float nb = -(Dt<true>::kBase + (float)(1 << (BITS - 1))) * s;  // exact
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = bf_pack(fmaf(bf_lo(p[i]), s, nb), fmaf(bf_hi(p[i]), s, nb));
  } else {
    const _Float16 s = __builtin_bit_cast(_Float16, sbits);
    const half2t s2 = half2t{s, s}, zb = zero_bias<BITS>();
#pragma unroll
    for (int i = 0; i < 16; ++i)
      p[i] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(half2t, p[i]) + zb) * s2);
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) out[t] = u32x4{p[4 * t], p[4 * t + 1], p[4 * t + 2], p[4 * t + 3]};
}

template <bool BF>
__device__ __forceinline__ uint32_t opaque_magic() {
  uint32_t m = Dt<BF>::kMagic;
  asm volatile("" : "+v"(m));
  return m;
}

// Byte offset, within one expert's codes, of 32-code group G of row n in the
// tile-major layout with GB = 4 BITS byte groups: rows in tiles of 16 (the
// last may hold fewer), each tile as K chunks of 4 groups (the last may hold
// fewer), each chunk row by row; a full tile's chunk is 16 x 4 GB contiguous
// bytes.
template <int BITS>
__device__ __forceinline__ uint32_t moe_goff(int N, int K, int n, int G) {
  constexpr int GB = 4 * BITS;
  const int ng = K >> 5, rt = n >> 4, r = n & 15;
  const int rcnt = min(16, N - 16 * rt);
  const int c = G >> 2, gg = G & 3;
  const int gic = min(4, ng - 4 * c);
  return (uint32_t)(16 * rt * ng * GB + rcnt * 4 * GB * c + r * gic * GB + gg * GB);
}

struct MoeGemmArgs {
  const uint8_t* codes;    // [E][N][row_bytes], pair-interleaved groups
  const uint16_t* scales;  // [E][N][K/bs], fp16 or bf16
  const void* act;         // FC1: x [T][K]; FC2: h [T*k][K] (grouped order); fp16 or bf16
  int64_t N, K, row_bytes, nblk, bs;
  int top_k, E;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* items;
  const int32_t* nitems;
  const float* wts;        // FC2: routing weights per slot
  uint16_t* h_out;         // FC1 output [T*k][N/2] (grouped order), fp16 or bf16
  float* slot_out;         // FC2 output [T*k][N] (slot order)
  const uint16_t* bias;    // optional [E][N] projection bias (nullptr: none)
};

constexpr int kQBN = 64;         // weight rows per workgroup
constexpr int kQBK = 128;        // K per chunk
constexpr int kQPitch = kQBK + 8;
// 64-row weight tiles per workgroup: with 48- and 64-token tiles 2 (their
// accumulators would otherwise cost occupancy; 48-token tiles measured at 512
// tokens with three: INT3 unchanged, INT4 13% slower; with four: 5% slower);
// with 32-token tiles 2 for
// INT3 and 4 for INT4 (measured at 128 tokens against four tiles: INT3
// 95.6 -> 92.9 us and bf16 113.7 -> 107.9 with two; INT4 with two 103.4 us,
// with four 98.3, so INT4 keeps four)
template <int BM, int BITS>
constexpr int ntg_of() { return BM == 32 ? (BITS == 3 ? 2 : 4) : 2; }
int ntg_for(int bm, int bits) {
  if (bm == 32) return bits == 3 ? ntg_of<32, 3>() : ntg_of<32, 4>();
  return bits == 3 ? ntg_of<64, 3>() : ntg_of<64, 4>();
}

template <bool FC1, int BM, int BITS, bool BF>
__global__ void __launch_bounds__(256) qmoe_gemm(MoeGemmArgs g, int64_t groups_n, int64_t tiles_n) {
  constexpr uint32_t GB = 4 * BITS;    // bytes per 32-code group
  constexpr int kNTG = ntg_of<BM, BITS>();
  constexpr int TM = BM / 16;          // 16-token MFMA tiles
  constexpr int AP = BM * 16 / 256;    // 16-byte activation chunks per thread and chunk
  __shared__ __align__(16) _Float16 As[2][BM * kQPitch];
  __shared__ int32_t arow[BM];  // activation row of each tile row (-1: none)

  // work unit: item (expert, first token) x a group of kNTG 64-row weight tiles,
  // walked as one sequence of (tile, K chunk) steps.  Workgroups go to the 8
  // XCDs round-robin by index; all weight-tile groups of an item run on one XCD
  // (XCD b % 8 takes items 8 q + b % 8), so its activation rows come from HBM
  // into that XCD's L2 once.  The grid covers the item count rounded up to 8.
  const int bj = (int)(blockIdx.x >> 3);
  const int64_t item = (int64_t)(bj / groups_n) * 8 + (blockIdx.x & 7);
  const int nt0 = (int)(bj % groups_n) * kNTG;
  if (item >= *g.nitems) return;  // uniform for the workgroup
  const int e = g.items[2 * item];
  const int m0 = g.items[2 * item + 1];
  const int rows = min(BM, g.counts[e] - m0);
  const int vt = (rows + 15) >> 4;       // valid token tiles
  const int64_t seg0 = g.offsets[e] + m0;  // grouped position of tile row 0
  const int ntc = (int)(tiles_n - nt0 < kNTG ? tiles_n - nt0 : kNTG);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int i = tid; i < BM; i += 256) {
    int32_t r = -1;
    if (i < rows) r = FC1 ? g.perm[seg0 + i] / g.top_k : (int32_t)(seg0 + i);
    arow[i] = r;
  }
  __syncthreads();

  // activation staging: thread -> chunk (tid & 15) of rows (tid >> 4) + 16 j;
  // rows without a token read row 0 of the item instead (their results are
  // never stored: an MFMA output row depends on its own A row only)
  const int a_c = (tid & 15) * 8, a_r0 = tid >> 4;
  const _Float16* act = static_cast<const _Float16*>(g.act);
  const _Float16* a_src[AP];
#pragma unroll
  for (int j = 0; j < AP; ++j) {
    const int32_t r = arow[a_r0 + 16 * j];
    a_src[j] = act + (int64_t)(r >= 0 ? r : arow[0]) * g.K + a_c;
  }
  // weights: lane (n, gi) = (lane & 15, lane >> 4), row 64 t + 16 wave + n of
  // weight tile t.  Rows past N and groups past K read a valid group and get
  // scale 0.
  const int wn = lane & 15, wg = lane >> 4;
  const int Kc = (int)g.K;
  const int nch = (Kc + kQBK - 1) / kQBK;
  const int bshift = g.bs == 32 ? 5 : (g.bs == 64 ? 6 : 7);
  const uint32_t magic = opaque_magic<BF>();
  const uint8_t* wbase = g.codes + (int64_t)e * g.N * g.row_bytes;  // this expert's codes
  const int Nc = (int)g.N;
  const uint16_t* sbase = reinterpret_cast<const uint16_t*>(g.scales) + (int64_t)e * g.N * g.nblk;

  // All loads are unconditional (clamped addresses, validity applied where
  // the data is used), so the compiler keeps them in flight.  The steps walk
  // the K chunks; in chunk c all kNTG weight tiles use the same staged
  // activations (staged once per chunk, not once per tile): the wave
  // dequantizes its group of tile t, loaded kWS chunks earlier, and refills
  // that register stage with chunk c + kWS (the HBM stream); the activations
  // (L2-resident) move one chunk ahead through registers into the other LDS
  // buffer.  Tiles past ntc repeat the last tile and are never stored.
  struct WStage {
    typename Group<BITS>::W rw;
    uint32_t rs;
    bool ok;
  };
  // Tile-major offsets (N % 16 == 0, so every 16-row tile is full): group G =
  // 4c + wg of row 16 rt + wn sits at rt (16 ng GB) + 64 GB c + 4 GB wn + GB wg
  // in a full chunk and at rt (16 ng GB) + 64 GB c + gl (GB wn) + GB wg in a
  // last chunk of gl < 4 groups; the wave's row tile is uniform, so only the
  // lane term is per lane.  Groups past K use the chunk's last group (scale 0).
  const int ng = Kc >> 5, nfull = ng >> 2, gl = ng - 4 * nfull;
  const uint32_t lane_full = 4 * GB * wn + GB * wg;
  const uint32_t lane_last = gl ? GB * (uint32_t)(gl * wn + (wg < gl ? wg : gl - 1)) : lane_full;
  auto load_w = [&](WStage& st, int t, int c) {
    c = c < nch ? c : nch - 1;
    t = t < ntc ? t : ntc - 1;
    const int rt = (nt0 + t) * (kQBN / 16) + wave;  // the wave's row tile
    const bool rok = 16 * rt < Nc;                     // uniform
    const int G = 4 * c + wg;
    st.ok = rok && G < ng;
    const uint32_t off = (uint32_t)(rok ? rt : 0) * (uint32_t)(ng * 16 * GB) + 64 * GB * (uint32_t)c +
                         (c < nfull ? lane_full : lane_last);
    // streamed once: nontemporal, so that the weight stream does not push the
    // item's activation rows out of L2 (measured: 4% faster INT4 FC1 at 128 tokens)
    st.rw = __builtin_nontemporal_load(reinterpret_cast<const typename Group<BITS>::W*>(wbase + off));
    const int rowc = rok ? 16 * rt + wn : wn;
    st.rs = sbase[rowc * (int)g.nblk + ((32 * (G < ng ? G : ng - 1)) >> bshift)];
  };
  // (a_src already includes this thread's column a_c)
  u32x4 ra[AP];
  auto load_a = [&](int c) {
    c = c < nch ? c : nch - 1;
    const int k0 = c * kQBK;
    // columns past K (only in a last, partial chunk) read a valid column of
    // the same row; they are zeroed when stored
    const int kk = k0 + a_c < Kc ? k0 : Kc - 8 - a_c;
#pragma unroll
    for (int j = 0; j < AP; ++j) ra[j] = *reinterpret_cast<const u32x4*>(a_src[j] + kk);
  };
  const bool ktail = nch * kQBK > Kc;
  const bool a_tail = ktail && (nch - 1) * kQBK + a_c >= Kc;  // this thread's column in a last chunk is past K
  auto store_a = [&](int b, int c) {
    if (ktail && c == nch - 1) {  // uniform: the last, partial chunk
#pragma unroll
      for (int j = 0; j < AP; ++j)
        *reinterpret_cast<u32x4*>(&As[b][(a_r0 + 16 * j) * kQPitch + a_c]) = a_tail ? u32x4{0, 0, 0, 0} : ra[j];
    } else {
#pragma unroll
      for (int j = 0; j < AP; ++j)
        *reinterpret_cast<u32x4*>(&As[b][(a_r0 + 16 * j) * kQPitch + a_c]) = ra[j];
    }
  };

  f32x4 acc[kNTG][TM];
#pragma unroll
  for (int t = 0; t < kNTG; ++t)
#pragma unroll
    for (int i = 0; i < TM; ++i) acc[t][i] = f32x4{0, 0, 0, 0};
  const int fr = lane & 15;

  // outputs of weight tile t: lane l holds tokens 16i + 4(l/16) + r of token
  // tile i, weight row l%16 of this wave's 16
  auto epilogue = [&](int t) {
    const int64_t col = (int64_t)(nt0 + t) * kQBN + wave * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = i * 16 + 4 * (lane >> 4) + r;
        float v = acc[t][i][r];
        if (g.bias && col < g.N) v += Dt<BF>::to_f32(g.bias[(int64_t)e * g.N + col]);
        if (FC1) {
          // interleaved gate/up: even row = gate_i, odd row = up_i
          const float partner = __shfl_xor(v, 1);
          if ((lane & 1) == 0 && row < rows && col < g.N) {
            const float gt = v, up = partner;
            const float hv = gt / (1.0f + expf(-gt)) * up;
            g.h_out[(seg0 + row) * (g.N / 2) + col / 2] = Dt<BF>::from_f32(hv);
          }
        } else {
          if (row < rows && col < g.N) {
            const int32_t slot = g.perm[seg0 + row];
            g.slot_out[(int64_t)slot * g.N + col] = g.wts[slot] * v;
          }
        }
      }
    }
  };

  // kWS register stages of weights: chunk c is dequantized from stage
  // c % kWS, which then takes chunk c + kWS.  With 48- and 64-token items (many
  // workgroups per CU, each weight feeding more MFMAs) two stages keep two
  // chunks of the HBM stream in flight per wave (measured 3-4% faster at 512
  // tokens); with 32-token items one stage is faster (measured 3-12% at 128
  // tokens: the grid there puts only about three waves on a SIMD, and the
  // doubled loop body costs instruction fetch).
  // For two stages the chunk loop is unrolled by two so that each stage keeps
  // its registers (moving a register whose load is in flight would wait for
  // it).
  constexpr int kWS = BM >= 48 ? 2 : 1;
  WStage w0[kNTG], w1[kNTG];
#pragma unroll
  for (int t = 0; t < kNTG; ++t) load_w(w0[t], t, 0);
  if constexpr (kWS == 2) {
#pragma unroll
    for (int t = 0; t < kNTG; ++t) load_w(w1[t], t, 1);
  }
  load_a(0);
  store_a(0, 0);
  load_a(1);
  __syncthreads();
  // Chunk c first moves the activations of chunk c + 1 from registers to LDS
  // buffer b ^ 1 (last read in chunk c - 1, before the barrier that ended
  // it) and loads those of chunk c + 2, then refills the weight stages.
  // Vector loads complete in order, so activation loads issued after a
  // weight load of a later chunk would make the LDS store wait for that
  // weight load too; issued first, they leave kWS chunks of weights in flight.
  auto chunk = [&](WStage (&ws)[kNTG], int c) {
    const int b = c & 1;
    if (c + 1 < nch) {
      store_a(b ^ 1, c + 1);
      load_a(c + 2);
    }
#pragma unroll
    for (int t = 0; t < kNTG; ++t) {
      u32x4 wf[4];
      dequant_group<BITS, BF>(ws[t].rw, (uint16_t)(ws[t].ok ? ws[t].rs : 0u), magic, wf);
      load_w(ws[t], t, c + kWS);
      if (t < ntc) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int kk = 32 * wg + 8 * q;
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            if (i < vt) {
              const u32x4 a = *reinterpret_cast<const u32x4*>(&As[b][(i * 16 + fr) * kQPitch + kk]);
              acc[t][i] = mfma16x16x32<BF>(a, wf[q], acc[t][i]);
            }
          }
        }
      }
    }
    if (c + 1 < nch) __syncthreads();
  };
  if constexpr (kWS == 2) {
    for (int c = 0; c < nch; c += 2) {
      chunk(w0, c);
      if (c + 1 < nch) chunk(w1, c + 1);
    }
  } else {
    for (int c = 0; c < nch; ++c) chunk(w0, c);
  }
#pragma unroll
  for (int t = 0; t < kNTG; ++t)
    if (t < ntc) epilogue(t);
}

// ---------------------------------------------------------------------------
// Decode path (a few tokens): no grouping, no slot buffer.  Each selected
// (token, rank) pair is its own GEMV: with T * k small every pair reads its
// expert's weights once, which is what the grouped path would read as well.
// ---------------------------------------------------------------------------

// Reinterprets a 32-bit word as two halves.  The word is taken by value: this
// compiler folds __builtin_bit_cast of a vector element (v.y, v.z, v.w) to a
// read of element .x, so elements are always copied into a scalar first.
__device__ __forceinline__ half2t as_half2(uint32_t v) { return __builtin_bit_cast(half2t, v); }

// s * sum_k (q_k - z) a_k over one 32-code group, for the decode GEMVs: the
// codes become exact fp16 / bf16 (q - z) (no per-code scale multiply), v_dot2
// sums the exact products in fp32 and the group's scale is applied once.
template <int BITS, bool BF>
__device__ __forceinline__ float group_dot_unscaled(const typename Group<BITS>::W w, float s,
                                                    uint32_t magic, const u32x4* a16) {
  uint32_t p[16];
  raw_pairs(w, magic, p);
  float acc = 0.0f;
  if constexpr (BF) {
    const float zb = -(Dt<true>::kBase + (float)(1 << (BITS - 1)));
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = bf_pack(bf_lo(p[i]) + zb, bf_hi(p[i]) + zb);  // exact
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const u32x4 av = a16[t];
      const uint32_t a0 = av.x, a1 = av.y, a2 = av.z, a3 = av.w;
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p[4 * t]), __builtin_bit_cast(bf16x2, a0), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p[4 * t + 1]), __builtin_bit_cast(bf16x2, a1), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p[4 * t + 2]), __builtin_bit_cast(bf16x2, a2), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p[4 * t + 3]), __builtin_bit_cast(bf16x2, a3), acc, false);
    }
  } else {
    const half2t zb = zero_bias<BITS>();
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2t, p[i]) + zb);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const u32x4 av = a16[t];
      acc = __builtin_amdgcn_fdot2(as_half2(p[4 * t]), as_half2(av.x), acc, false);
      acc = __builtin_amdgcn_fdot2(as_half2(p[4 * t + 1]), as_half2(av.y), acc, false);
      acc = __builtin_amdgcn_fdot2(as_half2(p[4 * t + 2]), as_half2(av.z), acc, false);
      acc = __builtin_amdgcn_fdot2(as_half2(p[4 * t + 3]), as_half2(av.w), acc, false);
    }
  }
  return acc * s;
}

// Partial dot products of the 16-row weight tile at row0 of one expert with
// an fp16 / bf16 activation row held in LDS: lane (n, g) = (lane & 15,
// lane >> 4) takes group 4c + g of row row0 + n for the chunks c = c0,
// c0 + cstep, ... (one 768-byte (INT3) or 1024-byte (INT4) load per wave and
// chunk in the tile-major layout).  Loads
// are issued in batches of kDecFc1Batch chunks before any is used, the first
// batch before the activations are staged; groups past K read a valid group
// with scale 0.  Four chunks per wave cover a K = 2048 row with the FC1
// workgroup's four waves, so no slot of the batch reloads a clamped chunk
// (eight measured slower at T = 1: INT3 13.05 -> 12.1 us, INT4 13.95 ->
// 12.6 us with four); the FC2 half tiles below take two halves of
// kDecBatch / 2 chunks (three per half at I = 768 measured the same).
constexpr int kDecBatch = 8;
constexpr int kDecFc1Batch = 4;

struct TileRef {
  const uint8_t* codes;     // this expert's codes
  const uint16_t* scales;   // this expert's fp16 scales
  int N, K, nblk, bshift, row, ng, nch, g;
};

template <int BITS, bool BF>
struct TileBatch {
  typename Group<BITS>::W w[kDecFc1Batch];
  uint16_t s[kDecFc1Batch];
  int G[kDecFc1Batch];
  uint32_t ok;  // bit u: group G[u] lies inside K (the loaded scale is used as is)
  int cnt;      // chunks of this batch inside K (wave-uniform)

  // (the loaded words are not touched here, so no wait is needed before the
  // caller's next steps)
  __device__ __forceinline__ void load(const TileRef& t, int c0, int cstep) {
    cnt = c0 < t.nch ? (t.nch - c0 + cstep - 1) / cstep : 0;
    ok = 0;
#pragma unroll
    for (int u = 0; u < kDecFc1Batch; ++u) {
      const int Gr = 4 * (c0 + u * cstep) + t.g;
      ok |= (Gr < t.ng ? 1u : 0u) << u;
      G[u] = Gr < t.ng ? Gr : t.ng - 1;
      w[u] = *reinterpret_cast<const typename Group<BITS>::W*>(t.codes + moe_goff<BITS>(t.N, t.K, t.row, G[u]));
      s[u] = t.scales[t.row * t.nblk + ((32 * G[u]) >> t.bshift)];
    }
  }
  __device__ __forceinline__ float dot(const _Float16* xs, uint32_t magic) const {
    float acc = 0.0f;
#pragma unroll
    for (int u = 0; u < kDecFc1Batch; ++u)
      if (u < cnt) {
        const uint16_t sc = (ok >> u) & 1u ? s[u] : (uint16_t)0;
        acc += group_dot_unscaled<BITS, BF>(w[u], Dt<BF>::to_f32(sc), magic,
                                  reinterpret_cast<const u32x4*>(xs + 32 * G[u]));
      }
    return acc;
  }
};

// Eight-row tiles, two K chunks per wave load: lane (n, g, h) = (lane & 7,
// (lane >> 3) & 3, lane >> 5) takes group 4c + g of row n for the chunks
// c = c0 + 2u + h (used where 16-row tiles would leave CUs idle).  Chunks or
// groups past K are skipped per lane.
template <int BITS, bool BF>
struct HalfBatch {
  static constexpr int kU = kDecBatch / 2;
  typename Group<BITS>::W w[kU];
  uint16_t s[kU];
  int G[kU];
  uint32_t ok;  // bit u: chunk and group inside K

  __device__ __forceinline__ void load(const TileRef& t, int c0, int h) {
    ok = 0;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = c0 + 2 * u + h;
      const int Gr = 4 * c + t.g;
      const bool v = c < t.nch && Gr < t.ng;
      ok |= (v ? 1u : 0u) << u;
      G[u] = v ? Gr : t.ng - 1;
      w[u] = *reinterpret_cast<const typename Group<BITS>::W*>(t.codes + moe_goff<BITS>(t.N, t.K, t.row, G[u]));
      s[u] = t.scales[t.row * t.nblk + ((32 * G[u]) >> t.bshift)];
    }
  }
  __device__ __forceinline__ float dot(const _Float16* xs, uint32_t magic) const {
    float acc = 0.0f;
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if ((ok >> u) & 1u)
        acc += group_dot_unscaled<BITS, BF>(w[u], Dt<BF>::to_f32(s[u]), magic,
                                  reinterpret_cast<const u32x4*>(xs + 32 * G[u]));
    return acc;
  }
};

// Stages n 16-byte pieces of src into LDS dst with nt threads: the first two
// pieces per thread are loaded by stage_first (before the caller issues its
// weight loads: loads complete in order, so waiting for these does not wait
// for the weights) and stored by stage_rest, which also copies any further
// pieces.
struct Stage2 {
  u32x4 v[2];
  __device__ __forceinline__ void first(const u32x4* src, int n, int tid, int nt) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = tid + u * nt;
      v[u] = src[i < n ? i : n - 1];
    }
  }
  __device__ __forceinline__ void rest(const u32x4* src, u32x4* dst, int n, int tid, int nt) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (tid + u * nt < n) dst[tid + u * nt] = v[u];
    for (int i = tid + 2 * nt; i < n; i += nt) dst[i] = src[i];
  }
};

// The decode launches pass flat arguments (their leading ones, at most 14
// dwords, arrive preloaded in SGPRs): the codes pointer with the scales at
// codes + off_s, and the shape packed in two words, kn = K | N << 16 and
// ek = E | top_k << 16 | bs_shift << 24 (bs = 32 << bs_shift; K, N and E below
// 2^16 on this path).  The blocked row of BITS-bit codes holds K BITS / 8
// bytes (K is a multiple of the block size).
template <int BITS>
__device__ __forceinline__ MoeGemmArgs decode_args(const uint8_t* codes, uint32_t off_s,
                                                   const void* act, uint32_t kn, uint32_t ek) {
  MoeGemmArgs g{};
  g.codes = codes;
  g.scales = reinterpret_cast<const uint16_t*>(codes + off_s);
  g.act = act;
  g.K = kn & 0xFFFFu;
  g.N = kn >> 16;
  g.E = (int)(ek & 0xFFFFu);
  g.top_k = (int)((ek >> 16) & 0xFFu);
  g.bs = 32 << (ek >> 24);
  g.row_bytes = g.K * BITS / 8;
  g.nblk = g.K / g.bs;
  return g;
}

__device__ __forceinline__ TileRef tile_ref(const MoeGemmArgs& g, int e, int row0, int lane) {
  TileRef t;
  t.N = (int)g.N;
  t.K = (int)g.K;
  t.codes = g.codes + (int64_t)e * t.N * g.row_bytes;
  t.scales = g.scales + (int64_t)e * t.N * g.nblk;
  t.nblk = (int)g.nblk;
  t.bshift = g.bs == 32 ? 5 : (g.bs == 64 ? 6 : 7);
  t.row = row0 + (lane & 15);
  t.ng = t.K >> 5;
  t.nch = (t.ng + 3) >> 2;
  t.g = lane >> 4;
  return t;
}

// (Routing +) FC1 + SwiGLU: a workgroup per (slot, 16-row tile = 8 gate/up
// pairs).  With ROUTE (used for very few slots, where a separate routing
// launch costs more than the repeated work), wave 0 routes the slot's token
// (every workgroup recomputes the same top-k; the tile-0 workgroup of rank 0
// also writes it out for FC2) while the token's row of x is loading into
// LDS; otherwise the ids come from the routing kernel.  Wave w then takes the K
// chunks w, w + 4, ... of expert ids[t, j]'s tile; partials are summed in a
// fixed order and h[slot I + 8 tile + m] = fp16(silu(g_m) u_m) for gate row
// 2m, up row 2m + 1.
template <int kPer, bool ROUTE, int BITS, bool BF>
__global__ void __launch_bounds__(256) qmoe_fc1_decode(const void* __restrict__ act,
                                                       const float* __restrict__ logits,
                                                       const uint8_t* __restrict__ codes,
                                                       uint16_t* __restrict__ h_out, uint32_t off_s,
                                                       uint32_t kn, uint32_t ek,
                                                       int32_t* __restrict__ ids,
                                                       float* __restrict__ wts,
                                                       const uint16_t* __restrict__ bias) {
  MoeGemmArgs g = decode_args<BITS>(codes, off_s, act, kn, ek);
  g.h_out = h_out;
  g.bias = bias;
  extern __shared__ __align__(16) uint8_t sm[];
  const int K = (int)g.K, N = (int)g.N, I = N / 2, ntile = N >> 4, k = g.top_k;
  _Float16* xs = reinterpret_cast<_Float16*>(sm);
  float* red = reinterpret_cast<float*>(sm + 2 * K);  // K % 32 == 0: 16-byte aligned
  int32_t* rid = reinterpret_cast<int32_t*>(red + 256);
  float* rw = reinterpret_cast<float*>(rid + 16);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = (int)blockIdx.x / ntile, tile = (int)blockIdx.x % ntile;
  const int t = slot / k, j = slot % k;
  const u32x4* xr = reinterpret_cast<const u32x4*>(static_cast<const _Float16*>(g.act) + (int64_t)t * K);
  Stage2 xst;
  xst.first(xr, K / 8, tid, 256);
  __builtin_amdgcn_sched_barrier(0);
  int e;
  if constexpr (ROUTE) {
    if (wave == 0) route_token<kPer>(logits + (int64_t)t * g.E, g.E, k, lane, rid, rw);
    __syncthreads();
    if (tile == 0 && j == 0 && tid < k) {
      ids[t * k + tid] = rid[tid];
      wts[t * k + tid] = rw[tid];
    }
    e = clamp_id(rid[j], g.E);
  } else {
    e = clamp_id(ids[slot], g.E);
  }
  const TileRef tr = tile_ref(g, e, 16 * tile, lane);
  TileBatch<BITS, BF> b;
  b.load(tr, wave, 4);
  __builtin_amdgcn_sched_barrier(0);
  xst.rest(xr, reinterpret_cast<u32x4*>(xs), K / 8, tid, 256);
  __syncthreads();
  const uint32_t magic = opaque_magic<BF>();
  float acc = b.dot(xs, magic);
  for (int c = wave + 4 * kDecFc1Batch; c < tr.nch; c += 4 * kDecFc1Batch) {
    b.load(tr, c, 4);
    acc += b.dot(xs, magic);
  }
  red[wave * 64 + lane] = acc;
  __syncthreads();
  if (tid < 8) {
    float gs = 0.0f, us = 0.0f;
    for (int w = 0; w < 4; ++w)
      for (int q = 0; q < 4; ++q) {
        gs += red[w * 64 + q * 16 + 2 * tid];
        us += red[w * 64 + q * 16 + 2 * tid + 1];
      }
    if (g.bias) {
      const uint16_t* b = g.bias + (int64_t)e * N + 16 * tile + 2 * tid;
      gs += Dt<BF>::to_f32(b[0]);
      us += Dt<BF>::to_f32(b[1]);
    }
    g.h_out[(int64_t)slot * I + 8 * tile + tid] = Dt<BF>::from_f32(gs / (1.0f + expf(-gs)) * us);
  }
}

// FC2 + combine: a workgroup per (token t, 8-row half tile) with one wave per rank
// j; the token's k rows of h are staged in LDS; wave j forms the partials of
// expert ids[t, j]'s tile rows, then out[t, n] = fp16(sum_j r_j y_j[n]) with
// y_j and the rank sum in fixed orders.
template <int BITS, bool BF>
__global__ void __launch_bounds__(1024) qmoe_fc2_decode(const void* __restrict__ act,
                                                        const int32_t* __restrict__ ids,
                                                        const uint8_t* __restrict__ codes,
                                                        const float* __restrict__ wts,
                                                        uint16_t* __restrict__ out, uint32_t off_s,
                                                        uint32_t kn, uint32_t ek,
                                                        const uint16_t* __restrict__ bias,
                                                        float* __restrict__ slot_dbg) {
  MoeGemmArgs g = decode_args<BITS>(codes, off_s, act, kn, ek);
  g.perm = ids;
  g.wts = wts;
  g.bias = bias;
  extern __shared__ __align__(16) uint8_t sm[];
  const int H = (int)g.N, I = (int)g.K, k = g.top_k, ntile = H >> 3;  // 8-row tiles
  _Float16* hs = reinterpret_cast<_Float16*>(sm);
  float* red = reinterpret_cast<float*>(sm + 2 * k * I);  // I % 32 == 0: 16-byte aligned
  const int tid = threadIdx.x, lane = tid & 63;
  const int j = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = (int)blockIdx.x / ntile, tile = (int)blockIdx.x % ntile;
  const int e = clamp_id(g.perm[t * k + j], g.E);  // perm holds the routed ids here
  TileRef tr = tile_ref(g, e, 8 * tile, lane & 7);
  tr.g = (lane >> 3) & 3;
  const int hsel = lane >> 5;
  const u32x4* hr = reinterpret_cast<const u32x4*>(static_cast<const _Float16*>(g.act) + (int64_t)t * k * I);
  Stage2 hst;
  hst.first(hr, k * I / 8, tid, 64 * k);
  __builtin_amdgcn_sched_barrier(0);
  HalfBatch<BITS, BF> b;
  b.load(tr, 0, hsel);
  __builtin_amdgcn_sched_barrier(0);
  hst.rest(hr, reinterpret_cast<u32x4*>(hs), k * I / 8, tid, 64 * k);
  __syncthreads();
  const uint32_t magic = opaque_magic<BF>();
  const _Float16* hj = hs + j * I;
  float acc = b.dot(hj, magic);
  for (int c = 2 * HalfBatch<BITS, BF>::kU; c < tr.nch; c += 2 * HalfBatch<BITS, BF>::kU) {
    b.load(tr, c, hsel);
    acc += b.dot(hj, magic);
  }
  red[j * 64 + lane] = acc;
  __syncthreads();
  if (tid < 8) {
    const int n = 8 * tile + tid;
    float o = 0.0f;
    for (int r = 0; r < k; ++r) {
      float y = 0.0f;
      for (int q = 0; q < 8; ++q) y += red[r * 64 + q * 8 + tid];
      if (g.bias) y += Dt<BF>::to_f32(g.bias[(int64_t)clamp_id(g.perm[t * k + r], g.E) * H + n]);
      const float ry = g.wts[t * k + r] * y;
      if (slot_dbg) slot_dbg[((int64_t)t * k + r) * H + n] = ry;
      o += ry;
    }
    out[(int64_t)t * H + n] = Dt<BF>::from_f32(o);
  }
}

// ---------------------------------------------------------------------------
// 5. combine
// ---------------------------------------------------------------------------
template <bool BF>
__global__ void __launch_bounds__(256) qmoe_combine(const float* __restrict__ slots, int64_t T,
                                                    int k, int64_t H, uint16_t* __restrict__ out) {
  // four consecutive outputs per thread (H % 32 == 0): 16-byte slot loads
  const int64_t i4 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i4 >= T * H / 4) return;
  const int64_t i = 4 * i4;
  const int64_t t = i / H, n = i % H;
  f32x4 acc = f32x4{0, 0, 0, 0};
  for (int j = 0; j < k; ++j) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(slots + (t * k + j) * H + n);
    acc = f32x4{acc.x + v.x, acc.y + v.y, acc.z + v.z, acc.w + v.w};
  }
  const uint32_t lo = (uint32_t)Dt<BF>::from_f32(acc.x) | ((uint32_t)Dt<BF>::from_f32(acc.y) << 16);
  const uint32_t hi = (uint32_t)Dt<BF>::from_f32(acc.z) | ((uint32_t)Dt<BF>::from_f32(acc.w) << 16);
  *reinterpret_cast<u32x2*>(out + i) = u32x2{lo, hi};
}

// debug: h rows back in slot order
__global__ void qmoe_gather_h(const uint16_t* __restrict__ h, const int32_t* __restrict__ inv,
                              int64_t S, int64_t I, uint16_t* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= S * I) return;
  const int64_t slot = i / I, c = i % I;
  dst[i] = h[(int64_t)inv[slot] * I + c];
}

struct Ws {
  uint64_t ids, wts, counts, offsets, perm, inv, items, nitems, h, slots, total;
};

constexpr int kMaxBM = 64;  // largest token tile of a work item

int64_t max_items(int64_t Tt, int k, int64_t E, int bm) {
  const int64_t S = Tt * k;
  return (S < E ? S : E) + (S + bm - 1) / bm;
}

// Token tile of the work items: about the expected tokens per expert, so a
// weight tile is dequantized once for all of an expert's tokens, with as few
// padding rows as the 16-token MFMA tiles allow (at 512 tokens, top-8 of 128
// experts, about 32 tokens per expert: 48-token items measured 4% faster than
// 64-token ones, INT3 and INT4).
int pick_bm(int64_t Tt, int k, int64_t E) { return Tt * k <= 24 * E ? 32 : (Tt * k <= 40 * E ? 48 : kMaxBM); }

Ws ws_layout(const Sizes& s1, const Sizes& s2, int k, int64_t T) {
  const int64_t Tt = T < kTokTile ? T : kTokTile;
  const int64_t S = Tt * k, E = s1.E, I = s2.K, H = s1.K;
  Ws w;
  uint64_t o = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t at = o;
    o += align256(bytes);
    return at;
  };
  w.ids = take(S * 4);
  w.wts = take(S * 4);
  w.counts = take(E * 4);
  w.offsets = take((E + 1) * 4);
  w.perm = take(S * 4);
  w.inv = take(S * 4);
  w.items = take(max_items(Tt, k, E, 32) * 8);  // the smallest tile has the most items
  w.nitems = take(4);
  w.h = take(S * I * 2);
  w.slots = take(S * H * 4);
  w.total = o;
  return w;
}

// Calls f with the code width (3 or 4) and the bfloat16 flag as compile-time
// constants.
template <typename F>
void by_kind(int64_t bits, bool bf, F&& f) {
  if (bits == 4) {
    if (bf)
      f(std::integral_constant<int, 4>(), std::true_type());
    else
      f(std::integral_constant<int, 4>(), std::false_type());
  } else {
    if (bf)
      f(std::integral_constant<int, 3>(), std::true_type());
    else
      f(std::integral_constant<int, 3>(), std::false_type());
  }
}

// An asynchronous device-to-device copy that keeps the first failure.
hipError_t copy_d2d(hipError_t prev, void* dst, const void* src, int64_t bytes, hipStream_t st) {
  const hipError_t e = hipMemcpyAsync(dst, src, (size_t)bytes, hipMemcpyDeviceToDevice, st);
  return prev != hipSuccess ? prev : e;
}

void launch_route(const float* logits, int64_t T, int E, int k, int32_t* ids, float* wts,
                  hipStream_t st) {
  const dim3 grid((unsigned)((T + 3) / 4)), block(256);
  if (E <= 128)
    hipLaunchKernelGGL(qmoe_route<2>, grid, block, 0, st, logits, T, E, k, ids, wts);
  else if (E <= 256)
    hipLaunchKernelGGL(qmoe_route<4>, grid, block, 0, st, logits, T, E, k, ids, wts);
  else
    hipLaunchKernelGGL(qmoe_route<kMaxE / 64>, grid, block, 0, st, logits, T, E, k, ids, wts);
}


}  // namespace

// Byte offset of a plan's scales from its codes for the flat decode
// launches (the sections of a plan made by mnb_prepare follow the codes).
bool scales_offset(const mnb_plan& p, uint32_t* off) {
  const uintptr_t c = reinterpret_cast<uintptr_t>(p.codes), v = reinterpret_cast<uintptr_t>(p.scales);
  if (v < c || v - c > 0xFFFFFF00u || (v - c) % 2) return false;
  *off = (uint32_t)(v - c);
  return true;
}

bool qmoe_supported(const Sizes& s1, const Sizes& s2, int top_k) {
  // the grouping kernel's per-expert histograms and the routing kernels'
  // register-held top-k bound E and k; in-expert code offsets are 32-bit
  return s1.E <= kMaxE && top_k <= kMaxTopK && s1.N * s1.row_bytes < (int64_t(1) << 31) &&
         s2.N * s2.row_bytes < (int64_t(1) << 31);
}

uint64_t qmoe_ws_bytes(const Sizes& s1, const Sizes& s2, int top_k, int64_t T) {
  if (T <= 0) return 0;
  return ws_layout(s1, s2, top_k, T).total;
}

hipError_t launch_qmoe(const Sizes& s1, const mnb_plan& p1, const Sizes& s2, const mnb_plan& p2,
                       int top_k, int64_t T, const uint16_t* x, const float* logits,
                       const uint16_t* b1, const uint16_t* b2, uint16_t* out, void* ws,
                       hipStream_t st, const QmoeDebug* dbg) {
  const int64_t E = s1.E, H = s1.K, I = s2.K;
  const int k = top_k;
  // the C ABI rejects these as unsupported before calling; kept as a guard
  if (!qmoe_supported(s1, s2, k)) return hipErrorNotSupported;
  const Ws L = ws_layout(s1, s2, k, T);
  uint8_t* w = static_cast<uint8_t*>(ws);
  int32_t* ids = reinterpret_cast<int32_t*>(w + L.ids);
  float* wts = reinterpret_cast<float*>(w + L.wts);
  GroupOut go{reinterpret_cast<int32_t*>(w + L.counts), reinterpret_cast<int32_t*>(w + L.offsets),
              reinterpret_cast<int32_t*>(w + L.perm), reinterpret_cast<int32_t*>(w + L.inv),
              reinterpret_cast<int32_t*>(w + L.items), reinterpret_cast<int32_t*>(w + L.nitems)};
  uint16_t* hbuf = reinterpret_cast<uint16_t*>(w + L.h);
  float* slots = reinterpret_cast<float*>(w + L.slots);
  // activations, scales, biases, h and out share the plans' 16-bit type
  const bool bf = p1.desc.scale_dtype == MNB_DTYPE_BF16;
  const size_t group_lds = (size_t)(5 + kGroupThreads / 64) * E * 4;

  // few tokens: per-slot GEMVs, no grouping (every slot reads its expert once);
  // the activation rows they stage in LDS bound H and k * I
  uint32_t os1, os2;
  if (T * k <= kDecodeSlots && H <= 16384 && k * I <= 16384 &&
      scales_offset(p1, &os1) && scales_offset(p2, &os2)) {
    const int64_t S = T * k;
    const uint32_t ek = (uint32_t)E | ((uint32_t)k << 16);
    const uint32_t kn1 = (uint32_t)s1.K | ((uint32_t)s1.N << 16), kn2 = (uint32_t)s2.K | ((uint32_t)s2.N << 16);
    const uint32_t ek1 = ek | ((uint32_t)(s1.bs == 32 ? 0 : (s1.bs == 64 ? 1 : 2)) << 24);
    const uint32_t ek2 = ek | ((uint32_t)(s2.bs == 32 ? 0 : (s2.bs == 64 ? 1 : 2)) << 24);
    const uint8_t* c1 = static_cast<const uint8_t*>(p1.codes);
    const uint8_t* c2 = static_cast<const uint8_t*>(p2.codes);
    const dim3 g1((unsigned)(S * (s1.N / 16))), wg1(256);
    const size_t l1 = (size_t)(2 * H + 4 * 256 + 128);
    if (S > kFusedRouteSlots) launch_route(logits, T, (int)E, k, ids, wts, st);
    by_kind(s1.bits, bf, [&](auto bits, auto bfc) {
      constexpr int B = decltype(bits)::value;
      constexpr bool BF = decltype(bfc)::value;
      if (S > kFusedRouteSlots)
        hipLaunchKernelGGL((qmoe_fc1_decode<2, false, B, BF>), g1, wg1, l1, st, x, logits, c1, hbuf, os1, kn1, ek1, ids, wts, b1);
      else if (E <= 128)
        hipLaunchKernelGGL((qmoe_fc1_decode<2, true, B, BF>), g1, wg1, l1, st, x, logits, c1, hbuf, os1, kn1, ek1, ids, wts, b1);
      else if (E <= 256)
        hipLaunchKernelGGL((qmoe_fc1_decode<4, true, B, BF>), g1, wg1, l1, st, x, logits, c1, hbuf, os1, kn1, ek1, ids, wts, b1);
      else
        hipLaunchKernelGGL((qmoe_fc1_decode<kMaxE / 64, true, B, BF>), g1, wg1, l1, st, x, logits, c1, hbuf, os1, kn1, ek1, ids, wts, b1);
    });
    by_kind(s2.bits, bf, [&](auto bits, auto bfc) {
      constexpr int B = decltype(bits)::value;
      constexpr bool BF = decltype(bfc)::value;
      hipLaunchKernelGGL((qmoe_fc2_decode<B, BF>), dim3((unsigned)(T * (H / 8))), dim3(64 * k),
                         (size_t)(2 * k * I + 4 * 64 * k), st, hbuf, ids, c2, wts, out, os2, kn2, ek2,
                         b2, dbg ? dbg->slot : nullptr);
    });
    if (dbg) {
      hipError_t e = hipSuccess;
      if (dbg->ids) e = copy_d2d(e, dbg->ids, ids, S * 4, st);
      if (dbg->w) e = copy_d2d(e, dbg->w, wts, S * 4, st);
      if (dbg->h) e = copy_d2d(e, dbg->h, hbuf, S * I * 2, st);
      if (e != hipSuccess) return e;
    }
    return hipGetLastError();
  }

  for (int64_t t0 = 0; t0 < T; t0 += kTokTile) {
    const int64_t Tt = (T - t0) < kTokTile ? (T - t0) : kTokTile;
    const int64_t S = Tt * k;
    const int bm = pick_bm(Tt, k, E);
    const int64_t items = max_items(Tt, k, E, bm);
    launch_route(logits + t0 * E, Tt, (int)E, k, ids, wts, st);
    hipLaunchKernelGGL(qmoe_group, dim3(1), dim3(kGroupThreads), group_lds, st, ids, Tt, k, (int)E,
                       items, bm, go);
    MoeGemmArgs a1{static_cast<const uint8_t*>(p1.codes), static_cast<const uint16_t*>(p1.scales),
                   x + t0 * H, s1.N, s1.K, s1.row_bytes, s1.nb, s1.bs, k, (int)E,
                   go.counts, go.offsets, go.perm, go.items, go.nitems, wts, hbuf, nullptr,
                   b1};
    const int ntg1 = ntg_for(bm, (int)s1.bits), ntg2 = ntg_for(bm, (int)s2.bits);
    const int64_t nt1 = (s1.N + kQBN - 1) / kQBN, ng1 = (nt1 + ntg1 - 1) / ntg1;
    const dim3 grid1((unsigned)((items + 7) / 8 * 8 * ng1));
    by_kind(s1.bits, bf, [&](auto bits, auto bfc) {
      constexpr int B = decltype(bits)::value;
      constexpr bool BF = decltype(bfc)::value;
      if (bm == 32)
        hipLaunchKernelGGL((qmoe_gemm<true, 32, B, BF>), grid1, dim3(256), 0, st, a1, ng1, nt1);
      else if (bm == 48)
        hipLaunchKernelGGL((qmoe_gemm<true, 48, B, BF>), grid1, dim3(256), 0, st, a1, ng1, nt1);
      else
        hipLaunchKernelGGL((qmoe_gemm<true, kMaxBM, B, BF>), grid1, dim3(256), 0, st, a1, ng1, nt1);
    });
    MoeGemmArgs a2{static_cast<const uint8_t*>(p2.codes), static_cast<const uint16_t*>(p2.scales),
                   hbuf, s2.N, s2.K, s2.row_bytes, s2.nb, s2.bs, k, (int)E,
                   go.counts, go.offsets, go.perm, go.items, go.nitems, wts, nullptr, slots,
                   b2};
    const int64_t nt2 = (s2.N + kQBN - 1) / kQBN, ng2 = (nt2 + ntg2 - 1) / ntg2;
    const dim3 grid2((unsigned)((items + 7) / 8 * 8 * ng2));
    by_kind(s2.bits, bf, [&](auto bits, auto bfc) {
      constexpr int B = decltype(bits)::value;
      constexpr bool BF = decltype(bfc)::value;
      if (bm == 32)
        hipLaunchKernelGGL((qmoe_gemm<false, 32, B, BF>), grid2, dim3(256), 0, st, a2, ng2, nt2);
      else if (bm == 48)
        hipLaunchKernelGGL((qmoe_gemm<false, 48, B, BF>), grid2, dim3(256), 0, st, a2, ng2, nt2);
      else
        hipLaunchKernelGGL((qmoe_gemm<false, kMaxBM, B, BF>), grid2, dim3(256), 0, st, a2, ng2, nt2);
    });
    const dim3 gridc((unsigned)((Tt * H / 4 + 255) / 256));
    if (bf)
      hipLaunchKernelGGL(qmoe_combine<true>, gridc, dim3(256), 0, st, slots, Tt, k, H, out + t0 * H);
    else
      hipLaunchKernelGGL(qmoe_combine<false>, gridc, dim3(256), 0, st, slots, Tt, k, H, out + t0 * H);
    if (dbg) {
      hipError_t e = hipSuccess;
      if (dbg->ids) e = copy_d2d(e, dbg->ids + t0 * k, ids, S * 4, st);
      if (dbg->w) e = copy_d2d(e, dbg->w + t0 * k, wts, S * 4, st);
      if (dbg->slot) e = copy_d2d(e, dbg->slot + t0 * k * H, slots, S * H * 4, st);
      if (e != hipSuccess) return e;
      if (dbg->h)
        hipLaunchKernelGGL(qmoe_gather_h, dim3((unsigned)((S * I + 255) / 256)), dim3(256), 0, st,
                           hbuf, go.inv, S, I, dbg->h + t0 * k * I);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mnb
