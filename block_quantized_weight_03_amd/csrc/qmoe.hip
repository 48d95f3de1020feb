// Top-k routed INT3 QMoE layer for gfx950.
//
// Sources: onnxruntime PR "INT3 QMoE CUDA correctness baseline and Qwen
// experimental results" (PR summary: routing, fused gate/up SwiGLU, an
// independent down projection and aggregation, with bounded activation tiling
// and no floating expert weights; embedded P0/P1 body, section "P0" for the
// row-local LSB-first 3-bit format and "P1" for the fused interleaved gate/up
// and swiglu profile; embedded Olive body for the (code - 4) * scale decode)
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
//              T*k slots into expert-grouped order that is stable in (token,
//              rank) order, and the list of (expert, row-tile) work items.
//  3. fc1:     per work item, G = X_e W1_e^T on the matrix cores (gathered
//              token rows; INT3 tiles dequantized into LDS as
//              fp16((q - 4) * s)); epilogue h_i = silu(g_i) * u_i from the
//              interleaved gate/up columns, rounded to fp16.
//  4. fc2:     per work item, Y_e = h_e W2_e^T; epilogue multiplies by the
//              slot's routing weight and writes an fp32 slot row.
//  5. combine: out[t] = fp16(sum_j slot[t, j]) in rank order (deterministic).

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace mnb {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x3 __attribute__((ext_vector_type(3), aligned(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTokTile = 512;   // tokens per pass (bounds the workspace)
constexpr int kMaxE = 1024;     // experts supported by the grouping kernel
constexpr int kBM = 32;         // token rows per work item
constexpr int kBN = 64;         // weight rows per workgroup
constexpr int kBK = 128;        // K per step
constexpr int kPitch = kBK + 8; // LDS pitch (halves): conflict-free fragment reads
constexpr int kGroupThreads = 1024;

// ---------------------------------------------------------------------------
// 1. routing
// ---------------------------------------------------------------------------
__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

__global__ void __launch_bounds__(256) qmoe_route(const float* __restrict__ logits, int64_t T,
                                                  int E, int k, int32_t* __restrict__ ids,
                                                  float* __restrict__ wts) {
  constexpr int kPer = kMaxE / 64;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;  // whole waves leave together
  const float* l = logits + t * E;
  float v[kPer];
  uint32_t taken = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = i * 64 + lane;
    const float x = e < E ? l[e] : 0.0f;
    v[i] = x != x ? -INFINITY : x;  // NaN ranks last, so k <= E picks are always valid
  }
  float lmax = 0.0f, den = 0.0f;
  float sel_v[16];
  int sel_i[16];
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = i * 64 + lane;
      if (e < E && !((taken >> i) & 1u) && better(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(bv, m);
      const int oi = __shfl_xor(bi, m);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    // every lane now holds the same winner
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (j == 0) lmax = bv;
    const float ex = expf(bv - lmax);
    den += ex;
    if (j < 16) {
      sel_v[j] = ex;
      sel_i[j] = bi;
    }
  }
  if (lane == 0) {
    for (int j = 0; j < k && j < 16; ++j) {
      ids[t * k + j] = sel_i[j];
      wts[t * k + j] = sel_v[j] / den;
    }
  }
}

// ---------------------------------------------------------------------------
// 2. grouping: counts, offsets, stable permutation, work items
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

__global__ void __launch_bounds__(kGroupThreads) qmoe_group(const int32_t* __restrict__ ids,
                                                            int64_t T, int k, int E, int64_t max_items,
                                                            GroupOut o) {
  extern __shared__ __align__(16) int32_t gsm[];
  int32_t* cnt = gsm;                 // [E]
  int32_t* off = cnt + E;             // [E + 1]
  int32_t* carry = off + E + 1;       // [E]
  int32_t* segpre = carry + E;        // [segs][E]
  const int tid = threadIdx.x;
  const int segs = E >= kGroupThreads ? 1 : kGroupThreads / E;
  uint16_t* mx = reinterpret_cast<uint16_t*>(segpre + segs * E);  // [rows][E]
  const int rows = (int)((16384 / E) < kTokTile ? (16384 / E) : kTokTile);  // tokens per sub-tile
  const int64_t S = T * k;

  for (int e = tid; e < E; e += kGroupThreads) {
    cnt[e] = 0;
    carry[e] = 0;
  }
  __syncthreads();
  for (int64_t s = tid; s < S; s += kGroupThreads) atomicAdd(&cnt[clamp_id(ids[s], E)], 1);
  __syncthreads();
  if (tid == 0) {
    int32_t acc = 0, items = 0;
    for (int e = 0; e < E; ++e) {
      off[e] = acc;
      acc += cnt[e];
      for (int32_t m0 = 0; m0 < cnt[e] && items < max_items; m0 += kBM, ++items) {
        o.items[2 * items] = e;
        o.items[2 * items + 1] = m0;
      }
    }
    off[E] = acc;
    *o.nitems = items;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += kGroupThreads) {
    o.offsets[e] = off[e];
    if (e < E) o.counts[e] = cnt[e];
  }
  // position of slot (t, j) inside its expert's segment = number of earlier
  // tokens that chose the same expert: a column-wise exclusive scan of the
  // token x expert incidence matrix, one sub-tile of `rows` tokens at a time
  const int seg_rows = (rows + segs - 1) / segs;
  for (int64_t t0 = 0; t0 < T; t0 += rows) {
    const int nt = (int)((T - t0) < rows ? (T - t0) : rows);
    for (int i = tid; i < rows * E; i += kGroupThreads) mx[i] = 0;
    __syncthreads();
    for (int i = tid; i < nt * k; i += kGroupThreads) mx[(i / k) * E + clamp_id(ids[(t0 * k) + i], E)] = 1;
    __syncthreads();
    if (tid < segs * E) {
      const int e = tid % E, sg = tid / E;
      int32_t run = 0;
      const int r1 = (sg + 1) * seg_rows < nt ? (sg + 1) * seg_rows : nt;
      for (int r = sg * seg_rows; r < r1; ++r) {
        const int32_t v = mx[r * E + e];
        mx[r * E + e] = (uint16_t)run;
        run += v;
      }
      segpre[sg * E + e] = run;
    }
    __syncthreads();
    if (tid < E) {  // exclusive prefix of the segment totals, plus the carry
      int32_t acc = carry[tid];
      for (int sg = 0; sg < segs; ++sg) {
        const int32_t v = segpre[sg * E + tid];
        segpre[sg * E + tid] = acc;
        acc += v;
      }
      carry[tid] = acc;
    }
    __syncthreads();
    for (int i = tid; i < nt * k; i += kGroupThreads) {
      const int r = i / k;
      const int64_t slot = t0 * k + i;
      const int e = clamp_id(ids[slot], E);
      const int32_t pos = off[e] + segpre[(r / seg_rows) * E + e] + mx[r * E + e];
      o.perm[pos] = (int32_t)slot;
      o.inv[slot] = pos;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// 3./4. grouped INT3 GEMM (FC1 with SwiGLU epilogue, FC2 with route weights)
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t cvt_pk_rn(float a, float b) {
  const half2v h = half2v{(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// 3-bit code j (0..31) of a 96-bit little-endian stream held in d0, d1, d2.
template <int J>
__device__ __forceinline__ uint32_t code3(uint32_t d0, uint32_t d1, uint32_t d2) {
  constexpr int bit = 3 * J;
  if constexpr (bit + 3 <= 32) return (d0 >> bit) & 7u;
  else if constexpr (bit < 32) return __builtin_amdgcn_alignbit(d1, d0, bit) & 7u;
  else if constexpr (bit + 3 <= 64) return (d1 >> (bit - 32)) & 7u;
  else if constexpr (bit < 64) return __builtin_amdgcn_alignbit(d2, d1, bit - 32) & 7u;
  else return (d2 >> (bit - 64)) & 7u;
}

template <int J>
__device__ __forceinline__ void dequant_pairs(uint32_t d0, uint32_t d1, uint32_t d2, float s,
                                              uint32_t* out) {
  if constexpr (J < 32) {
    // (q - 4) * s is exact in fp32 (3-bit integer times an fp16 value), so the
    // packed conversion rounds once: fp16((q - 4) * s)
    const float a = ((float)code3<J>(d0, d1, d2) - 4.0f) * s;
    const float b = ((float)code3<J + 1>(d0, d1, d2) - 4.0f) * s;
    out[J / 2] = cvt_pk_rn(a, b);
    dequant_pairs<J + 2>(d0, d1, d2, s, out);
  }
}

struct MoeGemmArgs {
  const uint8_t* codes;    // [E][N][row_bytes]
  const __half* scales;    // [E][N][K/bs]
  const void* act;         // FC1: x fp16 [T][K]; FC2: h fp16 [T*k][K] (grouped order)
  int64_t N, K, row_bytes, nblk, bs;
  int top_k;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* items;
  const int32_t* nitems;
  const float* wts;        // FC2: routing weights per slot
  __half* h_out;           // FC1 output [T*k][N/2] (grouped order)
  float* slot_out;         // FC2 output [T*k][N] (slot order)
};

template <bool FC1>
__global__ void __launch_bounds__(256) qmoe_gemm(MoeGemmArgs g, int64_t tiles_n) {
  __shared__ __align__(16) _Float16 As[kBM * kPitch];
  __shared__ __align__(16) _Float16 Ws[kBN * kPitch];
  __shared__ int32_t arow[kBM];  // activation row index of each tile row (-1: none)

  const int64_t item = blockIdx.x / tiles_n;
  const int64_t nt = blockIdx.x % tiles_n;
  if (item >= *g.nitems) return;  // uniform for the workgroup
  const int e = g.items[2 * item];
  const int m0 = g.items[2 * item + 1];
  const int rows = min(kBM, g.counts[e] - m0);
  const int64_t seg0 = g.offsets[e] + m0;  // grouped position of tile row 0
  const int64_t n0 = nt * kBN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid < kBM) {
    int32_t r = -1;
    if (tid < rows) r = FC1 ? g.perm[seg0 + tid] / g.top_k : (int32_t)(seg0 + tid);
    arow[tid] = r;
  }
  __syncthreads();

  // staging: activations 32 rows x 128 halves (8 threads per row, 32 B each),
  // weights 64 rows x 48 bytes (4 threads per row, 12 B = 32 codes each)
  const int a_r = tid >> 3, a_c = (tid & 7) * 16;
  const int w_r = tid >> 2, w_q = tid & 3;
  const int32_t my_arow = arow[a_r];
  const int64_t wrow = n0 + w_r;
  const uint8_t* wsrc = g.codes + ((int64_t)e * g.N + wrow) * g.row_bytes;
  const __half* ssrc = g.scales + ((int64_t)e * g.N + wrow) * g.nblk;
  const _Float16* act = static_cast<const _Float16*>(g.act);

  u32x4 ra0, ra1;
  u32x3 rw;
  float rs;
  auto load_step = [&](int64_t k0) {
    ra0 = u32x4{0, 0, 0, 0};
    ra1 = u32x4{0, 0, 0, 0};
    if (my_arow >= 0 && k0 + a_c < g.K) {  // K is a multiple of 32: chunks are whole
      const u32x4* src = reinterpret_cast<const u32x4*>(act + (int64_t)my_arow * g.K + k0 + a_c);
      ra0 = src[0];
      ra1 = src[1];
    }
    rw = u32x3{0, 0, 0};
    rs = 0.0f;
    if (wrow < g.N && k0 + w_q * 32 < g.K) {
      rw = *reinterpret_cast<const u32x3*>(wsrc + (k0 / 8) * 3 + w_q * 12);
      rs = __half2float(ssrc[(k0 + w_q * 32) / g.bs]);
    }
  };
  auto store_step = [&]() {
    *reinterpret_cast<u32x4*>(&As[a_r * kPitch + a_c]) = ra0;
    *reinterpret_cast<u32x4*>(&As[a_r * kPitch + a_c + 8]) = ra1;
    uint32_t out[16];
    dequant_pairs<0>(rw.x, rw.y, rw.z, rs, out);
    uint32_t* dst = reinterpret_cast<uint32_t*>(&Ws[w_r * kPitch + w_q * 32]);
#pragma unroll
    for (int i = 0; i < 16; i += 4) *reinterpret_cast<u32x4*>(dst + i) = u32x4{out[i], out[i + 1], out[i + 2], out[i + 3]};
  };

  f32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
  const int fr = lane & 15, fk = (lane >> 4) * 8;
  load_step(0);
  store_step();
  __syncthreads();
  for (int64_t k0 = 0; k0 < g.K; k0 += kBK) {
    const bool more = k0 + kBK < g.K;
    if (more) load_step(k0 + kBK);
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
      const half8 b = *reinterpret_cast<const half8*>(&Ws[(wave * 16 + fr) * kPitch + kk + fk]);
      const half8 a0 = *reinterpret_cast<const half8*>(&As[fr * kPitch + kk + fk]);
      const half8 a1 = *reinterpret_cast<const half8*>(&As[(16 + fr) * kPitch + kk + fk]);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b, acc1, 0, 0, 0);
    }
    __syncthreads();
    if (more) {
      store_step();
      __syncthreads();
    }
  }

  // lane l holds rows 4(l/16) + r of each 16-row tile, column l%16
  const int64_t col = n0 + wave * 16 + (lane & 15);
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const f32x4 a = mt ? acc1 : acc0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = mt * 16 + 4 * (lane >> 4) + r;
      const float v = a[r];
      if (FC1) {
        // interleaved gate/up: even column = gate_i, odd column = up_i
        const float partner = __shfl_xor(v, 1);
        if ((lane & 1) == 0 && row < rows && col < g.N) {
          const float gt = v, up = partner;
          const float hv = gt / (1.0f + expf(-gt)) * up;
          g.h_out[(seg0 + row) * (g.N / 2) + col / 2] = __float2half_rn(hv);
        }
      } else {
        if (row < rows && col < g.N) {
          const int32_t slot = g.perm[seg0 + row];
          g.slot_out[(int64_t)slot * g.N + col] = g.wts[slot] * v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 5. combine
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) qmoe_combine(const float* __restrict__ slots, int64_t T,
                                                    int k, int64_t H, __half* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= T * H) return;
  const int64_t t = i / H, n = i % H;
  float acc = 0.0f;
  for (int j = 0; j < k; ++j) acc += slots[(t * k + j) * H + n];
  out[i] = __float2half_rn(acc);
}

// debug: h rows back in slot order
__global__ void qmoe_gather_h(const __half* __restrict__ h, const int32_t* __restrict__ inv,
                              int64_t S, int64_t I, __half* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= S * I) return;
  const int64_t slot = i / I, c = i % I;
  dst[i] = h[(int64_t)inv[slot] * I + c];
}

struct Ws {
  uint64_t ids, wts, counts, offsets, perm, inv, items, nitems, h, slots, total;
};

int64_t max_items(int64_t Tt, int k, int64_t E) {
  const int64_t S = Tt * k;
  return (S < E ? S : E) + (S + kBM - 1) / kBM;
}

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
  w.items = take(max_items(Tt, k, E) * 8);
  w.nitems = take(4);
  w.h = take(S * I * 2);
  w.slots = take(S * H * 4);
  w.total = o;
  return w;
}

}  // namespace

uint64_t qmoe_ws_bytes(const Sizes& s1, const Sizes& s2, int top_k, int64_t T) {
  if (T <= 0) return 0;
  return ws_layout(s1, s2, top_k, T).total;
}

hipError_t launch_qmoe(const Sizes& s1, const mnb_plan& p1, const Sizes& s2, const mnb_plan& p2,
                       int top_k, int64_t T, const uint16_t* x, const float* logits, uint16_t* out,
                       void* ws, hipStream_t st, const QmoeDebug* dbg) {
  const int64_t E = s1.E, H = s1.K, I = s2.K;
  const int k = top_k;
  // limits of these kernels (checked before any launch)
  if (E > kMaxE || k > 16 || H % 32 || I % 32) return hipErrorNotSupported;
  const Ws L = ws_layout(s1, s2, k, T);
  uint8_t* w = static_cast<uint8_t*>(ws);
  int32_t* ids = reinterpret_cast<int32_t*>(w + L.ids);
  float* wts = reinterpret_cast<float*>(w + L.wts);
  GroupOut go{reinterpret_cast<int32_t*>(w + L.counts), reinterpret_cast<int32_t*>(w + L.offsets),
              reinterpret_cast<int32_t*>(w + L.perm), reinterpret_cast<int32_t*>(w + L.inv),
              reinterpret_cast<int32_t*>(w + L.items), reinterpret_cast<int32_t*>(w + L.nitems)};
  __half* hbuf = reinterpret_cast<__half*>(w + L.h);
  float* slots = reinterpret_cast<float*>(w + L.slots);
  const int segs = E >= kGroupThreads ? 1 : kGroupThreads / (int)E;
  const int rows = (int)((16384 / E) < kTokTile ? (16384 / E) : kTokTile);
  const size_t group_lds = (size_t)(E + E + 1 + E + segs * E) * 4 + (size_t)rows * E * 2;

  for (int64_t t0 = 0; t0 < T; t0 += kTokTile) {
    const int64_t Tt = (T - t0) < kTokTile ? (T - t0) : kTokTile;
    const int64_t S = Tt * k;
    const int64_t items = max_items(Tt, k, E);
    hipLaunchKernelGGL(qmoe_route, dim3((unsigned)((Tt + 3) / 4)), dim3(256), 0, st,
                       logits + t0 * E, Tt, (int)E, k, ids, wts);
    hipLaunchKernelGGL(qmoe_group, dim3(1), dim3(kGroupThreads), group_lds, st, ids, Tt, k, (int)E,
                       items, go);
    MoeGemmArgs a1{static_cast<const uint8_t*>(p1.codes), static_cast<const __half*>(p1.scales),
                   x + t0 * H, s1.N, s1.K, s1.row_bytes, s1.nb, s1.bs, k,
                   go.counts, go.offsets, go.perm, go.items, go.nitems, wts, hbuf, nullptr};
    const int64_t nt1 = (s1.N + kBN - 1) / kBN;
    hipLaunchKernelGGL(qmoe_gemm<true>, dim3((unsigned)(items * nt1)), dim3(256), 0, st, a1, nt1);
    MoeGemmArgs a2{static_cast<const uint8_t*>(p2.codes), static_cast<const __half*>(p2.scales),
                   hbuf, s2.N, s2.K, s2.row_bytes, s2.nb, s2.bs, k,
                   go.counts, go.offsets, go.perm, go.items, go.nitems, wts, nullptr, slots};
    const int64_t nt2 = (s2.N + kBN - 1) / kBN;
    hipLaunchKernelGGL(qmoe_gemm<false>, dim3((unsigned)(items * nt2)), dim3(256), 0, st, a2, nt2);
    hipLaunchKernelGGL(qmoe_combine, dim3((unsigned)((Tt * H + 255) / 256)), dim3(256), 0, st,
                       slots, Tt, k, H, reinterpret_cast<__half*>(out + t0 * H));
    if (dbg) {
      if (dbg->ids)
        (void)hipMemcpyAsync(dbg->ids + t0 * k, ids, S * 4, hipMemcpyDeviceToDevice, st);
      if (dbg->w) (void)hipMemcpyAsync(dbg->w + t0 * k, wts, S * 4, hipMemcpyDeviceToDevice, st);
      if (dbg->slot)
        (void)hipMemcpyAsync(dbg->slot + t0 * k * H, slots, S * H * 4, hipMemcpyDeviceToDevice, st);
      if (dbg->h)
        hipLaunchKernelGGL(qmoe_gather_h, dim3((unsigned)((S * I + 255) / 256)), dim3(256), 0, st,
                           hbuf, go.inv, S, I, reinterpret_cast<__half*>(dbg->h + t0 * k * I));
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mnb
