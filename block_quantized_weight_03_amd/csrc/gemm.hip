// Small-M / prefill GEMM on the same compressed INT4 weights, for gfx950.
//
// Operation ("Qwen3 Missing-Kernel Implementation Plan", section "PR
// sequence", step K03: reuse the same compressed weights for short prompts
// and prefill, bounded workspace, partial blocks and output tails):
//   Y[m,n] = sum_{k<K} A[m,k] * (q[n,k] - z[n,b]) * s[n,b].
// A dense contraction, so it runs on the matrix cores: A is rounded to fp16
// (RN) as it is staged into LDS; each weight tile is dequantized once per
// workgroup into LDS as w = fp16(fma(q, s, -(z*s))) (for the implicit zero
// point 8 this is exactly fp16(fp32((q - 8) * s))); v_mfma_f32_32x32x16_f16
// accumulates in fp32.  Only a BN x 32 tile of the float weights ever
// exists, in LDS.
//
// Tiling.  A workgroup of 4 waves computes a BM x BN tile of Y; each wave a
// (BM/WAVES_M) x (BN/WAVES_N) sub-tile of 32 x 32 MFMA tiles whose
// accumulators live in AGPRs.  K advances 32 codes per step (one scale per
// row and step for block sizes 32/64/128).  Two LDS stages: while the MFMAs
// consume stage s, the global loads of step s+1 are in flight into
// registers, then converted into stage s+1; one barrier per step.  LDS rows
// are 64 bytes with the four 16-byte chunks of row r stored at chunk
// c ^ ((r >> 2) & 3), which makes the fragment reads conflict-free without
// padding.  Workgroups are numbered so that each XCD (workgroups are handed
// to the 8 XCDs round-robin) works on a contiguous range of tiles, keeping
// the A rows a range shares in that XCD's L2.  When the tile count is too
// small to fill the chip, K is split S ways; each split writes an fp32
// partial tile to the workspace and a second kernel sums the S partials in
// split order (deterministic).

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace mnb {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBK = 32;     // K per step (halves per LDS row)
constexpr int kXcds = 8;    // XCDs of an MI355X

__device__ __forceinline__ uint32_t cvt_pk_rn(float a, float b) {
  const half2v h = half2v{(_Float16)a, (_Float16)b};  // v_cvt_pk_f16_f32 (round to nearest even)
  return __builtin_bit_cast(uint32_t, h);
}

// half offset of 16-byte chunk c of LDS row r (swizzled)
__device__ __forceinline__ int lds_off(int r, int c) { return r * kBK + ((c ^ ((r >> 2) & 3)) << 3); }

template <int BM, int BN, int WAVES_M>
struct Cfg {
  static constexpr int WAVES_N = 4 / WAVES_M;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int A_PER = BM * kBK / 256;  // fp32 values of A per thread and step
  static constexpr int A_TPR = kBK / A_PER;     // threads per A row
  static constexpr int W_PER = BN * kBK / 256;  // codes per thread and step
  static constexpr int W_TPR = kBK / W_PER;     // threads per weight row
  static_assert(WAVES_M * WAVES_N == 4 && TM >= 1 && TN >= 1, "4 waves of 32x32 tiles");
  static_assert(A_PER % 4 == 0 && (W_PER == 16 || W_PER == 32), "staging shapes");
};

template <int BM, int BN, int WAVES_M, bool HAS_ZP>
__global__ void __launch_bounds__(256) gemm_int4_mfma(
    const float* __restrict__ A, const uint8_t* __restrict__ codes,
    const float* __restrict__ scales, const uint32_t* __restrict__ zeros, float* __restrict__ Y,
    float* __restrict__ part, int64_t M, int64_t N, int64_t K, int64_t row_bytes, int64_t nb,
    int32_t bs_shift, int64_t tiles_n, int64_t work, int32_t splits, int64_t kc) {
  using C = Cfg<BM, BN, WAVES_M>;
  __shared__ __align__(16) _Float16 As[2][BM * kBK];
  __shared__ __align__(16) _Float16 Ws[2][BN * kBK];

  // XCD-aware numbering: XCD x (= blockIdx % 8) takes work items
  // [x * per, (x + 1) * per)
  const int64_t per = (work + kXcds - 1) / kXcds;
  const int64_t L = (int64_t)(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (L >= work) return;  // whole workgroup
  const int split = (int)(L % splits);
  const int64_t tile = L / splits;
  const int64_t m0 = (tile / tiles_n) * BM;
  const int64_t n0 = (tile % tiles_n) * BN;
  const int64_t kbeg = split * kc;
  const int64_t kend = kbeg + kc < K ? kbeg + kc : K;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  // rows of A are 16-byte aligned: vector loads
  const bool a_vec = (K & 3) == 0 && (reinterpret_cast<uintptr_t>(A) & 15) == 0;

  // staging registers of one step
  float ra[C::A_PER];
  uint32_t rw[C::W_PER / 8];
  float rs = 0.0f, rz = 0.0f;
  const int a_row = tid / C::A_TPR, a_col = (tid % C::A_TPR) * C::A_PER;
  const int w_row = tid / C::W_TPR, w_col = (tid % C::W_TPR) * C::W_PER;
  const int64_t am = m0 + a_row, wn_row = n0 + w_row;
  const float* arow = A + am * K;
  const uint8_t* wrow = codes + wn_row * row_bytes;

  auto load_step = [&](int64_t k0) {
    const int64_t k = k0 + a_col;
    if (am < M && a_vec && k + C::A_PER <= K) {
#pragma unroll
      for (int i = 0; i < C::A_PER; i += 4) {
        const float4 v = *reinterpret_cast<const float4*>(arow + k + i);
        ra[i] = v.x;
        ra[i + 1] = v.y;
        ra[i + 2] = v.z;
        ra[i + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::A_PER; ++i) ra[i] = (am < M && k + i < K) ? arow[k + i] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < C::W_PER / 8; ++i) rw[i] = 0u;
    rs = 0.0f;
    rz = 8.0f;
    if (wn_row < N) {
      const int64_t sb = k0 >> 5;
      const int64_t b = sb >> bs_shift;
      const uint8_t* src = wrow + sb * 16 + w_col / 2;
      if (C::W_PER == 32) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(src);
        rw[0] = v.x;
        rw[1] = v.y;
        rw[2] = v.z;
        rw[3] = v.w;
      } else {
        const u32x2 v = *reinterpret_cast<const u32x2*>(src);
        rw[0] = v.x;
        rw[1] = v.y;
      }
      rs = scales[wn_row * nb + b];
      if (HAS_ZP) rz = (float)((zeros[(wn_row >> 3) * nb + b] >> (4 * (wn_row & 7))) & 15u);
    }
  };

  auto store_step = [&](int st) {
    // A: fp32 -> fp16 (RN)
    uint32_t pa[C::A_PER / 2];
#pragma unroll
    for (int i = 0; i < C::A_PER; i += 2) pa[i / 2] = cvt_pk_rn(ra[i], ra[i + 1]);
    _Float16* as = As[st];
#pragma unroll
    for (int c = 0; c < C::A_PER / 8; ++c)
      *reinterpret_cast<u32x4*>(&as[lds_off(a_row, a_col / 8 + c)]) =
          u32x4{pa[4 * c], pa[4 * c + 1], pa[4 * c + 2], pa[4 * c + 3]};
    if (C::A_PER % 8)  // 4 values: half a chunk
      *reinterpret_cast<u32x2*>(&as[lds_off(a_row, a_col / 8) + (a_col % 8)]) =
          u32x2{pa[0], pa[1]};
    // weights: stored nibbles are (q - 8); w = fp16(fma(q, s, -(z*s)))
    const float nzs = -(rz * rs);
    uint32_t pw[C::W_PER / 2];
#pragma unroll
    for (int i = 0; i < C::W_PER / 8; ++i) {
      const uint32_t x = rw[i] ^ 0x88888888u;
      const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float qa = (float)((lo >> (8 * j)) & 0xFFu);  // code 2j
        const float qb = (float)((hi >> (8 * j)) & 0xFFu);  // code 2j+1
        pw[4 * i + j] = cvt_pk_rn(fmaf(qa, rs, nzs), fmaf(qb, rs, nzs));
      }
    }
    _Float16* ws = Ws[st];
#pragma unroll
    for (int c = 0; c < C::W_PER / 8; ++c)
      *reinterpret_cast<u32x4*>(&ws[lds_off(w_row, w_col / 8 + c)]) =
          u32x4{pw[4 * c], pw[4 * c + 1], pw[4 * c + 2], pw[4 * c + 3]};
  };

  f32x16 acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int fr = lane & 31;   // fragment row (A) / column (B)
  const int fg = lane >> 5;   // which 8-value half of a 16-wide k slice

  int st = 0;
  if (kbeg < kend) {
    load_step(kbeg);
    store_step(0);
  }
  __syncthreads();
  for (int64_t k0 = kbeg; k0 < kend; k0 += kBK) {
    const bool more = k0 + kBK < kend;
    if (more) load_step(k0 + kBK);
    const _Float16* as = As[st];
    const _Float16* ws = Ws[st];
#pragma unroll
    for (int kk = 0; kk < kBK / 8; kk += 2) {
      half8 af[C::TM], bf[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
        af[i] = *reinterpret_cast<const half8*>(&as[lds_off(wm * C::WM + i * 32 + fr, kk + fg)]);
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        bf[j] = *reinterpret_cast<const half8*>(&ws[lds_off(wn * C::WN + j * 32 + fr, kk + fg)]);
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (more) store_step(st ^ 1);
    __syncthreads();
    st ^= 1;
  }

  // epilogue: lane l holds column l%32 and rows 8(r/4) + 4(l/32) + r%4
  float* out = splits > 1 ? part + (int64_t)split * M * N : Y;
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      const int64_t col = n0 + wn * C::WN + j * 32 + fr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * C::WM + i * 32 + 8 * (r >> 2) + 4 * fg + (r & 3);
        if (row < M && col < N) out[row * N + col] = acc[i][j][r];
      }
    }
}

// Fast path for K % 32 == 0: the same tiles and LDS layout, but a branch-free
// main loop whose global loads run two steps ahead (two register sets, the
// loop unrolled by two so the sets are static), and whose fp16 conversion of
// the next step is interleaved with the current step's MFMAs by scheduling
// groups.  Rows past M and columns past N read clamped (valid) addresses and
// produce results that are never stored.
template <int BM, int BN, int WAVES_M, bool HAS_ZP>
__global__ void __launch_bounds__(256) gemm_int4_fast(
    const float* __restrict__ A, const uint8_t* __restrict__ codes,
    const float* __restrict__ scales, const uint32_t* __restrict__ zeros, float* __restrict__ Y,
    float* __restrict__ part, int64_t M, int64_t N, int64_t K, int64_t row_bytes, int64_t nb,
    int32_t bs_shift, int64_t tiles_n, int64_t work, int32_t splits, int64_t kc) {
  using C = Cfg<BM, BN, WAVES_M>;
  constexpr int AP = BM / 32;   // float4 of A per thread and step (8 threads per row)
  constexpr int WW = C::W_PER / 8;  // 32-bit code words per thread and step
  extern __shared__ __align__(16) _Float16 smem[];
  _Float16* As0 = smem;
  _Float16* As1 = smem + BM * kBK;
  _Float16* Ws0 = smem + 2 * BM * kBK;
  _Float16* Ws1 = smem + 2 * BM * kBK + BN * kBK;

  const int64_t per = (work + kXcds - 1) / kXcds;
  const int64_t L = (int64_t)(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (L >= work) return;
  const int split = (int)(L % splits);
  const int64_t tile = L / splits;
  const int64_t m0 = (tile / tiles_n) * BM;
  const int64_t n0 = (tile % tiles_n) * BN;
  const int64_t kbeg = split * kc;
  const int64_t kend = kbeg + kc < K ? kbeg + kc : K;
  const int steps = (int)((kend - kbeg) / kBK);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

  // per-thread sources (clamped rows), as 32-bit element offsets from A
  // (the launcher guarantees M * K < 2^31)
  const int a_r = tid >> 3, a_c = (tid & 7) * 4;
  uint32_t aoff[AP];
#pragma unroll
  for (int p = 0; p < AP; ++p) {
    int64_t m = m0 + p * 32 + a_r;
    m = m < M ? m : M - 1;
    aoff[p] = (uint32_t)(m * K + a_c);
  }
  const int w_row = tid / C::W_TPR, w_col = (tid % C::W_TPR) * C::W_PER;
  int64_t wn_row = n0 + w_row;
  wn_row = wn_row < N ? wn_row : N - 1;
  const uint8_t* wsrc = codes + wn_row * row_bytes + w_col / 2;
  const float* ssrc = scales + wn_row * nb;
  const uint32_t* zsrc = HAS_ZP ? zeros + (wn_row >> 3) * nb : nullptr;
  const int zsh = 4 * (int)(wn_row & 7);

  float4 ra0[AP], ra1[AP];
  uint32_t rw0[WW], rw1[WW];
  float rs0, rs1, rz0 = 8.0f, rz1 = 8.0f;

  auto load = [&](float4 (&ra)[AP], uint32_t (&rw)[WW], float& rs, float& rz, int step) {
    const int st = step < steps ? step : steps - 1;  // past the end: harmless reload
    const int64_t k0 = kbeg + (int64_t)st * kBK;
#pragma unroll
    for (int p = 0; p < AP; ++p) ra[p] = *reinterpret_cast<const float4*>(A + aoff[p] + k0);
    const int64_t sb = k0 >> 5;
    if (WW == 4) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(wsrc + sb * 16);
      rw[0] = v.x;
      rw[1] = v.y;
      rw[2] = v.z;
      rw[3] = v.w;
    } else {
      const u32x2 v = *reinterpret_cast<const u32x2*>(wsrc + sb * 16);
      rw[0] = v.x;
      rw[1] = v.y;
    }
    const int64_t b = sb >> bs_shift;
    rs = ssrc[b];
    if (HAS_ZP) rz = (float)((zsrc[b] >> zsh) & 15u);
  };

  auto convert = [&](const float4 (&ra)[AP], const uint32_t (&rw)[WW], float rs, float rz,
                     _Float16* as, _Float16* ws) {
#pragma unroll
    for (int p = 0; p < AP; ++p) {
      const int r = p * 32 + a_r;
      *reinterpret_cast<u32x2*>(&as[lds_off(r, a_c >> 3) + (a_c & 7)]) =
          u32x2{cvt_pk_rn(ra[p].x, ra[p].y), cvt_pk_rn(ra[p].z, ra[p].w)};
    }
    const float nzs = -(rz * rs);
#pragma unroll
    for (int i = 0; i < WW; ++i) {
      const uint32_t x = rw[i] ^ 0x88888888u;
      const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
      uint32_t pw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        pw[j] = cvt_pk_rn(fmaf((float)((lo >> (8 * j)) & 0xFFu), rs, nzs),
                          fmaf((float)((hi >> (8 * j)) & 0xFFu), rs, nzs));
      *reinterpret_cast<u32x4*>(&ws[lds_off(w_row, (w_col >> 3) + i)]) =
          u32x4{pw[0], pw[1], pw[2], pw[3]};
    }
  };

  f32x16 acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int fr = lane & 31, fg = lane >> 5;
  auto compute = [&](const _Float16* as, const _Float16* ws) {
#pragma unroll
    for (int kk = 0; kk < kBK / 8; kk += 2) {
      half8 af[C::TM], bf[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
        af[i] = *reinterpret_cast<const half8*>(&as[lds_off(wm * C::WM + i * 32 + fr, kk + fg)]);
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        bf[j] = *reinterpret_cast<const half8*>(&ws[lds_off(wn * C::WN + j * 32 + fr, kk + fg)]);
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  };

  // interleave: each MFMA followed by a few VALU, LDS and global-memory ops
  auto schedule = [&]() {
    constexpr int kMfma = 2 * C::TM * C::TN;
#pragma unroll
    for (int i = 0; i < kMfma; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
    }
  };

  load(ra0, rw0, rs0, rz0, 0);
  load(ra1, rw1, rs1, rz1, 1);
  convert(ra0, rw0, rs0, rz0, As0, Ws0);
  __syncthreads();
  for (int s = 0; s < steps; s += 2) {
    // even step s: data of step s+1 is in set 1; loads of step s+2 go to set 0
    load(ra0, rw0, rs0, rz0, s + 2);
    compute(As0, Ws0);
    if (s + 1 < steps) convert(ra1, rw1, rs1, rz1, As1, Ws1);
    schedule();
    __syncthreads();
    if (s + 1 >= steps) break;
    // odd step s+1: data of step s+2 is in set 0; loads of step s+3 go to set 1
    load(ra1, rw1, rs1, rz1, s + 3);
    compute(As1, Ws1);
    if (s + 2 < steps) convert(ra0, rw0, rs0, rz0, As0, Ws0);
    schedule();
    __syncthreads();
  }

  float* out = splits > 1 ? part + (int64_t)split * M * N : Y;
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      const int64_t col = n0 + wn * C::WN + j * 32 + fr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * C::WM + i * 32 + 8 * (r >> 2) + 4 * fg + (r & 3);
        if (row < M && col < N) out[row * N + col] = acc[i][j][r];
      }
    }
}

// Y = sum over the S partials, in split order.
__global__ void __launch_bounds__(256) gemm_splitk_reduce(const float* __restrict__ part,
                                                          float* __restrict__ Y, int64_t MN,
                                                          int32_t splits) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= MN) return;
  float acc = part[i];
  for (int s = 1; s < splits; ++s) acc += part[(int64_t)s * MN + i];
  Y[i] = acc;
}

int bs_shift_of(const Sizes& s) { return s.bs == 32 ? 0 : (s.bs == 64 ? 1 : 2); }

bool fast_ok(const Sizes& s, int64_t M, const void* A) {
  return (s.K % kBK) == 0 && (reinterpret_cast<uintptr_t>(A) & 15) == 0 &&
         (uint64_t)M * (uint64_t)s.K < (1ull << 31);
}

struct Plan {
  bool lds;         // the LDS-streaming kernel (gemm_lds.hip), bm x (128 tn) tiles
  int bm, tn;
  int64_t n_split;  // > 0: 256 x 256 tiles below this column, 256 x 128 above
  int cfg;          // else: index into the configuration table below
  int64_t tiles_n, tiles;
  int32_t splits;
  int64_t kc;       // K per split (multiple of the kernel's K step)
};

struct CfgDesc {
  int bm, bn;
};
constexpr CfgDesc kCfgs[] = {{256, 256}, {128, 256}, {128, 128}, {64, 256}, {32, 256}};

constexpr int64_t kTargetWork = 256;                 // workgroups wanted (one per CU)
constexpr uint64_t kMaxPartialBytes = 64ull << 20;  // split-K workspace bound

// Splits K so that tiles * splits reaches about one workgroup per CU, with at
// least 8 steps of `step` codes per split and a bounded partial workspace.
// With `fit` (the LDS-streaming kernel) tiles * splits stays within one
// workgroup per CU, except that a long K (each of two splits keeping at least
// 32 steps) is split in two even where that exceeds it: measured on the K =
// 2048 / 6144 prefill shapes, rounding the split count up put a second
// workgroup on some CUs and cost 13-17% at M = 384 and 9-13% at M = 640-896
// (K = 6144), while no split at M = 1152-1280, K = 6144 cost 3-5%.
void split_k(Plan& p, const Sizes& s, int64_t M, int64_t step, bool fit = false) {
  const int64_t ksteps = (s.K + step - 1) / step;
  int64_t S = 1;
  if (p.tiles < kTargetWork * 3 / 4) {
    S = (kTargetWork + p.tiles - 1) / p.tiles;
    if (fit) {
      S = kTargetWork / p.tiles;
      if (S == 1 && ksteps >= 64) S = 2;
    }
    const int64_t max_by_k = ksteps / 8 > 1 ? ksteps / 8 : 1;
    if (S > max_by_k) S = max_by_k;
    while (S > 1 && (uint64_t)S * (uint64_t)M * (uint64_t)s.N * 4 > kMaxPartialBytes) --S;
  }
  const int64_t steps_per = (ksteps + S - 1) / S;
  p.splits = (int32_t)((ksteps + steps_per - 1) / steps_per);  // no empty split
  p.kc = steps_per * step;
}

// rows of A from which the LDS-streaming kernel is used (its 128-row tiles
// clamp the rows past M; from M = 64 it measured faster than the register-
// staged kernels: M = 64 / 96 / 127 at K = 2048, N = 6144 19.4 / 23.8 / 25.1
// -> 16.7 / 19.0 / 20.5 us, at K = 6144, N = 2048 17.6 / 19.1 / 20.7 -> 15.6 /
// 16.1 / 21.0 us; below 64 it was slower at K = 6144, but from M = 40 faster
// at K = 2048: M = 40 / 48 / 56 16.6 / 17.3 / 19.1 -> 15.9 / 16.2 / 16.5 us,
// so K <= 2048 takes it from kLdsMinShortK); it takes 128 x 128
// tiles while they number at most kLds128MaxTiles (one and a half rounds of
// two workgroups per CU: measured faster than 256 x 256 tiles up to there),
// else 256 x 256 tiles
constexpr int64_t kLdsMinM = 64;
constexpr int64_t kLdsMinShortK = 40;
constexpr int64_t kLds128MaxTiles = 384;

// Columns covered by 256 x 256 tiles when the rest take 256 x 128 ones, so
// that the wide tiles number at most one per CU and the two widths together
// take about two rounds (the launch interleaves them in its dispatch order;
// 0: one tile shape).  Used when 256 x 256 tiles alone would
// need between one and two rounds with an idle remainder: at M = 4096, K =
// 2048, N = 6144 (384 such tiles) 256 wide tiles plus 256 narrow ones took
// 127 against 135 us.
int64_t mixed_split(const Sizes& s, int64_t M) {
  const int64_t rows = (M + 255) / 256, cols = (s.N + 255) / 256;
  const int64_t tiles = rows * cols;
  // Too few 256 x 256 tiles for one per CU, and 256 x 128 tiles alone would
  // need a second, mostly idle round: as many wide column blocks as make
  // both widths fit one round (M = 1536, N = 6144: 36 wide and 216 narrow
  // tiles, 65.6 us against 82.1 us for 288 narrow ones).
  if (tiles < kTargetWork * 3 / 4 && 2 * tiles > kTargetWork) {
    const int64_t w = 2 * cols - kTargetWork / rows;
    return w >= 1 && w < cols ? w * 256 : 0;
  }
  if (tiles <= kTargetWork || tiles >= 2 * kTargetWork) return 0;
  const int64_t wide = kTargetWork / rows;  // 256-column blocks in the first round
  if (wide < 1 || wide >= cols) return 0;
  return wide * 256;
}

Plan choose(const Sizes& s, int64_t M, bool fast) {
  const int64_t N = s.N, K = s.K;
  (void)K;
  if (fast && M >= (s.K <= 2048 ? kLdsMinShortK : kLdsMinM) && gemm_lds_supported(s, M)) {
    Plan p;
    p.lds = true;
    const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
    const int64_t narrow1 = ((M + 255) / 256) * ((N + 127) / 128);
    // 128 x 128 tiles up to kLds128MaxTiles, except where they would exceed
    // one per CU while 256 x 128 tiles fill three quarters of the chip or
    // more in one round (M = 1024, K = 2048, N = 6144: 43.8 -> 41.3 us;
    // M = 3072, K = 6144, N = 2048: 128.3 -> 117.5 us)
    const bool narrow_round = t128 > kTargetWork && narrow1 >= kTargetWork * 3 / 4 && narrow1 <= kTargetWork;
    // 256 x 256 tiles just over one per CU (by at most an eighth) leave the
    // rest for a second, mostly idle round whatever the mix; 128 x 128 tiles
    // spread it finer (M = 2688 / 2816, K = 2048, N = 6144, 264 such tiles:
    // 119.9 / 118.5 -> 97.1 / 113.0 us; 288 tiles at M = 3072: equal)
    const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
    const bool wide_spill = t256 > kTargetWork && t256 <= kTargetWork * 9 / 8;
    p.bm = (t128 <= kLds128MaxTiles && !narrow_round) || wide_spill ? 128 : 256;
    p.tn = p.bm / 128;
    p.cfg = -1;
    p.tiles_n = (N + p.bm - 1) / p.bm;
    p.tiles = ((M + p.bm - 1) / p.bm) * p.tiles_n;
    p.n_split = p.bm == 256 ? mixed_split(s, M) : 0;
    if (p.n_split > 0) {  // no split of K: the tiles already fill the chip
      p.splits = 1;
      p.kc = s.K;
      return p;
    }
    // too few 256 x 256 tiles for the chip, enough 256 x 128 ones: those,
    // over the whole of K, instead of splitting K (no partials, no reduce;
    // at M = 4096, K = 6144, N = 2048: 256 narrow tiles against 128 wide
    // tiles split in two)
    if (p.bm == 256 && p.tiles < kTargetWork * 3 / 4 && narrow1 >= kTargetWork * 3 / 4) {
      p.tn = 1;
      p.tiles_n = (N + 127) / 128;
      p.tiles = narrow1;
      p.splits = 1;
      p.kc = s.K;
      return p;
    }
    split_k(p, s, M, 64, true);
    return p;
  }
  auto tiles_of = [&](int c) {
    return ((M + kCfgs[c].bm - 1) / kCfgs[c].bm) * ((N + kCfgs[c].bn - 1) / kCfgs[c].bn);
  };
  int c;
  if (M <= 32)
    c = 4;
  else if (M <= 64)
    c = 3;
  else if (M <= 128)
    c = 2;
  else {
    c = 2;
    for (int cand : {0, 1, 2})
      if ((!fast || cand != 0) && tiles_of(cand) >= kTargetWork * 3 / 4) {
        c = cand;
        break;
      }
  }
  Plan p;
  p.lds = false;
  p.bm = 0;
  p.tn = 0;
  p.n_split = 0;
  p.cfg = c;
  p.tiles_n = (N + kCfgs[c].bn - 1) / kCfgs[c].bn;
  p.tiles = tiles_of(c);
  split_k(p, s, M, kBK);
  return p;
}

uint64_t plan_ws_bytes(const Plan& p, const Sizes& s, int64_t M) {
  uint64_t b = p.splits > 1 ? align256((uint64_t)p.splits * (uint64_t)M * (uint64_t)s.N * 4) : 0;
  if (p.lds) b += gemm_lds_a16_bytes(s, M);
  return b;
}

template <int BM, int BN, int WAVES_M>
hipError_t launch_cfg(const Sizes& s, const mnb_plan& p, const Plan& pl, int64_t M, const float* A,
                      float* Y, float* part, hipStream_t st) {
  const int64_t work = pl.tiles * pl.splits;
  const int64_t blocks = (work + kXcds - 1) / kXcds * kXcds;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  // the 256x256 tile does not fit the fast kernel's register budget (it would
  // spill), so the plan never selects it when the fast kernel applies
  if constexpr (BM * BN <= 128 * 256) if (fast_ok(s, M, A)) {
    const size_t lds = (size_t)2 * (BM + BN) * kBK * sizeof(_Float16);
    if (s.zeros)
      hipLaunchKernelGGL((gemm_int4_fast<BM, BN, WAVES_M, true>), dim3((unsigned)blocks), dim3(256),
                         lds, st, A, static_cast<const uint8_t*>(p.codes),
                         static_cast<const float*>(p.scales), static_cast<const uint32_t*>(p.zeros),
                         Y, part, M, s.N, s.K, s.row_bytes, s.nb, bs_shift_of(s), pl.tiles_n, work,
                         pl.splits, pl.kc);
    else
      hipLaunchKernelGGL((gemm_int4_fast<BM, BN, WAVES_M, false>), dim3((unsigned)blocks), dim3(256),
                         lds, st, A, static_cast<const uint8_t*>(p.codes),
                         static_cast<const float*>(p.scales), nullptr, Y, part, M, s.N, s.K,
                         s.row_bytes, s.nb, bs_shift_of(s), pl.tiles_n, work, pl.splits, pl.kc);
    return hipGetLastError();
  }
  if (s.zeros)
    hipLaunchKernelGGL((gemm_int4_mfma<BM, BN, WAVES_M, true>), dim3((unsigned)blocks), dim3(256),
                       0, st, A, static_cast<const uint8_t*>(p.codes),
                       static_cast<const float*>(p.scales), static_cast<const uint32_t*>(p.zeros),
                       Y, part, M, s.N, s.K, s.row_bytes, s.nb, bs_shift_of(s), pl.tiles_n, work,
                       pl.splits, pl.kc);
  else
    hipLaunchKernelGGL((gemm_int4_mfma<BM, BN, WAVES_M, false>), dim3((unsigned)blocks), dim3(256),
                       0, st, A, static_cast<const uint8_t*>(p.codes),
                       static_cast<const float*>(p.scales), nullptr, Y, part, M, s.N, s.K,
                       s.row_bytes, s.nb, bs_shift_of(s), pl.tiles_n, work, pl.splits, pl.kc);
  return hipGetLastError();
}

}  // namespace

uint64_t gemm_ws_bytes(const Sizes& s, int64_t M) {
  if (M <= 0) return 0;
  // the plan may differ between the fast and the general kernel: size for both
  const uint64_t bf = plan_ws_bytes(choose(s, M, true), s, M);
  const uint64_t bg = plan_ws_bytes(choose(s, M, false), s, M);
  return bf > bg ? bf : bg;
}

hipError_t launch_gemm(const Sizes& s, const mnb_plan& p, int64_t M, const float* A, float* Y,
                       void* ws, hipStream_t st) {
  if (gemm_small_supported(s, M, A)) return launch_gemm_small(s, p, M, A, Y, st);
  const Plan pl = choose(s, M, fast_ok(s, M, A));
  hipError_t e;
  if (pl.lds) {
    // workspace: [fp16 copy of A][split partials]
    float* part = pl.splits > 1
                      ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) +
                                                 gemm_lds_a16_bytes(s, M))
                      : nullptr;
    e = launch_gemm_lds(s, p, M, A, ws, Y, part, pl.splits, pl.kc, pl.bm, pl.tn, pl.n_split, st);
    if (e != hipSuccess || pl.splits == 1) return e;
    const int64_t MN = M * s.N;
    hipLaunchKernelGGL(gemm_splitk_reduce, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, st,
                       static_cast<const float*>(part), Y, MN, pl.splits);
    return hipGetLastError();
  }
  float* part = pl.splits > 1 ? static_cast<float*>(ws) : nullptr;
  switch (pl.cfg) {
    case 0: e = launch_cfg<256, 256, 2>(s, p, pl, M, A, Y, part, st); break;
    case 1: e = launch_cfg<128, 256, 2>(s, p, pl, M, A, Y, part, st); break;
    case 2: e = launch_cfg<128, 128, 2>(s, p, pl, M, A, Y, part, st); break;
    case 3: e = launch_cfg<64, 256, 1>(s, p, pl, M, A, Y, part, st); break;
    default: e = launch_cfg<32, 256, 1>(s, p, pl, M, A, Y, part, st); break;
  }
  if (e != hipSuccess || pl.splits == 1) return e;
  const int64_t MN = M * s.N;
  hipLaunchKernelGGL(gemm_splitk_reduce, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, st,
                     static_cast<const float*>(part), Y, MN, pl.splits);
  return hipGetLastError();
}

}  // namespace mnb
