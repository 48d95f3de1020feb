// Small-M / prefill GEMM on the same compressed INT4 weights, for gfx950.
//
// Operation ("Qwen3 Missing-Kernel Implementation Plan", section "PR
// sequence", step K03: reuse the same compressed weights for short prompts
// and prefill, bounded workspace, partial blocks and output tails):
//   Y[m,n] = sum_{k<K} A[m,k] * (q[n,k] - z[n,b]) * s[n,b].
// This is a dense contraction, so it runs on the matrix cores: A is rounded
// to fp16 (RN) while it is staged into LDS, each weight tile is dequantized
// once per workgroup into LDS as fp16(fp32((q - z) * s)), and
// v_mfma_f32_32x32x16_f16 accumulates in fp32.  The float weight matrix is
// never formed: only a BN x 32 tile of it exists at a time, in LDS.
//
// Tiling.  A workgroup of 4 waves computes a BM x BN tile of Y; each wave a
// WM x WN sub-tile made of (WM/32) x (WN/32) MFMA tiles.  K advances in steps
// of 32 (one 32-code sub-block, so one scale per row and step for block sizes
// 32/64/128).  Global loads of the next step are issued into registers before
// the current step's MFMAs (register-staged double buffering).  Rows and
// columns past M / N and positions past K are masked; pad codes meet zero
// activations.

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace mnb {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBK = 32;        // K per step
constexpr int kPitch = 40;     // LDS row pitch in halves (32 + 8): conflict-free fragment reads

__device__ __forceinline__ uint32_t cvt_pk_rn(float a, float b) {
  const half2v h = half2v{(_Float16)a, (_Float16)b};  // v_cvt_pk_f16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}

template <int BM, int BN, int WM, int WN>
struct Cfg {
  static constexpr int WAVES_N = BN / WN;
  static constexpr int WAVES_M = BM / WM;
  static_assert(WAVES_N * WAVES_M == 4, "4 waves per workgroup");
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int A_PASSES = BM / 32;     // 8 threads per A row, 32 rows per pass
  static constexpr int W_PASSES = BN / 128;    // 2 threads per W row, 128 rows per pass
  static_assert(BN % 128 == 0, "BN multiple of 128");
};

template <int BM, int BN, int WM, int WN, bool HAS_ZP>
__global__ void __launch_bounds__(256) gemm_int4_mfma(
    const float* __restrict__ A, const uint8_t* __restrict__ codes,
    const float* __restrict__ scales, const uint32_t* __restrict__ zeros, float* __restrict__ Y,
    int64_t M, int64_t N, int64_t K, int64_t row_bytes, int64_t nb, int32_t bs_shift,
    int64_t tiles_n) {
  using C = Cfg<BM, BN, WM, WN>;
  __shared__ __align__(16) _Float16 As[BM * kPitch];
  __shared__ __align__(16) _Float16 Ws[BN * kPitch];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int64_t tile = blockIdx.x;
  const int64_t m0 = (tile / tiles_n) * BM;
  const int64_t n0 = (tile % tiles_n) * BN;
  const bool a_vec = (K & 3) == 0;  // rows of A 16-byte aligned

  // ---- staging registers -----------------------------------------------
  float4 ra[C::A_PASSES];
  u32x2 rw[C::W_PASSES];
  float rs[C::W_PASSES];
  int rz[C::W_PASSES];

  const int a_row = tid >> 3, a_col = (tid & 7) * 4;
  const int w_row = tid >> 1, w_half = tid & 1;

  auto load_step = [&](int64_t k0) {
#pragma unroll
    for (int p = 0; p < C::A_PASSES; ++p) {
      const int64_t m = m0 + p * 32 + a_row;
      const int64_t k = k0 + a_col;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (m < M) {
        const float* src = A + m * K + k;
        if (a_vec && k + 3 < K) {
          v = *reinterpret_cast<const float4*>(src);
        } else {
          if (k + 0 < K) v.x = src[0];
          if (k + 1 < K) v.y = src[1];
          if (k + 2 < K) v.z = src[2];
          if (k + 3 < K) v.w = src[3];
        }
      }
      ra[p] = v;
    }
    const int64_t sb = k0 >> 5;
    const int64_t b = sb >> bs_shift;
#pragma unroll
    for (int p = 0; p < C::W_PASSES; ++p) {
      const int64_t n = n0 + p * 128 + w_row;
      rw[p] = u32x2{0u, 0u};
      rs[p] = 0.0f;
      rz[p] = 8;
      if (n < N) {
        rw[p] = *reinterpret_cast<const u32x2*>(codes + n * row_bytes + sb * 16 + w_half * 8);
        rs[p] = scales[n * nb + b];
        if (HAS_ZP) rz[p] = (int)((zeros[(n >> 3) * nb + b] >> (4 * (n & 7))) & 15u);
      }
    }
  };

  auto store_step = [&]() {
#pragma unroll
    for (int p = 0; p < C::A_PASSES; ++p) {
      const uint32_t lo = cvt_pk_rn(ra[p].x, ra[p].y), hi = cvt_pk_rn(ra[p].z, ra[p].w);
      *reinterpret_cast<u32x2*>(&As[(p * 32 + a_row) * kPitch + a_col]) = u32x2{lo, hi};
    }
#pragma unroll
    for (int p = 0; p < C::W_PASSES; ++p) {
      // stored nibbles are (q - 8) two's complement; XOR 8 gives q
      const uint32_t x0 = rw[p].x ^ 0x88888888u, x1 = rw[p].y ^ 0x88888888u;
      const float zf = (float)rz[p], s = rs[p];
      uint32_t out[8];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t x = h ? x1 : x0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // codes 2j (low nibble) and 2j+1 (high nibble) of byte j
          const float qa = (float)((x >> (8 * j)) & 15u);
          const float qb = (float)((x >> (8 * j + 4)) & 15u);
          out[h * 4 + j] = cvt_pk_rn((qa - zf) * s, (qb - zf) * s);
        }
      }
      uint32_t* dst = reinterpret_cast<uint32_t*>(&Ws[(p * 128 + w_row) * kPitch + w_half * 16]);
#pragma unroll
      for (int i = 0; i < 8; i += 4)
        *reinterpret_cast<u32x4*>(dst + i) = u32x4{out[i], out[i + 1], out[i + 2], out[i + 3]};
    }
  };

  f32x16 acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int fr = lane & 31;          // fragment row (A) / column (B)
  const int fk = (lane >> 5) * 8;    // k offset of this lane's 8 values

  load_step(0);
  store_step();
  __syncthreads();
  for (int64_t k0 = 0; k0 < K; k0 += kBK) {
    const bool more = k0 + kBK < K;
    if (more) load_step(k0 + kBK);
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 16) {
      half8 af[C::TM], bf[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
        af[i] = *reinterpret_cast<const half8*>(&As[(wm * WM + i * 32 + fr) * kPitch + kk + fk]);
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        bf[j] = *reinterpret_cast<const half8*>(&Ws[(wn * WN + j * 32 + fr) * kPitch + kk + fk]);
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
    if (more) {
      store_step();
      __syncthreads();
    }
  }

  // ---- epilogue: lane l holds column l%32 and rows 8(r/4) + 4(l/32) + r%4
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      const int64_t col = n0 + wn * WN + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < M && col < N) Y[row * N + col] = acc[i][j][r];
      }
    }
}

int bs_shift_of(const Sizes& s) { return s.bs == 32 ? 0 : (s.bs == 64 ? 1 : 2); }

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const Sizes& s, const mnb_plan& p, int64_t M, const float* A, float* Y,
                      hipStream_t st) {
  const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (s.N + BN - 1) / BN;
  const int64_t blocks = tiles_m * tiles_n;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (s.zeros)
    hipLaunchKernelGGL((gemm_int4_mfma<BM, BN, WM, WN, true>), dim3((unsigned)blocks), dim3(256),
                       0, st, A, static_cast<const uint8_t*>(p.codes),
                       static_cast<const float*>(p.scales), static_cast<const uint32_t*>(p.zeros),
                       Y, M, s.N, s.K, s.row_bytes, s.nb, bs_shift_of(s), tiles_n);
  else
    hipLaunchKernelGGL((gemm_int4_mfma<BM, BN, WM, WN, false>), dim3((unsigned)blocks), dim3(256),
                       0, st, A, static_cast<const uint8_t*>(p.codes),
                       static_cast<const float*>(p.scales), nullptr, Y, M, s.N, s.K, s.row_bytes,
                       s.nb, bs_shift_of(s), tiles_n);
  return hipGetLastError();
}

}  // namespace

uint64_t gemm_ws_bytes(const Sizes&, int64_t) { return 0; }

hipError_t launch_gemm(const Sizes& s, const mnb_plan& p, int64_t M, const float* A, float* Y,
                       void*, hipStream_t st) {
  if (M <= 32) return launch_cfg<32, 256, 32, 64>(s, p, M, A, Y, st);
  if (M <= 64) return launch_cfg<64, 256, 64, 64>(s, p, M, A, Y, st);
  if (M <= 128) return launch_cfg<128, 128, 64, 64>(s, p, M, A, Y, st);
  return launch_cfg<256, 128, 128, 64>(s, p, M, A, Y, st);
}

}  // namespace mnb
