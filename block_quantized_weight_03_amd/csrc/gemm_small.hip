// Small-M GEMM (M <= 32) on dense INT4 weights for gfx950: one launch, no
// workspace (used for M <= 4, or M <= 32 with N >= 4096; see
// gemm_small_supported).
//
// Operation ("Qwen3 Missing-Kernel Implementation Plan", section "PR
// sequence", step K03, small-M/prefill on the same compressed weights):
//   Y[m,n] = sum_{k<K} A[m,k] * (q[n,k] - z[n,b]) * s[n,b],  b = k / bs,
// with the rounding chain of the other matrix-core paths: A rounded to fp16,
// each weight rounded once as fp16(fma(q, s, -(z*s))) from fp32, products
// accumulated in fp32.
//
// At M <= 32 the product is a stream over the weights that must keep enough
// bytes in flight to cover HBM latency.  A workgroup owns one 16-row weight
// tile; its W waves split the 128-code K chunks into contiguous ranges, and
// each wave issues the 16-byte loads of all its chunks before it uses the
// first, so the whole weight matrix is in flight at once.  Lane (r, g) =
// (lane & 15, lane >> 4) takes 32-code block 4c + g of row r in chunk c, and
// the activations of token r at the same 32 k straight from L2 into its MFMA
// operand (fp32 -> fp16 in registers, one chunk ahead): each A chunk is used
// by one wave of the workgroup, so staging it in LDS would buy no reuse.  The
// W partial 16 x 16 tiles are summed in LDS in a fixed order, so there is no
// A pre-pass, no split partial in HBM and no reduction launch.

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace mnb {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t pk_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, half2v{(_Float16)a, (_Float16)b});  // v_cvt_pk_f16_f32, RNE
}

// 8 activations (two float4) as one fp16 MFMA operand
__device__ __forceinline__ half8 a_operand(const f32x4 x, const f32x4 y) {
  return __builtin_bit_cast(half8, u32x4{pk_f16(x.x, x.y), pk_f16(x.z, x.w), pk_f16(y.x, y.y),
                                         pk_f16(y.z, y.w)});
}

// 8 codes of one 32-bit word of the prepared layout (nibble j = (q - 8) in
// two's complement, even k in the low nibble) as fp16(fma(q, s, -(z s))),
// in k order
__device__ __forceinline__ half8 w_operand(uint32_t word, float s, float nzs) {
  const uint32_t x = word ^ 0x88888888u;  // back to q
  const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
  uint32_t p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    p[j] = pk_f16(fmaf((float)((lo >> (8 * j)) & 0xFFu), s, nzs),
                  fmaf((float)((hi >> (8 * j)) & 0xFFu), s, nzs));
  return __builtin_bit_cast(half8, u32x4{p[0], p[1], p[2], p[3]});
}

// CPW: chunks per wave (at least ceil(nch / W); extra slots reload the last
// chunk of the range and are not used); RT: 16-row weight tiles per
// workgroup, each wave computing all of them so that one A load feeds RT
// MFMAs; TT: 16-token tiles (M <= 16 TT), each dequantized weight operand
// feeding TT MFMAs.  K % 128 == 0.
template <int CPW, int W, int RT, bool HAS_ZP, int TT>
__global__ void __launch_bounds__(64 * W) gemm_int4_small(
    const float* __restrict__ A, const uint8_t* __restrict__ codes,
    const float* __restrict__ scales, const uint32_t* __restrict__ zeros, float* __restrict__ Y,
    int32_t M, int32_t N, int32_t K, int64_t row_bytes, int64_t nb, int32_t bs_shift) {
  __shared__ f32x4 red[W][TT * RT][64];
  const int lane = (int)(threadIdx.x & 63);
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int n0 = (int)blockIdx.x * 16 * RT;
  const int nch = K >> 7;
  const int c_beg = nch * wave / W, c_end = nch * (wave + 1) / W;
  const int cnt = c_end - c_beg;  // wave-uniform, <= CPW
  const int r = lane & 15, g = lane >> 4;

  // every chunk of the range in flight before the first is used (clamped:
  // a wave with no chunk reloads chunk 0 and adds nothing); rows past N
  // compute a copy of the last row (not stored)
  u32x4 wq[RT][CPW];
  float sc[RT][CPW], nz[RT][CPW];
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const int row = min(n0 + 16 * t + r, N - 1);
    const uint8_t* wrow = codes + (int64_t)row * row_bytes;
    const float* srow = scales + (int64_t)row * nb;
    const uint32_t* zrow = HAS_ZP ? zeros + (int64_t)(row >> 3) * nb : nullptr;
    const int zsh = 4 * (row & 7);
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      int c = c_beg + u;
      c = c < c_end ? c : c_end - 1;
      c = c < 0 ? 0 : c;
      const int G = 4 * c + g;  // 32-code block index along the row
      wq[t][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow + (int64_t)G * 16));
      const int b = G >> bs_shift;
      sc[t][u] = __builtin_nontemporal_load(srow + b);
      nz[t][u] = HAS_ZP ? (float)((__builtin_nontemporal_load(zrow + b) >> zsh) & 15u) : 8.0f;
    }
  }
  // token row of lane r in token tile tt (tokens past M compute a copy of
  // the last one, not stored)
  const float* arow[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) arow[tt] = A + (int64_t)min(16 * tt + r, M - 1) * K + 32 * g;
  f32x4 a0[TT][8], a1[TT][8];
  auto load_a = [&](f32x4 (&a)[TT][8], int u) {
    int c = c_beg + u;
    c = c < c_end ? c : c_end - 1;
    c = c < 0 ? 0 : c;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const f32x4* src = reinterpret_cast<const f32x4*>(arow[tt] + 128 * c);
#pragma unroll
      for (int i = 0; i < 8; ++i) a[tt][i] = src[i];
    }
  };
  f32x4 acc[TT][RT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[tt][t] = f32x4{0, 0, 0, 0};
  auto chunk = [&](const f32x4 (&a)[TT][8], int u) {
    half8 ao[TT][4];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) ao[tt][i] = a_operand(a[tt][2 * i], a[tt][2 * i + 1]);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const float s = sc[t][u], nzs = -(nz[t][u] * s);
      const u32x4 w = wq[t][u];
      const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
      // MFMA i takes k = 32 g + 8 i + [0, 8) in lane group g on both sides
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const half8 wo = w_operand(wv[i], s, nzs);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          acc[tt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ao[tt][i], wo, acc[tt][t], 0, 0, 0);
      }
    }
  };
  load_a(a0, 0);
#pragma unroll
  for (int u = 0; u < CPW; u += 2) {
    if (u < cnt) {
      if (u + 1 < cnt) load_a(a1, u + 1);
      chunk(a0, u);
    }
    if (u + 1 < CPW && u + 1 < cnt) {
      if (u + 2 < cnt) load_a(a0, u + 2);
      chunk(a1, u + 1);
    }
  }
  // lane l holds tokens 16 tt + 4 (l >> 4) + i of weight row n0 + 16 t + (l & 15)
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int t = 0; t < RT; ++t) red[wave][tt * RT + t][lane] = acc[tt][t];
  __syncthreads();
  if (wave < TT * RT) {  // wave j sums tile j = (tt, t) over the waves, in wave order
    const int j = wave, tt = j / RT, t = j % RT;
    f32x4 o = red[0][j][lane];
#pragma unroll
    for (int w = 1; w < W; ++w) {
      const f32x4 v = red[w][j][lane];
      o = f32x4{o.x + v.x, o.y + v.y, o.z + v.z, o.w + v.w};
    }
    const int n = n0 + 16 * t + r;
    if (n < N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * tt + 4 * g + i;
        if (m < M) Y[(int64_t)m * N + n] = o[i];
      }
    }
  }
}

template <int CPW, int W, int RT, int TT>
hipError_t launch_cwt(const Sizes& s, const mnb_plan& p, int64_t M, const float* A, float* Y,
                      int bs_shift, hipStream_t st) {
  const dim3 grid((unsigned)((s.N + 16 * RT - 1) / (16 * RT))), block(64 * W);
  if (s.zeros)
    hipLaunchKernelGGL((gemm_int4_small<CPW, W, RT, true, TT>), grid, block, 0, st, A,
                       static_cast<const uint8_t*>(p.codes), static_cast<const float*>(p.scales),
                       static_cast<const uint32_t*>(p.zeros), Y, (int32_t)M, (int32_t)s.N,
                       (int32_t)s.K, s.row_bytes, s.nb, bs_shift);
  else
    hipLaunchKernelGGL((gemm_int4_small<CPW, W, RT, false, TT>), grid, block, 0, st, A,
                       static_cast<const uint8_t*>(p.codes), static_cast<const float*>(p.scales),
                       nullptr, Y, (int32_t)M, (int32_t)s.N, (int32_t)s.K, s.row_bytes, s.nb,
                       bs_shift);
  return hipGetLastError();
}

// one 16-token tile up to M = 16, two up to 32
template <int CPW, int W, int RT = 1>
hipError_t launch_cw(const Sizes& s, const mnb_plan& p, int64_t M, const float* A, float* Y,
                     int bs_shift, hipStream_t st) {
  return M <= 16 ? launch_cwt<CPW, W, RT, 1>(s, p, M, A, Y, bs_shift, st)
                 : launch_cwt<CPW, W, RT, 2>(s, p, M, A, Y, bs_shift, st);
}

int cus() {
  static int n = 0;
  if (!n) {
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
      n = prop.multiProcessorCount;
    if (n <= 0) n = 256;
  }
  return n;
}

}  // namespace

// Used where it is the faster kernel: a workgroup per weight tile covers the
// chip only with at least one tile per CU (N >= 4096), and every workgroup
// reads all of A from L2, which dominates past a few rows of A.  Measured
// (graph replays): K = 2048, N = 6144, M = 1/4/8/16: 5.6-6.0/6.7/7.3/8.2 us
// (32-row tiles) against 10.9/11.6/11.8/12.4 us for the split-K kernel;
// K = 6144, N = 2048 (128 tiles): M = 1/4 9.2/10.6 against 11.4/11.5 us, but
// M = 8/16 12.6/16.4 against 11.5/12.0 us.  With two 16-token tiles sharing
// each dequantized weight operand (M = 17..32), K = 2048, N = 6144, M =
// 17/24/32: 9.4/10.6/12.0 against 12.5/13.3/14.0 us for the next kernel.
bool gemm_small_supported(const Sizes& s, int64_t M, const void* A) {
  const bool shape = M >= 1 && M <= 32 && s.K % 128 == 0 && s.K <= 8192 &&
                     s.N <= (int64_t(1) << 30) && (reinterpret_cast<uintptr_t>(A) & 15) == 0;
  return shape && (M <= 4 || (s.N + 15) / 16 >= 256);
}

hipError_t launch_gemm_small(const Sizes& s, const mnb_plan& p, int64_t M, const float* A,
                             float* Y, hipStream_t st) {
  const int nch = (int)(s.K / 128);
  const int bs_shift = s.bs == 32 ? 0 : (s.bs == 64 ? 1 : 2);
  // up to 16 chunks (K <= 2048): 4 waves per 16-row tile while the tiles fit
  // one round of one workgroup per CU, else 32-row tiles (two per wave, each
  // A load feeding both) over 8 waves, which keeps one round (K = 2048, M =
  // 16: N = 6144 8.2 against 11.0 us, N = 4096 6.8 against 8.1 us for the
  // other choice); 8 waves per 16-row tile beyond 16 chunks.  Chunks per wave
  // are rounded up to an instantiated count.
  if (nch <= 16) {
    if ((s.N + 15) / 16 > cus()) return launch_cw<2, 8, 2>(s, p, M, A, Y, bs_shift, st);
    const int cpw = (nch + 3) / 4;
    if (cpw <= 2) return launch_cw<2, 4>(s, p, M, A, Y, bs_shift, st);
    return launch_cw<4, 4>(s, p, M, A, Y, bs_shift, st);
  }
  const int cpw = (nch + 7) / 8;
  if (cpw <= 4) return launch_cw<4, 8>(s, p, M, A, Y, bs_shift, st);
  if (cpw <= 6) return launch_cw<6, 8>(s, p, M, A, Y, bs_shift, st);
  return launch_cw<8, 8>(s, p, M, A, Y, bs_shift, st);
}

}  // namespace mnb
