// Producer-side INT3 round-to-nearest quantizer for gfx950: fp32 weights
// [rows, K] -> row-local LSB-first 3-bit codes, fp16 or bf16 scales and a
// status per group, in the QMoE projection contract (ready for mnb_prepare).
//
// Sources: onnxruntime PR "INT3 QMoE CUDA correctness baseline and Qwen
// experimental results": embedded Olive body, "Summary" (symmetric scale
// max|w| / 3.5 with implicit zero point 4; an all-zero group takes scale
// 1 / 3.5 and code 4; non-finite weights, non-finite scales and scales that
// round to zero for a nonzero group are reported, never clamped; nonzero
// subnormal stored scales stay allowed) and embedded P0/P1 body, section
// "P0: Portable Format and Numerical References" (RTN with stored-scale
// rounding: codes are taken against the scale as stored; row-local LSB-first
// packing; FP16 or BF16 scales, P1 section).
//
// The work is a stream over the weights (4 bytes in, 3/8 byte + 2/bs out per
// weight), so the kernel is shaped for HBM: each lane takes pieces of 8
// consecutive weights as two 16-byte loads each, the bs/8 lanes of a group
// combine their maxima with lane shuffles, and every 4 lanes merge their 24
// code bits into three coalesced 32-bit stores (8 codes of 3 bits are exactly 3 bytes, and
// 4 lanes' 12 bytes start on a 4-byte boundary of the row).

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace mnb {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// The stored scale type: fp16, or bf16 (the top half of an fp32).
template <bool BF> __device__ __forceinline__ uint16_t store16(float v) {
  if constexpr (BF)
    return __builtin_bit_cast(uint16_t, (__bf16)v);  // round to nearest even
  else
    return __half_as_ushort(__float2half_rn(v));
}
template <bool BF> __device__ __forceinline__ float load16(uint16_t b) {
  if constexpr (BF)
    return __uint_as_float((uint32_t)b << 16);
  else
    return __half2float(__ushort_as_half(b));
}

// Status of a group (also the meaning of the status output):
//  0 ok, 1 a weight is NaN or infinite, 2 a nonzero group whose scale rounds
//  to zero in the stored type, 3 a scale beyond its range.
//
// One 8-weight piece i: a, b are its two 16-byte halves (zeros when invalid).
template <int BS, bool BF>
__device__ __forceinline__ void rtn_piece(f32x4 a, f32x4 b, int64_t i, bool valid,
                                          uint32_t* __restrict__ B, uint16_t* __restrict__ scales,
                                          uint8_t* __restrict__ status) {
  constexpr int L = BS / 8;  // lanes per group (4, 8 or 16)
  float w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  float amax = 0.0f;
  int finite = 1;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bool f = __builtin_isfinite(w[j]);
    finite &= f ? 1 : 0;
    amax = f ? fmaxf(amax, fabsf(w[j])) : amax;
  }
#pragma unroll
  for (int m = 1; m < L; m <<= 1) {
    amax = fmaxf(amax, __shfl_xor(amax, m));
    finite &= __shfl_xor(finite, m);
  }
  // the stored scale: the fp32 quotient rounded once to the stored type
  constexpr uint16_t kInf = BF ? 0x7F80u : 0x7C00u;
  int st = 0;
  uint16_t s16 = 0;
  if (!finite) {
    st = 1;
  } else if (amax == 0.0f) {
    s16 = store16<BF>(1.0f / 3.5f);
  } else {
    s16 = store16<BF>(amax / 3.5f);
    if ((s16 & 0x7FFFu) == 0)
      st = 2;
    else if ((s16 & 0x7FFFu) == kInf)
      st = 3;
  }
  if (st) s16 = 0;
  const float sd = load16<BF>(s16);
  // codes against the stored scale; ties to even; groups with a status keep 4
  uint32_t c24 = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    int q = 4;
    if (!st) q = min(7, max(0, (int)__builtin_rintf(w[j] / sd) + 4));
    c24 |= (uint32_t)q << (3 * j);
  }
  // lanes 4p .. 4p+3 hold bytes [12p, 12p + 12) of the stream: lane 4p + k
  // writes word k (k < 3) from its own bits and its right neighbour's
  const uint32_t next = (uint32_t)__shfl_down((int)c24, 1);
  const int k = (int)(i & 3);
  if (valid && k < 3) {
    const uint32_t word = (c24 >> (8 * k)) | (next << (24 - 8 * k));
    B[3 * (i >> 2) + k] = word;
  }
  if (valid && (i % L) == 0) {
    scales[i / L] = s16;
    status[i / L] = (uint8_t)st;
  }
}

// Each thread takes kPieces pieces a grid apart (all loads issued before any
// is used, so several 16-byte loads per lane are in flight).  Groups are
// whole runs of L consecutive pieces (K is a multiple of BS) and the grid
// stride is a multiple of 256, so a group is either entirely inside the
// valid range or entirely outside; every lane still takes part in the
// shuffles.
constexpr int kPieces = 2;

template <int BS, bool BF>
__global__ void __launch_bounds__(256) rtn_int3_kernel(const float* __restrict__ W, int64_t pieces,
                                                       uint32_t* __restrict__ B,
                                                       uint16_t* __restrict__ scales,
                                                       uint8_t* __restrict__ status) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  f32x4 a[kPieces], b[kPieces];
#pragma unroll
  for (int u = 0; u < kPieces; ++u) {
    const int64_t i = i0 + u * stride;
    a[u] = f32x4{0, 0, 0, 0};
    b[u] = f32x4{0, 0, 0, 0};
    if (i < pieces) {
      const f32x4* src = reinterpret_cast<const f32x4*>(W) + 2 * i;
      a[u] = __builtin_nontemporal_load(src);
      b[u] = __builtin_nontemporal_load(src + 1);
    }
  }
#pragma unroll
  for (int u = 0; u < kPieces; ++u) {
    const int64_t i = i0 + u * stride;
    rtn_piece<BS, BF>(a[u], b[u], i, i < pieces, B, scales, status);
  }
}

}  // namespace

namespace {
template <bool BF>
void launch_rtn_t(const float* W, int64_t pieces, int bs, uint32_t* B32, uint16_t* scales,
                  uint8_t* status, hipStream_t st) {
  const dim3 grid((unsigned)((pieces + 256 * kPieces - 1) / (256 * kPieces))), block(256);
  if (bs == 32)
    hipLaunchKernelGGL((rtn_int3_kernel<32, BF>), grid, block, 0, st, W, pieces, B32, scales, status);
  else if (bs == 64)
    hipLaunchKernelGGL((rtn_int3_kernel<64, BF>), grid, block, 0, st, W, pieces, B32, scales, status);
  else
    hipLaunchKernelGGL((rtn_int3_kernel<128, BF>), grid, block, 0, st, W, pieces, B32, scales, status);
}
}  // namespace

hipError_t launch_rtn_int3(const float* W, int64_t rows, int64_t K, int bs, bool bf16, uint8_t* B,
                           uint16_t* scales, uint8_t* status, hipStream_t st) {
  const int64_t pieces = rows * (K / 8);
  if (pieces == 0) return hipSuccess;
  uint32_t* B32 = reinterpret_cast<uint32_t*>(B);
  if (bf16)
    launch_rtn_t<true>(W, pieces, bs, B32, scales, status, st);
  else
    launch_rtn_t<false>(W, pieces, bs, B32, scales, status, st);
  return hipGetLastError();
}

}  // namespace mnb
