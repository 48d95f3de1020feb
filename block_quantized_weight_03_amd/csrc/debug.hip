// Test-only readers of the prepared device layout (logical codes and the
// fp16 dequantized weights of the matrix-core paths) and a plain streaming
// read that measures the read ceiling of the same buffers.  They let the tests
// check the prepacked bytes and the rounding chain bit-exactly against the
// oracle (onnxruntime PR "INT3 QMoE CUDA correctness baseline and Qwen
// experimental results", embedded P0/P1 body, section "P0: Portable Format
// and Numerical References": INT3 decodes as (code - 4) * scale); the INT3
// codes are read from the private pair-interleaved groups.

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace mnb {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct Rows {
  const uint8_t* codes;
  const void* scales;
  const uint8_t* zeros;
  int64_t N, K, nb, bs, row_bytes, zrow, row_base;  // row_base = expert * N + row0
  int kind, bits;
  bool bf16;  // QMoE plan with bfloat16 scales (outputs bfloat16 patterns)
};

// byte offset of 32-code group G of row n of expert e in the tile-major QMoE
// layout with GB-byte groups (rows in tiles of 16, each tile as chunks of 4
// groups, row by row)
__device__ __forceinline__ int64_t moe_goff(int64_t N, int64_t K, int64_t GB, int64_t e, int64_t n,
                                            int64_t G) {
  const int64_t ng = K / 32, rt = n / 16, r = n % 16;
  const int64_t rcnt = (N - 16 * rt) < 16 ? (N - 16 * rt) : 16;
  const int64_t c = G / 4, g = G % 4;
  const int64_t gic = (ng - 4 * c) < 4 ? (ng - 4 * c) : 4;
  return (e * N + 16 * rt) * (ng * GB) + rcnt * 4 * GB * c + r * gic * GB + g * GB;
}

__device__ __forceinline__ unsigned code_of(const Rows& r, int64_t row, int64_t k) {
  const uint8_t* src = r.codes + row * r.row_bytes;
  if (r.kind == kDenseInt4) {
    const int64_t b = k / r.bs, j = k % r.bs;
    const uint8_t byte = src[b * (r.bs / 2) + j / 2];
    return (((j & 1) ? (byte >> 4) : byte) & 15u) ^ 8u;
  }
  // QMoE: pair-interleaved groups of bits words per 32 codes, tile-major
  const uint32_t* w = reinterpret_cast<const uint32_t*>(
      r.codes + moe_goff(r.N, r.K, 4 * r.bits, row / r.N, row % r.N, k / 32));
  const int i = (int)(k % 32);
  if (r.bits == 4) return (w[int4_word(i)] >> int4_bit(i)) & 15u;
  if (i < 30) return (w[int3_word(i)] >> int3_bit(i)) & 7u;
  const int b = i == 30 ? 15 : 31;
  return ((w[0] >> b) & 1u) | (((w[1] >> b) & 1u) << 1) | (((w[2] >> b) & 1u) << 2);
}

__global__ void debug_unpack_kernel(Rows r, int64_t nrows, uint8_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nrows * r.K) return;
  const int64_t row = i / r.K, k = i % r.K;
  out[i] = (uint8_t)code_of(r, r.row_base + row, k);
}

__global__ void debug_dequant_kernel(Rows r, int64_t nrows, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nrows * r.K) return;
  const int64_t row = i / r.K, k = i % r.K;
  const int64_t grow = r.row_base + row;
  const unsigned q = code_of(r, grow, k);
  const int64_t b = k / r.bs;
  float v;
  if (r.kind == kDenseInt4) {
    unsigned z = 8;
    if (r.zeros) {
      const uint32_t w = reinterpret_cast<const uint32_t*>(r.zeros)[(grow / 8) * r.nb + b];
      z = (w >> (4 * (grow % 8))) & 15u;
    }
    const float s = static_cast<const float*>(r.scales)[grow * r.nb + b];
    // the matrix-core chain: fp32 fma(q, s, -(z*s)), then one fp16 rounding
    // (for z = 8, -(z*s) is exact and this is fp32((q - 8) * s))
    v = fmaf((float)q, s, -((float)z * s));
  } else {
    const uint16_t sb = static_cast<const uint16_t*>(r.scales)[grow * r.nb + b];
    const float s = r.bf16 ? __uint_as_float((uint32_t)sb << 16) : __half2float(__ushort_as_half(sb));
    v = (float)((int)q - (1 << (r.bits - 1))) * s;  // exact in fp32
    if (r.bf16) {
      out[i] = __builtin_bit_cast(uint16_t, (__bf16)v);
      return;
    }
  }
  out[i] = __half_as_ushort(__float2half_rn(v));
}

Rows make_rows(const Sizes& s, const mnb_plan& p, int64_t expert, int64_t row0) {
  Rows r;
  r.codes = static_cast<const uint8_t*>(p.codes);
  r.scales = p.scales;
  r.zeros = static_cast<const uint8_t*>(p.zeros);
  r.N = s.N;
  r.K = s.K;
  r.nb = s.nb;
  r.bs = s.bs;
  r.row_bytes = s.row_bytes;
  r.zrow = (int64_t)s.zrow;
  r.row_base = expert * s.N + row0;
  r.kind = s.kind;
  r.bits = (int)s.bits;
  r.bf16 = p.desc.scale_dtype == MNB_DTYPE_BF16;
  return r;
}

// Streaming read of up to kMaxSegs device buffers in one launch: every
// thread issues four 16-byte nontemporal loads (1024 lanes' worth per
// workgroup, 16 KiB) and folds them together; the result is stored only if it
// equals a value no realistic input produces, which keeps the loads live.
// One or two buffers take flat arguments (preloaded into SGPRs, like the
// short-row GEMV's), more a segment table.
struct ReadSegs {
  const u32x4* ptr[kMaxSegs];
  int64_t n16[kMaxSegs];       // 16-byte chunks per segment
  int64_t first[kMaxSegs + 1]; // first workgroup of each segment (prefix sums)
  int count;
};

__device__ __forceinline__ void stream_read_body(const u32x4* p, int64_t n, int64_t blk,
                                                 uint32_t* __restrict__ sink) {
  const int64_t base = blk * 1024 + threadIdx.x;
  u32x4 v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t i = base + 256 * j;
    v[j] = __builtin_nontemporal_load(p + (i < n ? i : n - 1));
  }
  const u32x4 x = (v[0] ^ v[1]) ^ (v[2] ^ v[3]);
  const uint32_t f = x.x ^ x.y ^ x.z ^ x.w;
  if (f == 0x9E3779B9u && x.x == 0x7F4A7C15u) sink[0] = f;
}

__global__ void __launch_bounds__(256) stream_read_kernel(ReadSegs r, uint32_t* __restrict__ sink) {
  int seg = 0;
  while (seg + 1 < r.count && (int64_t)blockIdx.x >= r.first[seg + 1]) ++seg;
  stream_read_body(r.ptr[seg], r.n16[seg], (int64_t)blockIdx.x - r.first[seg], sink);
}

__global__ void __launch_bounds__(256) stream_read_1(const u32x4* p, int64_t n, uint32_t* __restrict__ sink) {
  stream_read_body(p, n, (int64_t)blockIdx.x, sink);
}

// the second buffer owns the workgroups from first1 on
__global__ void __launch_bounds__(256) stream_read_2(const u32x4* p0, const u32x4* p1, int64_t n0,
                                                     int64_t n1, int64_t first1,
                                                     uint32_t* __restrict__ sink) {
  const bool second = (int64_t)blockIdx.x >= first1;
  stream_read_body(second ? p1 : p0, second ? n1 : n0, (int64_t)blockIdx.x - (second ? first1 : 0),
                   sink);
}

}  // namespace

hipError_t launch_stream_read(const void* const* src, const uint64_t* bytes, int count,
                              uint32_t* sink, hipStream_t st) {
  ReadSegs r{};
  r.count = count;
  r.first[0] = 0;
  for (int i = 0; i < count; ++i) {
    r.ptr[i] = static_cast<const u32x4*>(src[i]);
    r.n16[i] = (int64_t)(bytes[i] / 16);
    r.first[i + 1] = r.first[i] + (r.n16[i] + 1023) / 1024;
  }
  if (r.first[count] == 0) return hipSuccess;
  const dim3 grid((unsigned)r.first[count]);
  if (count == 1)
    hipLaunchKernelGGL(stream_read_1, grid, dim3(256), 0, st, r.ptr[0], r.n16[0], sink);
  else if (count == 2 && r.n16[0] > 0 && r.n16[1] > 0)
    hipLaunchKernelGGL(stream_read_2, grid, dim3(256), 0, st, r.ptr[0], r.ptr[1], r.n16[0], r.n16[1],
                       r.first[1], sink);
  else
    hipLaunchKernelGGL(stream_read_kernel, grid, dim3(256), 0, st, r, sink);
  return hipGetLastError();
}

hipError_t launch_debug_unpack(const Sizes& s, const mnb_plan& p, int64_t expert, int64_t row0,
                               int64_t nrows, uint8_t* codes, hipStream_t st) {
  const int64_t n = nrows * s.K;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(debug_unpack_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     make_rows(s, p, expert, row0), nrows, codes);
  return hipGetLastError();
}

hipError_t launch_debug_dequant_f16(const Sizes& s, const mnb_plan& p, int64_t expert,
                                    int64_t row0, int64_t nrows, uint16_t* out, hipStream_t st) {
  const int64_t n = nrows * s.K;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(debug_dequant_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     make_rows(s, p, expert, row0), nrows, out);
  return hipGetLastError();
}

}  // namespace mnb
