// M = 1 decode GEMV on packed INT4 weights for gfx950.
//
// Operation ("Qwen3 Missing-Kernel Implementation Plan", section "PR
// sequence", steps K01/K02):
//   y[n] = sum_{k<K} a[k] * (q[n,k] - z[n,b]) * s[n,b],  b = k / bs,
// with scales and zero points applied while the packed panel streams by and
// the float weight matrix never formed.
//
// Why integer dot products.  At 8 TB/s an MI355X receives 16e12 INT4 codes
// per second, while its integer VALU issues about 39e12 lane-ops per second,
// so a convert + subtract + FMA per code would make the kernel ALU-bound.
// Instead, the prepared weights store every code as (q - 8) in 4-bit two's
// complement, and each 32-element sub-block of a is put in block fixed point:
//   a[k] * 2^e = a_int[k] = sum_{p<8} d[k,p] * 16^p,  d in [-8, 7],
// with e chosen per sub-block so that max|a| * 2^e < 2^30 (so a_int is exact
// to 2^-31 of the sub-block maximum).  Then
//   sum_k (q-8) a_int = sum_p 16^p * dot8(q - 8, d[., p])
// where dot8 is one v_dot8c_i32_i4 over 8 packed nibbles: the raw 16-byte
// load of 32 codes feeds the dot products directly, with no unpacking.
// Explicit zero points add (8 - z) * sum_k a_int per sub-block, from digit
// sums computed with the digits.  The integer part is exact; the rest is a
// few fp32 roundings per 32 codes, so the exact special cases stay exact
// (integer inputs; all codes equal to the zero point give exactly 0).
//
// Short row streams (N up to 32768) use a plain fp32 variant of the same
// mapping instead (below), which needs no digit planes.
//
// Work mapping.  A K-chunk is 64 sub-blocks (2048 codes).  Lane l of a wave
// owns sub-block 64c + l of chunk c and keeps that chunk's 32 digit words in
// registers; the wave walks R rows at a time with one 16-byte coalesced load
// per lane and row (1 KiB per wave), one scale and optionally one zero-point
// byte.  When K spans several chunks (up to 4, K <= 8192), the waves of a
// team each own one chunk and combine in LDS in a fixed order.  The digits
// are computed inside the kernel by the whole workgroup (so one launch does
// the whole GEMV), while the first rows' loads are already in flight.  For
// K > 8192 a separate pre-pass writes the digits to the workspace and each
// wave reloads them per chunk.  Row partials are reduced across the wave
// through LDS in a fixed order: the result is deterministic.

#include <hip/hip_runtime.h>

#include <climits>

#include "kernels.h"

namespace mnb {
namespace {

constexpr int kDig = 8;            // balanced base-16 digits per element
constexpr int kBadExp = INT_MIN;   // marks a sub-block holding NaN/Inf
constexpr int kMaxTeam = 4;        // chunks held in registers by one team
constexpr int64_t kF32MaxRows = 32768;  // N up to which the plain fp32 path is used

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---- digit planes of a (shared by the in-kernel prologue and the pre-pass) --

// DPP move within groups of 4 lanes (quad_perm), used for the 4-lane
// reductions of a sub-block's quarters.
template <int CTRL>
__device__ __forceinline__ int quad_mov(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]

// Converts quarter w (8 elements) of sub-block sb.  The 4 quarters of one
// sub-block must sit in the 4 lanes of one DPP quad (they share a maximum).
// Writes plane words to dig[((c*kDig + p)*4 + w)*64 + l] (c = sb/64, l = sb%64),
// digit sums to sums[(c*4 + j)*64 + l] and -e to nexp[c*64 + l].
__device__ __forceinline__ void make_digits(const float* __restrict__ A, int64_t K, int64_t sb,
                                            int w, uint32_t* dig, int32_t* sums,
                                            int32_t* nexp) {
  float v[8];
  const int64_t k0 = sb * 32 + w * 8;
  float m = 0.0f;
  int bad = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = (k0 + i < K) ? A[k0 + i] : 0.0f;
    bad |= !isfinite(v[i]);
    m = fmaxf(m, fabsf(v[i]));
  }
  m = fmaxf(m, __int_as_float(quad_mov<kQuadSwap1>(__float_as_int(m))));
  m = fmaxf(m, __int_as_float(quad_mov<kQuadSwap2>(__float_as_int(m))));
  bad |= quad_mov<kQuadSwap1>(bad);
  bad |= quad_mov<kQuadSwap2>(bad);
  int e = 0;
  if (!bad && m > 0.0f) {
    int E;
    frexpf(m, &E);  // m < 2^E
    e = 30 - E;     // max|a| * 2^e < 2^30
  }
  uint32_t u[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float sv = bad ? 0.0f : ldexpf(v[i], e);  // exact power-of-two scaling
    const int32_t ai = (int32_t)rintf(sv);          // |ai| <= 2^30
    // adding 8 to every nibble position makes nibble p of u equal d_p + 8
    u[i] = (uint32_t)ai + 0x88888888u;
  }
  // 8 x 8 nibble transpose (word i holds value i's digits -> word p holds
  // plane p's digits of values 0..7) in three butterfly stages: 16-bit and
  // 8-bit blocks with byte permutes, 4-bit blocks with bitfield inserts.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = u[i], b = u[i + 4];
    u[i] = __builtin_amdgcn_perm(b, a, 0x05040100u);
    u[i + 4] = __builtin_amdgcn_perm(b, a, 0x07060302u);
  }
#pragma unroll
  for (int i : {0, 1, 4, 5}) {
    const uint32_t a = u[i], b = u[i + 2];
    u[i] = __builtin_amdgcn_perm(b, a, 0x06020400u);
    u[i + 2] = __builtin_amdgcn_perm(b, a, 0x07030501u);
  }
#pragma unroll
  for (int i : {0, 2, 4, 6}) {
    const uint32_t a = u[i], b = u[i + 1];
    u[i] = (a & 0x0F0F0F0Fu) | ((b << 4) & 0xF0F0F0F0u);
    u[i + 1] = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
  }
  const int64_t c = sb >> 6;
  const int l = (int)(sb & 63);
  int32_t sd[kDig];
#pragma unroll
  for (int p = 0; p < kDig; ++p) {
    // d_p in 4-bit two's complement is nib ^ 8
    dig[((c * kDig + p) * 4 + w) * 64 + l] = u[p] ^ 0x88888888u;
    // sum over the 8 values of d_p = (sum of the biased nibbles) - 64
    sd[p] = (int32_t)__builtin_amdgcn_udot8(u[p], 0x11111111u, 0u, false) - 64;
    sd[p] += quad_mov<kQuadSwap1>(sd[p]);
    sd[p] += quad_mov<kQuadSwap2>(sd[p]);
  }
  if (w == 0) {
#pragma unroll
    for (int j = 0; j < kDig / 2; ++j) sums[(c * (kDig / 2) + j) * 64 + l] = sd[2 * j] + 16 * sd[2 * j + 1];
    nexp[c * 64 + l] = bad ? kBadExp : -e;
  }
}

__global__ void __launch_bounds__(256) gemv_prep_a(const float* __restrict__ A, int64_t K,
                                                   int64_t nsb_pad, uint32_t* __restrict__ dig,
                                                   int32_t* __restrict__ sums,
                                                   int32_t* __restrict__ nexp) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if ((t >> 2) >= nsb_pad) return;  // whole groups of 4 lanes leave together
  make_digits(A, K, t >> 2, (int)(t & 3), dig, sums, nexp);
}

struct Digits {
  uint32_t d[kDig][4];
  int32_t sf[2];  // digit sums weighted as in F0 and F1 below (planes 0-3, 4-7)
  int32_t ne;
  float poison;
};

template <class P>
__device__ __forceinline__ void load_digits(Digits& g, const P* dig, const int32_t* sums,
                                            const int32_t* nexp, int64_t c, int lane) {
#pragma unroll
  for (int p = 0; p < kDig; ++p)
#pragma unroll
    for (int w = 0; w < 4; ++w) g.d[p][w] = dig[((c * kDig + p) * 4 + w) * 64 + lane];
  int32_t se[kDig / 2];
#pragma unroll
  for (int j = 0; j < kDig / 2; ++j) se[j] = sums[(c * (kDig / 2) + j) * 64 + lane];
  // |se| <= 256 + 16 * 256, so |sf| < 2^21 (exact 24-bit multiplies below)
  g.sf[0] = se[0] + 256 * se[1];
  g.sf[1] = se[2] + 256 * se[3];
  const int32_t ne = nexp[c * 64 + lane];
  g.poison = ne == kBadExp ? __builtin_nanf("") : 0.0f;
  g.ne = ne == kBadExp ? 0 : ne;
}

// Partial of one 32-code sub-block: sum_k (q_k - z) * a_k * s (fp32).
// F0 = D0 + 16 D1 + 256 D2 + 4096 D3 (D_p = the codes' dot product with digit
// plane p) is built by Horner's rule, each plane's four v_dot8 accumulating
// onto 16 times the planes above it, likewise F1 over planes 4..7; |D_p| <=
// 32 * 8 * 8, so |F| < 2^25 and nothing overflows.
template <bool HAS_ZP>
__device__ __forceinline__ float subblock_dot(const u32x4 q, const Digits& g, float s, int z) {
  int F[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int acc = 0;
#pragma unroll
    for (int p = 4 * h + 3; p >= 4 * h; --p) {
      acc *= 16;
      acc = __builtin_amdgcn_sdot8((int)q.x, (int)g.d[p][0], acc, false);
      acc = __builtin_amdgcn_sdot8((int)q.y, (int)g.d[p][1], acc, false);
      acc = __builtin_amdgcn_sdot8((int)q.z, (int)g.d[p][2], acc, false);
      acc = __builtin_amdgcn_sdot8((int)q.w, (int)g.d[p][3], acc, false);
    }
    F[h] = acc;
  }
  if (HAS_ZP) {
    // |8 - z| <= 8 and |sf| < 2^21: 24-bit multiplies are exact
    const int zc = 8 - z;
    F[0] = __mul24(zc, g.sf[0]) + F[0];
    F[1] = __mul24(zc, g.sf[1]) + F[1];
  }
  const float f = fmaf((float)F[1], 65536.0f, (float)F[0]);
  return ldexpf(f * s, g.ne) + g.poison;
}

// Raw buffer resource over `bytes` bytes at p: a load whose dwords lie past
// the end returns 0 for them, so clamps and tail branches are not needed.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_over(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

constexpr uint32_t kOutOfRange = 0x80000000u;  // buffer offset past every resource used here
constexpr int kNT = 2;                          // cache policy: nontemporal (streamed once)

template <int R, bool HAS_ZP>
struct RowTile {
  u32x4 q[R];
  float s[R];
  uint32_t zpk;  // zero point of row r in bits [4r, 4r+4) (R <= 8)
};

// Loads R rows starting at row n0 for sub-block sb (lane-local).  Rows past N
// and lanes past the last sub-block load nothing.
template <int R, bool HAS_ZP>
__device__ __forceinline__ void load_rows(RowTile<R, HAS_ZP>& t, const uint8_t* __restrict__ codes,
                                          const float* __restrict__ scales,
                                          const uint32_t* __restrict__ zeros, int64_t n0, int64_t N,
                                          int64_t row_bytes, int64_t nb, int64_t zrow, uint32_t qoff,
                                          uint32_t b, bool act) {
  t.zpk = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    t.q[r] = u32x4{0, 0, 0, 0};
    t.s[r] = 0.0f;
    const int64_t n = n0 + r;
    if (n < N) {  // wave-uniform
      const uint8_t* row = codes + n * row_bytes;
      const float* srow = scales + n * nb;
      if (act) {
        // streamed once: nontemporal loads keep them from displacing reused data
        t.q[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + qoff));
        t.s[r] = __builtin_nontemporal_load(srow + b);
      }
    }
  }
  // one word holds the zero points of the 8-row group containing these rows
  // (R divides 8 and n0 is a multiple of R); it is only shifted at compute time
  if (HAS_ZP && act && n0 < N)
    t.zpk = __builtin_nontemporal_load(zeros + (n0 >> 3) * nb + b) >> (4 * (n0 & 7));
}

// The same loads through buffer resources over the codes, scales and zero
// points: rows past N lie past the end of each resource and inactive lanes
// add an out-of-range offset, so every load returns zeros for them without
// a branch.  lq, ls and lz are the lane terms (kOutOfRange for inactive
// lanes); the launcher checks that the offsets of the rows a wave can touch
// stay below 2^31.
template <int R, bool HAS_ZP>
__device__ __forceinline__ void load_rows_buf(RowTile<R, HAS_ZP>& t, __amdgpu_buffer_rsrc_t rc,
                                              __amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rz,
                                              uint32_t n0, uint32_t row_bytes, uint32_t nb4,
                                              uint32_t lq, uint32_t ls, uint32_t lz) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t n = n0 + r;
    t.q[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, n * row_bytes + lq, 0, kNT));
    t.s[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, n * nb4 + ls, 0, kNT));
  }
  t.zpk = 0;
  if (HAS_ZP) t.zpk = __builtin_amdgcn_raw_buffer_load_b32(rz, (n0 >> 3) * nb4 + lz, 0, kNT) >> (4 * (n0 & 7));
}

// Reduces part[r] over the 64 lanes of the wave in a fixed order and returns,
// in lane r*(64/R) for each r < R, the total of row r (other lanes: garbage).
template <int R>
__device__ __forceinline__ float wave_reduce_rows(float (&part)[R], float* __restrict__ red,
                                                  int lane) {
  constexpr int P = 64 / R;  // lanes that share one row after the transpose
#pragma unroll
  for (int r = 0; r < R; ++r) red[r * 64 + lane] = part[r];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int r = lane / P, j = lane % P;
  float acc = 0.0f;
  const float* src = red + r * 64 + j * R;
#pragma unroll
  for (int i = 0; i < R; ++i) acc += src[i];
#pragma unroll
  for (int m = P / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, P);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();  // red is reused by the next iteration
  return acc;
}

template <int R>
constexpr int lds_red_floats() {
  return kMaxTeam * R * 64 + kMaxTeam * R;
}

// Fused kernel: in-kernel digits, K <= 8192 (team = nchunk waves, one chunk
// each), workgroups of nwaves waves, grid workgroups.
template <int R, bool HAS_ZP, bool BUF>
__device__ __forceinline__ void gemv_fused_body(
    const float* __restrict__ A, const uint8_t* __restrict__ codes,
    const float* __restrict__ scales, const uint32_t* __restrict__ zeros, float* __restrict__ Y,
    int64_t K, int64_t N, int64_t row_bytes, int64_t nb, int32_t nsb, int32_t nchunk,
    int32_t bs_shift, int64_t zrow, int nwaves, int64_t grid) {
  extern __shared__ __align__(16) uint32_t smem[];
  float* red_all = reinterpret_cast<float*>(smem);          // [4 waves][R][64]
  float* tot = red_all + kMaxTeam * R * 64;                  // [4 waves][R]
  uint32_t* dig = smem + lds_red_floats<R>();                // [nchunk][8][4][64]
  int32_t* sums = reinterpret_cast<int32_t*>(dig + nchunk * kDig * 4 * 64);  // [nchunk][4][64]
  int32_t* nexp = sums + nchunk * (kDig / 2) * 64;           // [nchunk][64]

  const int team = nchunk;
  const int teams = nwaves / team;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = (int)(threadIdx.x & 63);
  const int tm = wave / team, wit = wave - tm * team;

  const int32_t sb = wit * 64 + lane;
  const bool act = sb < nsb;
  const uint32_t qoff = (uint32_t)sb * 16u;
  const uint32_t b = (uint32_t)sb >> bs_shift;

  const int64_t nrg = (N + R - 1) / R;
  const int64_t stride = grid * teams;
  const int64_t base0 = (int64_t)blockIdx.x * teams;
  const int64_t iters = base0 < nrg ? (nrg - base0 + stride - 1) / stride : 0;
  int64_t rg = base0 + tm;

  // buffer path: resources over the codes, scales and zero-point words
  const __amdgpu_buffer_rsrc_t rc = buffer_over(codes, BUF ? (uint32_t)(N * row_bytes) : 0u);
  const __amdgpu_buffer_rsrc_t rs = buffer_over(scales, BUF ? (uint32_t)(N * nb * 4) : 0u);
  const __amdgpu_buffer_rsrc_t rz =
      buffer_over(zeros, BUF && HAS_ZP ? (uint32_t)(((N + 7) >> 3) * nb * 4) : 0u);
  const uint32_t lq = act ? qoff : kOutOfRange, ls = act ? 4u * b : kOutOfRange;
  const uint32_t rb32 = (uint32_t)row_bytes, nb4 = 4u * (uint32_t)nb;
  auto load = [&](RowTile<R, HAS_ZP>& t, int64_t g) {
    if constexpr (BUF)
      load_rows_buf<R, HAS_ZP>(t, rc, rs, rz, (uint32_t)(g * R), rb32, nb4, lq, ls, ls);
    else
      load_rows<R, HAS_ZP>(t, codes, scales, zeros, g * R, g < nrg ? N : 0, row_bytes, nb, zrow, qoff, b, act);
  };

  RowTile<R, HAS_ZP> t0, t1;
  if (iters > 0) load(t0, rg);

  // digits of this workgroup's chunks, computed by all threads
  const int64_t tasks = (int64_t)nchunk * 64 * 4;
  for (int64_t i = threadIdx.x; i < tasks; i += 64 * nwaves)
    make_digits(A, K, i >> 2, (int)(i & 3), dig, sums, nexp);
  __syncthreads();
  Digits g;
  load_digits(g, dig, sums, nexp, wit, lane);
  float* red = red_all + wave * R * 64;

  auto step = [&](RowTile<R, HAS_ZP>& cur, RowTile<R, HAS_ZP>& nxt, int64_t it) {
    const int64_t rgn = rg + stride;
    // Buffer path: the next group's loads are issued unconditionally (past the
    // last group they read zeros), so no branch joins the loop body and the
    // compiler waits only for this group's loads, not for every load in flight.
    if constexpr (BUF)
      load(nxt, rgn < nrg ? rgn : nrg);
    else if (it + 1 < iters)
      load(nxt, rgn);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of this group's arithmetic
    float part[R];
#pragma unroll
    for (int r = 0; r < R; ++r) part[r] = subblock_dot<HAS_ZP>(cur.q[r], g, cur.s[r], (int)((cur.zpk >> (4 * r)) & 15u));
    const float v = wave_reduce_rows<R>(part, red, lane);
    constexpr int P = 64 / R;
    const int r = lane / P;
    const bool leader = (lane % P) == 0;
    const int64_t n = rg * R + r;
    if (team == 1) {
      if (leader && rg < nrg && n < N) Y[n] = v;
    } else {
      if (leader) tot[wave * R + r] = v;
      __syncthreads();
      if (wit == 0 && lane < R) {
        float out = 0.0f;
        for (int w = 0; w < team; ++w) out += tot[(tm * team + w) * R + lane];
        const int64_t nn = rg * R + lane;
        if (rg < nrg && nn < N) Y[nn] = out;
      }
      __syncthreads();
    }
    rg = rgn;
  };

  for (int64_t it = 0; it < iters; it += 2) {
    step(t0, t1, it);
    if (it + 1 < iters) step(t1, t0, it + 1);
  }
}

template <int R, bool HAS_ZP, bool BUF>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) gemv_int4_fused(
    const float* __restrict__ A, const uint8_t* __restrict__ codes,
    const float* __restrict__ scales, const uint32_t* __restrict__ zeros, float* __restrict__ Y,
    int64_t K, int64_t N, int64_t row_bytes, int64_t nb, int32_t nsb, int32_t nchunk,
    int32_t bs_shift, int64_t zrow) {
  gemv_fused_body<R, HAS_ZP, BUF>(A, codes, scales, zeros, Y, K, N, row_bytes, nb, nsb, nchunk,
                                  bs_shift, zrow, (int)(blockDim.x >> 6), (int64_t)gridDim.x);
}

// The same with flat arguments, all preloaded into SGPRs (10 dwords; the
// block size follows from K as in the launcher and the grid size is an argument,
// so no implicit argument is read either): scales and zero points at
// codes + off_s and codes + off_z, meta = K | bs_shift << 16, blocked rows.
// Used where 32-bit offsets cover the matrix (the buffer path).
template <int R, bool HAS_ZP>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) gemv_int4_fused_flat(
    const float* __restrict__ A, const uint8_t* __restrict__ codes, float* __restrict__ Y,
    int32_t N, uint32_t meta, uint32_t off_s, uint32_t off_z, int32_t grid) {
  const int K = (int)(meta & 0xFFFFu), bs_shift = (int)(meta >> 16);
  const int nb = (K + (32 << bs_shift) - 1) >> (5 + bs_shift);
  const int nsb = nb << bs_shift;
  gemv_fused_body<R, HAS_ZP, true>(A, codes, reinterpret_cast<const float*>(codes + off_s),
                                   reinterpret_cast<const uint32_t*>(codes + off_z), Y, K, N,
                                   16 * nsb, nb, nsb, (nsb + 63) >> 6, bs_shift, 0,
                                   kMaxTeam / ((nsb + 63) >> 6) * ((nsb + 63) >> 6), grid);
}

// ---- plain fp32 path for small N ----------------------------------------
//
// When each wave only sees a few rows, building the digit planes costs more
// than it saves.  Lane l instead keeps the 32 activations of its sub-block in
// registers and takes every code as a sign-extended nibble: (q - z) is an
// exact small integer, and four fp32 FMA chains per row (one per 8-code word)
// add (q - z) * a in a fixed order; the sub-block partial is then scaled by
// s.  Rounding: at most ~32 ulp of fp32 relative to sum |(q - z) a| per
// sub-block; codes equal to the zero point contribute exactly 0.  A
// non-finite activation makes every output NaN, as in the digit path.
//
// These launches are short, and every dispatch starts with cold instruction
// caches, so the code is kept compact: activations come in through
// bounds-checked buffer loads (reads past K return 0, no tail branch) and the
// row loop is not unrolled.

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Acts {
  float a[32];
  float poison;
};

// (q - 8) / 16 of the low nibble of byte B of x: v_cvt_off_f32_i4 converts
// the signed 4-bit value in bits [3:0] of its source to float and divides by
// 16 (exact), and the byte is taken by an SDWA source select (the compiler
// folds the shift and mask).  The stored nibble is q ^ 8, i.e. q - 8 in 4-bit
// two's complement.
template <int B>
__device__ __forceinline__ float nib16(uint32_t x) {
  return __builtin_amdgcn_cvt_off_f32_i4(B == 3 ? x >> 24 : (x >> (8 * B)) & 0xFFu);
}

template <bool HAS_ZP>
__device__ __forceinline__ float subblock_dot_f32(const u32x4 q, const Acts& x, float s, int z) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float acc[4];
  if constexpr (HAS_ZP) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[i] = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int v = ((int)(w[i] << (28 - 4 * e)) >> 28) + 8 - z;  // stored nibble = q - 8
        acc[i] = fmaf((float)v, x.a[8 * i + e], acc[i]);
      }
    }
    return ((acc[0] + acc[1]) + (acc[2] + acc[3])) * s + x.poison;
  } else {
    // z = 8: the chains add (q - 8) a / 16 (every product and partial sum is
    // 2^-4 times the one of (q - 8) a, so the rounding is the same) and the
    // sub-block sum is scaled back by 16 exactly; codes in even and odd
    // nibble positions come from the word and the word shifted by 4
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = w[i];
      uint32_t hi = w[i] >> 4;
      asm("" : "+v"(hi));  // one shift, then byte selects (not a bit-field extract per code)
      float c = 0.0f;
      c = fmaf(nib16<0>(lo), x.a[8 * i + 0], c);
      c = fmaf(nib16<0>(hi), x.a[8 * i + 1], c);
      c = fmaf(nib16<1>(lo), x.a[8 * i + 2], c);
      c = fmaf(nib16<1>(hi), x.a[8 * i + 3], c);
      c = fmaf(nib16<2>(lo), x.a[8 * i + 4], c);
      c = fmaf(nib16<2>(hi), x.a[8 * i + 5], c);
      c = fmaf(nib16<3>(lo), x.a[8 * i + 6], c);
      c = fmaf(nib16<3>(hi), x.a[8 * i + 7], c);
      acc[i] = c;
    }
    return ldexpf((acc[0] + acc[1]) + (acc[2] + acc[3]), 4) * s + x.poison;
  }
}


// Sum over the 64 lanes of a wave with DPP moves (no LDS round trip); the
// total lands in lane 63.  Fixed order, so the result is deterministic.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xF, false));
}

__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_mov<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x141, 0xF>(v);  // row_half_mirror: 8-lane sums
  v += dpp_mov<0x140, 0xF>(v);  // row_mirror: 16-lane sums
  v += dpp_mov<0x142, 0xA>(v);  // row_bcast15: rows 1, 3 add rows 0, 2
  v += dpp_mov<0x143, 0xC>(v);  // row_bcast31: rows 2, 3 add lane 31
  return v;
}

constexpr int kTeams = 4;  // row groups (teams of waves) per workgroup of the fp32 path
constexpr int kNPT = 8 / kTeams;  // 16-byte pieces of A per thread

// Up to kMaxSegs weight matrices with the same K, block size and zero-point
// kind, multiplied by the same A in one launch: segment i owns workgroups
// [first[i], first[i + 1]).  Used when the matrices differ in N or in the
// placement of their sections; the common one- and two-matrix launches take
// flat arguments instead (below).
struct GemvSegs {
  const uint8_t* codes[kMaxSegs];
  const float* scales[kMaxSegs];
  const uint32_t* zeros[kMaxSegs];
  float* Y[kMaxSegs];
  int32_t N[kMaxSegs];
  int32_t first[kMaxSegs + 1];
  int32_t count;
};

// Shape terms of the short-row kernels.  The launch passes K and the
// block-size shift packed in one word (K < 2^16 on this path) and the
// kernel derives the rest on the scalar unit: nb blocks, nsb = nb * bs / 32
// sub-blocks, row_bytes = 16 * nsb (blocked rows), team = ceil(nsb / 64).
struct F32Shape {
  int K, nb, nsb, row_bytes, team, bs_shift;
};

__device__ __forceinline__ F32Shape f32_shape(uint32_t meta) {
  F32Shape h;
  h.K = (int)(meta & 0xFFFFu);
  h.bs_shift = (int)(meta >> 16);
  h.nb = (h.K + (32 << h.bs_shift) - 1) >> (5 + h.bs_shift);
  h.nsb = h.nb << h.bs_shift;
  h.row_bytes = h.nsb * 16;
  h.team = (h.nsb + 63) >> 6;
  return h;
}

// One-shot: every wave takes R consecutive rows of one K chunk, with 32-bit
// index math throughout (the launcher checks that the codes of the matrix
// span less than 2^31 bytes).  Inactive lanes and rows past N read through
// an out-of-range buffer offset and so contribute exact zeros.  The
// workgroup stages A once in LDS (every team's waves read it from there, so
// global A traffic is one copy per workgroup instead of one per wave):
// 16-byte chunk j of sub-block i sits at chunk j ^ ((i >> 1) & 7) of the
// sub-block's 128 bytes, so the 16 lanes served per LDS cycle hit 64
// distinct banks.  The A loads are issued before the weight loads; loads
// complete in order, so waiting for A does not wait for the weights.
// blk is the workgroup's index within its matrix.
template <int R, bool HAS_ZP>
__device__ __forceinline__ void gemv_f32_body(const float* __restrict__ A,
                                              const uint8_t* __restrict__ codes,
                                              const float* __restrict__ scales,
                                              const uint32_t* __restrict__ zeros,
                                              float* __restrict__ Y, const int N, const int blk,
                                              const F32Shape h) {
  // A: 64 * team sub-blocks of 128 bytes (the launcher sizes it), then the
  // team partials
  extern __shared__ __align__(16) u32x4 as[];
  const int team = h.team;
  float* tot = reinterpret_cast<float*>(as + 512 * team);

  const int tid = (int)threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  // kTeams teams of `team` waves (one K chunk each), one row group per team
  const int tm = (wave >= team) + (wave >= 2 * team) + (wave >= 3 * team);
  const int wit = wave - tm * team;
  const int n0 = (blk * kTeams + tm) * R;

  // A pieces of this thread: tid + nt * u (past K: zeros); the workgroup's
  // nt = 256 team threads hold all 8 * 64 * team pieces of its K chunks
  const int nt = 64 * kTeams * team;
  const __amdgpu_buffer_rsrc_t ra = buffer_over(A, (uint32_t)h.K * 4u);
  u32x4 ap[kNPT];
#pragma unroll
  for (int u = 0; u < kNPT; ++u)
    ap[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ra, 16u * (uint32_t)(tid + nt * u), 0, 0));

  const int sb = wit * 64 + lane;
  const bool act = sb < h.nsb;
  const uint32_t b = (uint32_t)sb >> h.bs_shift;
  const uint32_t row_bytes = (uint32_t)h.row_bytes, nb = (uint32_t)h.nb;
  const __amdgpu_buffer_rsrc_t rc = buffer_over(codes, (uint32_t)N * row_bytes);
  const __amdgpu_buffer_rsrc_t rs = buffer_over(scales, (uint32_t)N * nb * 4u);
  u32x4 q[R];
  float s[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t row = (uint32_t)(n0 + r);
    q[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         rc, act ? row * row_bytes + 16u * sb : kOutOfRange, 0, kNT));
    s[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                         rs, act ? (row * nb + b) * 4u : kOutOfRange, 0, kNT));
  }
  uint32_t zpk = 0;  // zero point of row n0 + r in bits [4r, 4r + 4)
  if (HAS_ZP) {
    const uint32_t zbytes = (uint32_t)((N + 7) >> 3) * nb * 4u;
    zpk = __builtin_amdgcn_raw_buffer_load_b32(buffer_over(zeros, zbytes),
                                               act ? ((n0 >> 3) * nb + b) * 4u : kOutOfRange, 0, kNT) >>
          (4 * (n0 & 7));
  }

#pragma unroll
  for (int u = 0; u < kNPT; ++u) {
    const int pc = tid + nt * u, i = pc >> 3, j = pc & 7;
    as[(i << 3) | (j ^ ((i >> 1) & 7))] = ap[u];
  }
  __syncthreads();
  Acts x;
  {
    float p = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const u32x4 v = as[(sb << 3) | (j ^ ((sb >> 1) & 7))];
      x.a[4 * j] = __uint_as_float(v.x);
      x.a[4 * j + 1] = __uint_as_float(v.y);
      x.a[4 * j + 2] = __uint_as_float(v.z);
      x.a[4 * j + 3] = __uint_as_float(v.w);
    }
    // a * 0 is 0 for finite a and NaN otherwise (four short chains)
    float pc[4] = {p, p, p, p};
#pragma unroll
    for (int i = 0; i < 32; ++i) pc[i & 3] = fmaf(x.a[i], 0.0f, pc[i & 3]);
    x.poison = (pc[0] + pc[1]) + (pc[2] + pc[3]);
  }

  float v[R];
#pragma unroll
  for (int r = 0; r < R; ++r)
    v[r] = wave_sum_dpp(subblock_dot_f32<HAS_ZP>(q[r], x, s[r], (int)((zpk >> (4 * r)) & 15u)));
  if (team == 1) {
    if (lane == 63) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (n0 + r < N) Y[n0 + r] = v[r];
    }
  } else {
    if (lane == 63) {
#pragma unroll
      for (int r = 0; r < R; ++r) tot[wave * R + r] = v[r];
    }
    __syncthreads();
    if (wit == 0 && lane < R) {
      float out = 0.0f;
      for (int w = 0; w < team; ++w) out += tot[(tm * team + w) * R + lane];
      if (n0 + lane < N) Y[n0 + lane] = out;
    }
  }
}

// Workgroups per matrix of N rows.
__host__ __device__ constexpr int f32_blocks(int N, int R) { return ((N + R - 1) / R + kTeams - 1) / kTeams; }

// One or two matrices with flat arguments, at most 14 dwords, so that a
// kernel built with kernel-argument preloading receives all of them in
// SGPRs at wave launch instead of loading them first.  The sections of a
// matrix are addressed from its codes: scales at codes + off_s, zero points
// at codes + off_z.  With two matrices (same N, same section offsets), the
// second owns the workgroups from f32_blocks(N) on.
template <int R, bool HAS_ZP>
__global__ void __launch_bounds__(1024) gemv_int4_f32(
    const float* __restrict__ A, const uint8_t* __restrict__ codes, float* __restrict__ Y,
    int32_t N, uint32_t meta, uint32_t off_s, uint32_t off_z) {
  gemv_f32_body<R, HAS_ZP>(A, codes, reinterpret_cast<const float*>(codes + off_s),
                           reinterpret_cast<const uint32_t*>(codes + off_z), Y, N,
                           (int)blockIdx.x, f32_shape(meta));
}

template <int R, bool HAS_ZP>
__global__ void __launch_bounds__(1024) gemv_int4_f32_pair(
    const float* __restrict__ A, const uint8_t* codes0, const uint8_t* codes1, float* Y0,
    float* Y1, int32_t N, uint32_t meta, uint32_t off_s, uint32_t off_z) {
  const int per = f32_blocks(N, R);
  const bool second = (int)blockIdx.x >= per;
  const uint8_t* codes = second ? codes1 : codes0;
  gemv_f32_body<R, HAS_ZP>(A, codes, reinterpret_cast<const float*>(codes + off_s),
                           reinterpret_cast<const uint32_t*>(codes + off_z), second ? Y1 : Y0, N,
                           (int)blockIdx.x - (second ? per : 0), f32_shape(meta));
}

template <int R, bool HAS_ZP>
__global__ void __launch_bounds__(1024) gemv_int4_f32_segs(const float* __restrict__ A,
                                                           const GemvSegs sg, uint32_t meta) {
  int seg = 0;
#pragma unroll
  for (int i = 1; i < kMaxSegs; ++i)
    if (i < sg.count && (int)blockIdx.x >= sg.first[i]) seg = i;
  gemv_f32_body<R, HAS_ZP>(A, sg.codes[seg], sg.scales[seg], sg.zeros[seg], sg.Y[seg], sg.N[seg],
                           (int)blockIdx.x - sg.first[seg], f32_shape(meta));
}

// K > 8192: digits precomputed in the workspace, each wave walks its chunks.
template <int R, bool HAS_ZP>
__global__ void __launch_bounds__(256) gemv_int4_ws(
    const uint8_t* __restrict__ codes, const float* __restrict__ scales,
    const uint32_t* __restrict__ zeros, const uint32_t* __restrict__ dig,
    const int32_t* __restrict__ sums, const int32_t* __restrict__ nexp, float* __restrict__ Y,
    int64_t N, int64_t row_bytes, int64_t nb, int64_t nsb, int64_t nchunk, int32_t bs_shift,
    int64_t zrow) {
  __shared__ __align__(16) float red_all[kMaxTeam * R * 64];
  __shared__ float tot[kMaxTeam][R];
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = (int)(threadIdx.x & 63);
  float* red = red_all + wave * R * 64;
  const int64_t nrg = (N + R - 1) / R;
  Digits g;
  for (int64_t rg = blockIdx.x; rg < nrg; rg += gridDim.x) {
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;
    for (int64_t c = wave; c < nchunk; c += kMaxTeam) {
      load_digits(g, dig, sums, nexp, c, lane);
      const int64_t sb = c * 64 + lane;
      const bool act = sb < nsb;
      RowTile<R, HAS_ZP> t;
      load_rows<R, HAS_ZP>(t, codes, scales, zeros, rg * R, N, row_bytes, nb, zrow,
                           (uint32_t)(sb * 16), (uint32_t)(sb >> bs_shift), act);
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] += subblock_dot<HAS_ZP>(t.q[r], g, t.s[r], (int)((t.zpk >> (4 * r)) & 15u));
    }
    const float v = wave_reduce_rows<R>(acc, red, lane);
    constexpr int P = 64 / R;
    if (lane % P == 0) tot[wave][lane / P] = v;
    __syncthreads();
    if (wave == 0 && lane < R) {
      const float out = ((tot[0][lane] + tot[1][lane]) + tot[2][lane]) + tot[3][lane];
      const int64_t n = rg * R + lane;
      if (n < N) Y[n] = out;
    }
    __syncthreads();
  }
}

struct WsLayout {
  uint64_t dig, sums, nexp, total;
};

WsLayout ws_layout(int64_t nchunk) {
  WsLayout w;
  w.dig = 0;
  w.sums = align256((uint64_t)nchunk * kDig * 4 * 64 * 4);
  w.nexp = w.sums + align256((uint64_t)nchunk * (kDig / 2) * 64 * 4);
  w.total = w.nexp + align256((uint64_t)nchunk * 64 * 4);
  return w;
}

int64_t n_subblocks(const Sizes& s) { return s.nb * (s.bs / 32); }
int bs_shift_of(const Sizes& s) { return s.bs == 32 ? 0 : (s.bs == 64 ? 1 : 2); }

int cu_count() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
      cus = prop.multiProcessorCount;
    if (cus <= 0) cus = 256;
  }
  return cus;
}

// Byte offset of section `sec` from the codes of plan p, if it fits the
// 32-bit offset of the flat launches (always, for plans made by
// mnb_prepare: the sections follow the codes, 256-byte aligned).
bool section_offset(const mnb_plan& p, const void* sec, uint32_t* off) {
  if (!sec) {
    *off = 0;
    return true;
  }
  const uintptr_t c = reinterpret_cast<uintptr_t>(p.codes), v = reinterpret_cast<uintptr_t>(sec);
  if (v < c || v - c > 0xFFFFFF00u || (v - c) % 4) return false;
  *off = (uint32_t)(v - c);
  return true;
}

template <int R, bool HAS_ZP>
hipError_t launch_fused(const Sizes& s, const mnb_plan& p, const float* A, float* Y, int64_t nsb,
                        int64_t nchunk, hipStream_t st) {
  // 32-bit buffer offsets for every row a wave can touch (row groups past the
  // last one, up to R * 64 rows past N, read zeros)
  const int64_t rows = s.N + (int64_t)R * 64;
  const bool buf = rows * s.row_bytes < (int64_t(1) << 31) && rows * s.nb * 4 < (int64_t(1) << 31);
  const int team = (int)nchunk;
  const int teams = kMaxTeam / team;
  const int threads = 64 * team * teams;
  const int64_t nrg = (s.N + R - 1) / R;
  int64_t blocks = (nrg + teams - 1) / teams;
  // a few resident workgroups per CU; each walks many row groups so that the
  // digit prologue is amortised
  const int64_t cap = (int64_t)cu_count() * 4;
  if (blocks > cap) blocks = cap;
  const size_t lds = (size_t)lds_red_floats<R>() * 4 + (size_t)nchunk * (kDig * 4 * 64 + (kDig / 2) * 64 + 64) * 4;
  uint32_t os, oz;
  if (buf && section_offset(p, p.scales, &os) && section_offset(p, HAS_ZP ? p.zeros : nullptr, &oz)) {
    hipLaunchKernelGGL((gemv_int4_fused_flat<R, HAS_ZP>), dim3((unsigned)blocks), dim3(threads), lds, st,
                       A, static_cast<const uint8_t*>(p.codes), Y, (int32_t)s.N,
                       (uint32_t)s.K | ((uint32_t)bs_shift_of(s) << 16), os, oz, (int32_t)blocks);
    return hipGetLastError();
  }
  auto kern = buf ? gemv_int4_fused<R, HAS_ZP, true> : gemv_int4_fused<R, HAS_ZP, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(threads), lds, st,
                     A, static_cast<const uint8_t*>(p.codes), static_cast<const float*>(p.scales),
                     static_cast<const uint32_t*>(p.zeros), Y, s.K, s.N, s.row_bytes, s.nb,
                     (int32_t)nsb, (int32_t)nchunk, bs_shift_of(s), (int64_t)s.zrow);
  return hipGetLastError();
}

// s: the shape shared by the matrices (K, block size, zero-point kind);
// matrix i multiplies plan p[i] (N = N[i]) into Y[i]
template <int R, bool HAS_ZP>
hipError_t launch_f32_segs(const Sizes& s, const mnb_plan* const* p, const int64_t* N, int count,
                           const float* A, float* const* Y, int64_t nsb, int64_t nchunk,
                           hipStream_t st) {
  const int team = (int)nchunk;
  const uint32_t meta = (uint32_t)s.K | ((uint32_t)bs_shift_of(s) << 16);
  const size_t lds = (size_t)team * 8192 + (size_t)kTeams * team * R * 4;
  const dim3 threads(64 * kTeams * team);
  (void)nsb;
  uint32_t os[2], oz[2];
  bool flat = count <= 2;
  for (int i = 0; i < count && flat; ++i)
    flat = section_offset(*p[i], p[i]->scales, &os[i]) && section_offset(*p[i], HAS_ZP ? p[i]->zeros : nullptr, &oz[i]);
  if (flat && count == 1) {
    hipLaunchKernelGGL((gemv_int4_f32<R, HAS_ZP>), dim3((unsigned)f32_blocks((int)N[0], R)), threads, lds,
                       st, A, static_cast<const uint8_t*>(p[0]->codes), Y[0], (int32_t)N[0], meta,
                       os[0], oz[0]);
    return hipGetLastError();
  }
  if (flat && count == 2 && N[0] == N[1] && os[0] == os[1] && oz[0] == oz[1]) {
    hipLaunchKernelGGL((gemv_int4_f32_pair<R, HAS_ZP>), dim3((unsigned)(2 * f32_blocks((int)N[0], R))),
                       threads, lds, st, A, static_cast<const uint8_t*>(p[0]->codes),
                       static_cast<const uint8_t*>(p[1]->codes), Y[0], Y[1], (int32_t)N[0], meta,
                       os[0], oz[0]);
    return hipGetLastError();
  }
  GemvSegs sg{};
  sg.count = count;
  int64_t blocks = 0;
  for (int i = 0; i < count; ++i) {
    sg.codes[i] = static_cast<const uint8_t*>(p[i]->codes);
    sg.scales[i] = static_cast<const float*>(p[i]->scales);
    sg.zeros[i] = static_cast<const uint32_t*>(p[i]->zeros);
    sg.Y[i] = Y[i];
    sg.N[i] = (int32_t)N[i];
    sg.first[i] = (int32_t)blocks;
    blocks += f32_blocks((int)N[i], R);
  }
  sg.first[count] = (int32_t)blocks;
  hipLaunchKernelGGL((gemv_int4_f32_segs<R, HAS_ZP>), dim3((unsigned)blocks), threads, lds, st, A, sg,
                     meta);
  return hipGetLastError();
}

template <int R, bool HAS_ZP>
hipError_t launch_f32(const Sizes& s, const mnb_plan& p, const float* A, float* Y, int64_t nsb,
                      int64_t nchunk, hipStream_t st) {
  const mnb_plan* pp = &p;
  return launch_f32_segs<R, HAS_ZP>(s, &pp, &s.N, 1, A, &Y, nsb, nchunk, st);
}

template <int R, bool HAS_ZP>
hipError_t launch_ws(const Sizes& s, const mnb_plan& p, const float* A, float* Y, void* ws,
                     int64_t nsb, int64_t nchunk, hipStream_t st) {
  const WsLayout L = ws_layout(nchunk);
  uint8_t* w = static_cast<uint8_t*>(ws);
  const int64_t threads = nchunk * 64 * 4;
  hipLaunchKernelGGL(gemv_prep_a, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, A,
                     s.K, nchunk * 64, reinterpret_cast<uint32_t*>(w + L.dig),
                     reinterpret_cast<int32_t*>(w + L.sums),
                     reinterpret_cast<int32_t*>(w + L.nexp));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nrg = (s.N + R - 1) / R;
  int64_t blocks = nrg;
  const int64_t cap = (int64_t)cu_count() * 8;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL((gemv_int4_ws<R, HAS_ZP>), dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<const uint8_t*>(p.codes), static_cast<const float*>(p.scales),
                     static_cast<const uint32_t*>(p.zeros),
                     reinterpret_cast<const uint32_t*>(w + L.dig),
                     reinterpret_cast<const int32_t*>(w + L.sums),
                     reinterpret_cast<const int32_t*>(w + L.nexp), Y, s.N, s.row_bytes, s.nb, nsb,
                     nchunk, bs_shift_of(s), (int64_t)s.zrow);
  return hipGetLastError();
}

// The plain fp32 path: N <= 32768, K <= 8192, and 32-bit offsets (rows of at
// most 4 KiB of codes)
bool f32_path(const Sizes& s) {
  const int64_t nchunk = (n_subblocks(s) + 63) / 64;
  return nchunk <= kMaxTeam && s.N <= kF32MaxRows && s.row_bytes * s.N < (int64_t(1) << 31);
}

template <bool HAS_ZP>
hipError_t dispatch(const Sizes& s, const mnb_plan& p, const float* A, float* Y, void* ws,
                    hipStream_t st) {
  const int64_t nsb = n_subblocks(s);
  const int64_t nchunk = (nsb + 63) / 64;
  if (nchunk > kMaxTeam) return launch_ws<8, HAS_ZP>(s, p, A, Y, ws, nsb, nchunk, st);
  // up to tens of thousands of rows: the plain fp32 path, two rows per wave
  // (measured faster there; the digit planes pay off on long row streams)
  if (f32_path(s)) return launch_f32<2, HAS_ZP>(s, p, A, Y, nsb, nchunk, st);
  // rows per wave iteration: enough row groups to fill the chip for small N,
  // deeper load batches for large N
  const int64_t teams = kMaxTeam / nchunk;
  const int64_t cap_groups = (int64_t)cu_count() * 4 * teams;
  if ((s.N + 7) / 8 >= cap_groups) return launch_fused<8, HAS_ZP>(s, p, A, Y, nsb, nchunk, st);
  if ((s.N + 3) / 4 >= cap_groups / 2) return launch_fused<4, HAS_ZP>(s, p, A, Y, nsb, nchunk, st);
  return launch_fused<2, HAS_ZP>(s, p, A, Y, nsb, nchunk, st);
}

}  // namespace

bool gemv_multi_fusable(const Sizes* s, int count) {
  if (count < 1 || count > kMaxSegs) return false;
  for (int i = 0; i < count; ++i)
    if (!f32_path(s[i]) || s[i].K != s[0].K || s[i].bs != s[0].bs ||
        (s[i].zeros != 0) != (s[0].zeros != 0))
      return false;
  return true;
}

hipError_t launch_gemv_multi(const Sizes* s, const mnb_plan* const* p, int count, const float* A,
                             float* const* Y, hipStream_t st) {
  const int64_t nsb = n_subblocks(s[0]);
  const int64_t nchunk = (nsb + 63) / 64;
  int64_t N[kMaxSegs];
  for (int i = 0; i < count; ++i) N[i] = s[i].N;
  return s[0].zeros ? launch_f32_segs<2, true>(s[0], p, N, count, A, Y, nsb, nchunk, st)
                    : launch_f32_segs<2, false>(s[0], p, N, count, A, Y, nsb, nchunk, st);
}

uint64_t gemv_ws_bytes(const Sizes& s) {
  const int64_t nchunk = (n_subblocks(s) + 63) / 64;
  return nchunk > kMaxTeam ? ws_layout(nchunk).total : 0;
}

hipError_t launch_gemv(const Sizes& s, const mnb_plan& p, const float* A, float* Y, void* ws,
                       hipStream_t st) {
  return s.zeros ? dispatch<true>(s, p, A, Y, ws, st) : dispatch<false>(s, p, A, Y, ws, st);
}

}  // namespace mnb
