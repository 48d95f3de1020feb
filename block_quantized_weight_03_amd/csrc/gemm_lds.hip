// Large-M prefill GEMM on the compressed INT4 weights, for gfx950.
//
// Operation ("Qwen3 Missing-Kernel Implementation Plan", section "PR
// sequence", step K03: prefill on the same compressed weights):
//   Y[m,n] = sum_{k<K} A[m,k] * (q[n,k] - z[n,b]) * s[n,b],
// with the same rounding as the other matrix-core kernels: A rounded to fp16
// (RN), w = fp16(fma(q, s, -(z*s))) in fp32, fp32 accumulation by
// v_mfma_f32_32x32x16_f16.
//
// Design.  A first kernel rounds A to fp16 into the workspace (read once,
// instead of once per column tile, at half the bytes).  The GEMM then
// streams two operands per 64-wide K stage straight from global memory into
// LDS with global_load_lds_dwordx4 (no staging registers, no VALU): the fp16
// A tile (256 rows x 128 bytes) and the packed codes of the 256 weight rows
// (256 x 32 bytes), plus per-lane scale and zero-point words.  Three LDS stages are in flight; each wave waits for its
// own copies of a stage with an explicit vmcnt, then one barrier publishes
// the stage.  A workgroup of 4 waves computes a 256 x 256 tile of Y; wave w
// owns the 64 output columns [64w, 64w + 64) across all 256 rows (8 x 2
// tiles of 32 x 32, 256 accumulators in AGPRs), so it dequantizes only its
// own weight rows, straight from LDS into MFMA operand registers: every
// weight is dequantized once per 256 rows of A.
//
// K order inside an MFMA is free as long as both operands use the same one:
// lane group g (lanes 32g .. 32g + 31) takes K positions [32g, 32g + 32) of
// the stage, i.e. one 32-code sub-block of the weight row (one scale, one
// zero point), and slice t of the stage takes [32g + 8t, 32g + 8t + 8).
// A rows are 128 bytes in LDS with 16-byte chunk c of row r stored at chunk
// c ^ ((r >> 1) & 7): a 16-byte-per-lane LDS read serves 16 lanes (256 bytes,
// all 64 banks) per cycle, and the 16 lanes of a read (rows r .. r + 15, one
// logical chunk) then cover every bank once.  The swizzle is applied by
// choosing which global chunk each lane copies.

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace mnb {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int kBK = 64;
constexpr int kXcds = 8;
constexpr int64_t kMixChunk = 128;  // blocks per class chunk in the mixed-width dispatch order

// Tile BM x BN (BN = 128 TN): wave w computes all BM rows of columns
// [32 TN w, 32 TN (w + 1)) as TM x TN tiles of 32 x 32.  The shapes used are
// 256 x 256, 256 x 128 and 128 x 128 (128 x 256, 128 x 384 and 256 x 128 on
// their own measured no faster than these at the prefill shapes).
template <int BM, int TN_>
struct Tile {
  static constexpr int TM = BM / 32, TN = TN_, BN = 128 * TN_;
  static constexpr int ABytes = BM * kBK * 2;     // fp16 A per stage (32 / 16 KiB)
  static constexpr int WBytes = BN * kBK / 2;     // packed codes per stage (4 KiB per TN)
  static constexpr int SBytes = 4 * TN * 64 * 4;  // one scale per lane and weight tile
  static constexpr int ACopies = BM / 32;         // 1 KiB A copies per wave and stage
  // LDS stages in flight (for 128-row tiles, 4 and 6 stages measured no
  // faster than 3, which leaves room for two workgroups per CU)
  static constexpr int Stages = 3;
  template <bool HAS_ZP>
  static constexpr int stage_bytes() { return ABytes + WBytes + (HAS_ZP ? 2 : 1) * SBytes; }
};

__device__ __forceinline__ uint32_t cvt_pk_rn(float a, float b) {
  const half2v h = half2v{(_Float16)a, (_Float16)b};  // v_cvt_pk_f16_f32, RN
  return __builtin_bit_cast(uint32_t, h);
}

// global_load_lds_dwordx4 / _dword: lane l writes its 16 (4) bytes at
// lds + 16 l (4 l); the LDS address must be wave-uniform
__device__ __forceinline__ void copy16(const void* src, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr)lds, 16, 0, 0);
}
__device__ __forceinline__ void copy4(const void* src, uint8_t* lds) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr)lds, 4, 0, 0);
}

// Eight weights of one 32-bit code word (nibble e = K position e) as fp16.
__device__ __forceinline__ half8 dequant8(uint32_t x, float s, float nzs) {
  x ^= 0x88888888u;  // stored nibbles are q ^ 8
  uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
  // opaque to the optimizer, so that it converts each byte with one
  // v_cvt_f32_ubyteN instead of re-extracting nibbles from x
  asm("" : "+v"(lo), "+v"(hi));
  uint32_t h[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    h[j] = cvt_pk_rn(fmaf((float)((lo >> (8 * j)) & 0xFFu), s, nzs),
                     fmaf((float)((hi >> (8 * j)) & 0xFFu), s, nzs));
  return __builtin_bit_cast(half8, u32x4{h[0], h[1], h[2], h[3]});
}

// s_waitcnt vmcnt(n) lgkmcnt(0) (gfx9 encoding; expcnt not waited on)
template <int n>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4));
}

__global__ void __launch_bounds__(256) round_a_f16(const float* __restrict__ A,
                                                   _Float16* __restrict__ A16, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(A) + 2 * i);
  const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(A) + 2 * i + 1);
  reinterpret_cast<u32x4*>(A16)[i] =
      u32x4{cvt_pk_rn(a.x, a.y), cvt_pk_rn(a.z, a.w), cvt_pk_rn(b.x, b.y), cvt_pk_rn(b.z, b.w)};
}

// One BM x (128 TN) output tile over the K range [kbeg, kbeg + 64 steps),
// written to out (Y or a split's partial buffer, row stride N), by 4 waves:
// wave w owns the 32 TN columns [32 TN w, 32 TN (w + 1)) of the tile over all
// BM rows.  (Eight waves, two per SIMD, each owning half the rows, measured
// slower: 144 against 135 us at M = 4096, K = 2048, N = 6144, every weight
// then being dequantized by two waves.)
template <bool HAS_ZP, int BM, int TN, int WM = 1>
__device__ __forceinline__ void lds_tile(
    uint8_t* smem, const _Float16* __restrict__ A16, const uint8_t* __restrict__ codes,
    const float* __restrict__ scales, const uint32_t* __restrict__ zeros, float* __restrict__ out,
    int64_t M, int64_t N, int64_t K, int64_t row_bytes, int64_t nb, int32_t bs_shift, int64_t m0,
    int64_t n0, int64_t kbeg, int steps) {
  using T_ = Tile<BM, TN>;
  constexpr int kBM = BM, kBN = T_::BN, kTN = T_::TN;
  constexpr int kTM = T_::TM / WM;          // 32-row tiles per wave
  constexpr int kABytes = T_::ABytes, kWBytes = T_::WBytes, kSBytes = T_::SBytes;
  constexpr int kAC = T_::ACopies / WM;     // 1 KiB A copies per wave and stage
  constexpr int kWC = kTN / WM;             // code (and scale) copies per wave and stage
  static_assert(kTN % WM == 0 && T_::ACopies % WM == 0, "copy split");
  // per stage: [A][codes][scales][zero-point words]
  constexpr int kStageBytes = T_::template stage_bytes<HAS_ZP>();
  constexpr int kGroup = kAC + kWC * (HAS_ZP ? 3 : 2);  // vector-memory ops per stage and wave

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave & 3, wm = wave >> 2;

  // A copies: wave w fills rows [w BM/(4 WM), (w + 1) BM/(4 WM)) of a stage,
  // 8 rows (1 KiB) per instruction; lane l writes physical chunk l & 7 of row
  // 8u + (l >> 3), which holds logical chunk (l & 7) ^ ((row >> 1) & 7).
  // Rows past M are clamped (their results are never stored).
  uint32_t a_off[kAC];  // element offsets into A16; the launcher checks M * K < 2^31
#pragma unroll
  for (int u = 0; u < kAC; ++u) {
    const int r = u * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    int64_t m = m0 + wave * (kBM / (4 * WM)) + r;
    m = m < M ? m : M - 1;
    a_off[u] = (uint32_t)(m * K + 8 * c);
  }
  // Codes, scales and zero points of column group wn (rows past N clamped):
  // this wave copies chunks j = wm kWC .. wm kWC + kWC - 1 of the group's kTN
  // chunks of 32 weight rows.  Codes: 32 rows x 32 bytes per instruction,
  // stored chunk-major (lane l: row l & 31, 16-byte half l >> 5), the order of
  // the operand reads; scale and zero-point word: one dword per lane, for the
  // lane's row and sub-block.
  const int wl_n = lane & 31, wl_g = lane >> 5;
  const uint8_t* w_src[kWC];
  const float* s_row[kWC];
  const uint32_t* z_row[kWC];
#pragma unroll
  for (int jj = 0; jj < kWC; ++jj) {
    int64_t n = n0 + wn * (kBN / 4) + (wm * kWC + jj) * 32 + wl_n;
    n = n < N ? n : N - 1;
    w_src[jj] = codes + n * row_bytes + 16 * wl_g;
    s_row[jj] = scales + n * nb;
    z_row[jj] = HAS_ZP ? zeros + (n >> 3) * nb : nullptr;
  }
  int z_sh[kTN];  // nibble of the zero-point word of this lane's row in chunk j
#pragma unroll
  for (int j = 0; j < kTN; ++j) {
    int64_t n = n0 + wn * (kBN / 4) + j * 32 + wl_n;
    n = n < N ? n : N - 1;
    z_sh[j] = 4 * (int)(n & 7);
  }

  // Starts the copies of stage st (clamped to the last one, so that every
  // stage issues the same number of vector-memory operations) into buffer b.
  auto issue = [&](int st, int b) {
    st = st < steps ? st : steps - 1;
    const int64_t k0 = kbeg + (int64_t)st * kBK;
    uint8_t* base = smem + b * kStageBytes;
#pragma unroll
    for (int u = 0; u < kAC; ++u) copy16(A16 + a_off[u] + k0, base + (wave * kAC + u) * 1024);
    base += kABytes;
    const int chunk0 = wn * kTN + wm * kWC;
#pragma unroll
    for (int jj = 0; jj < kWC; ++jj) copy16(w_src[jj] + (k0 >> 1), base + (chunk0 + jj) * 1024);
    base += kWBytes;
    const int64_t blk = ((k0 >> 5) + wl_g) >> bs_shift;
#pragma unroll
    for (int jj = 0; jj < kWC; ++jj) copy4(s_row[jj] + blk, base + (chunk0 + jj) * 256);
    if (HAS_ZP) {
      base += kSBytes;
#pragma unroll
      for (int jj = 0; jj < kWC; ++jj) copy4(z_row[jj] + blk, base + (chunk0 + jj) * 256);
    }
  };

  f32x16 acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // operand read offsets: A row (lane & 31) of each of this wave's 32-row
  // tiles, chunk (4 * (lane >> 5) + t) ^ ((row >> 1) & 7); per-lane words at
  // lane * 16 / lane * 4
  const int a_rd = (wm * (kBM / WM) + (lane & 31)) * 128;
  const int a_cx = (lane >> 1) & 7, a_cg = 4 * (lane >> 5);

  auto read_a = [&](half8 (&af)[kTM], const uint8_t* abase, int t) {
    const int coff = ((a_cg + t) ^ a_cx) << 4;
#pragma unroll
    for (int i = 0; i < kTM; ++i)
      af[i] = *reinterpret_cast<const half8*>(abase + i * 32 * 128 + a_rd + coff);
  };

  // Slices are software-pipelined: while the MFMAs of slice t run, the A
  // operands of slice t + 1 are read from LDS and its weights dequantized.
  auto compute = [&](int b) {
    const uint8_t* abase = smem + b * kStageBytes;
    const uint8_t* wbase = abase + kABytes + wn * (kTN * 1024) + lane * 16;
    const uint8_t* sbase = abase + kABytes + kWBytes + wn * (kTN * 256) + lane * 4;
    u32x4 wc[kTN];
    float sc[kTN], nzs[kTN];
    half8 af[2][kTM], bf[2][kTN];
    read_a(af[0], abase, 0);
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      wc[j] = *reinterpret_cast<const u32x4*>(wbase + j * 1024);
      sc[j] = *reinterpret_cast<const float*>(sbase + j * 256);
      float z = 8.0f;
      if (HAS_ZP) z = (float)((*reinterpret_cast<const uint32_t*>(sbase + kSBytes + j * 256) >>
                               z_sh[j]) & 15u);
      nzs[j] = -(z * sc[j]);
      bf[0][j] = dequant8(wc[j][0], sc[j], nzs[j]);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int c = t & 1;
      __builtin_amdgcn_sched_barrier(0);
      if (t < 3) {
        read_a(af[c ^ 1], abase, t + 1);
#pragma unroll
        for (int j = 0; j < kTN; ++j) bf[c ^ 1][j] = dequant8(wc[j][t + 1], sc[j], nzs[j]);
      }
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[c][i], bf[c][j], acc[i][j], 0, 0, 0);
      if (t < 3) {
        // one MFMA, then a share of the next slice's VALU and LDS reads
#pragma unroll
        for (int q = 0; q < kTM * kTN; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, (24 * kTN + kTM * kTN - 1) / (kTM * kTN), 0);  // VALU
          if ((q % kTN) == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Per stage s (buffer b = s mod S for S stages): wait for this wave's
  // copies of stage s (the newer groups, of stages s + 1 .. s + S - 2, may stay
  // in flight) and for its LDS reads of stage s - 1; publish with a barrier;
  // refill the buffer of stage s - 1 with stage s + S - 1; compute stage s.
  constexpr int S = T_::Stages;
  static_assert((S - 2) * kGroup < 64, "vmcnt range");
#pragma unroll
  for (int i = 0; i < S - 1; ++i) issue(i, i);
  int b = 0;
  for (int s = 0; s < steps; ++s) {
    wait_vm_lgkm0<(S - 2) * kGroup>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    issue(s + S - 1, b == 0 ? S - 1 : b - 1);
    compute(b);
    b = b == S - 1 ? 0 : b + 1;
  }
  // drain the copies still in flight before the workgroup's LDS is released
  wait_vm_lgkm0<0>();

  // streamed out once (nontemporal: measured 2-5% faster than plain stores);
  // tiles wholly inside Y store without per-element bounds checks
  const int64_t mw = m0 + wm * (kBM / WM);  // this wave's first row
  const bool whole = m0 + kBM <= M && n0 + kBN <= N;  // uniform
  float* tile_out = out + (mw + 4 * (lane >> 5)) * N + n0 + wn * (kBN / 4) + (lane & 31);
  if (whole) {
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __builtin_nontemporal_store(
              acc[i][j][r], tile_out + (int64_t)(i * 32 + 8 * (r >> 2) + (r & 3)) * N + j * 32);
  } else {
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
      for (int j = 0; j < kTN; ++j) {
        const int64_t col = n0 + wn * (kBN / 4) + j * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = mw + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row < M && col < N) __builtin_nontemporal_store(acc[i][j][r], out + row * N + col);
        }
      }
  }
}

// One tile shape over the whole of Y, K split `splits` ways: XCD x (=
// blockIdx % 8) takes work items [x * per, (x + 1) * per).
template <bool HAS_ZP, int BM, int TN>
__global__ void __launch_bounds__(256) gemm_int4_lds(
    const _Float16* __restrict__ A16, const uint8_t* __restrict__ codes,
    const float* __restrict__ scales, const uint32_t* __restrict__ zeros, float* __restrict__ Y,
    float* __restrict__ part, int64_t M, int64_t N, int64_t K, int64_t row_bytes, int64_t nb,
    int32_t bs_shift, int64_t tiles_n, int64_t work, int32_t splits, int64_t kc) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int64_t per = (work + kXcds - 1) / kXcds;
  const int64_t L = (int64_t)(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (L >= work) return;  // whole workgroup
  const int split = (int)(L % splits);
  const int64_t tile = L / splits;
  const int64_t kbeg = split * kc;
  const int64_t kend = kbeg + kc < K ? kbeg + kc : K;
  float* out = splits > 1 ? part + (int64_t)split * M * N : Y;
  lds_tile<HAS_ZP, BM, TN>(smem, A16, codes, scales, zeros, out, M, N, K, row_bytes, nb, bs_shift,
                           (tile / tiles_n) * BM, (tile % tiles_n) * (128 * TN), kbeg,
                           (int)((kend - kbeg) / kBK));
}

// Two tile widths in one launch, whole K: columns [0, n_split) in BM x (128
// TN0) tiles (the first work0 workgroups, dispatched first), the rest in
// BM x (128 TN1) tiles.  With as many wide tiles as CUs, the narrow ones fill
// the second round, which then takes about half as long instead of leaving
// CUs idle.  Within each class XCD x takes a contiguous range of its tiles.
template <bool HAS_ZP, int BM, int TN0, int TN1>
__global__ void __launch_bounds__(256) gemm_int4_lds_mix(
    const _Float16* __restrict__ A16, const uint8_t* __restrict__ codes,
    const float* __restrict__ scales, const uint32_t* __restrict__ zeros, float* __restrict__ Y,
    int64_t M, int64_t N, int64_t K, int64_t row_bytes, int64_t nb, int32_t bs_shift,
    int64_t n_split, int64_t tiles_n0, int64_t work0, int64_t blocks0, int64_t tiles_n1,
    int64_t work1) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int steps = (int)(K / kBK);
  // Dispatch order: chunks of kMixChunk blocks of the two classes alternate
  // while both last, then the rest of each class, so that a round holds both
  // tile widths and the narrow tiles' outputs leave while wide tiles still
  // compute (measured at M = 4096, K = 2048, N = 6144: 125.4/126.6 ->
  // 123.4/123.8 us against all wide tiles first).  The chunk is a multiple
  // of the XCD count, so a block keeps its XCD (b mod 8) and each class still
  // reaches every XCD in contiguous runs.
  int64_t b = blockIdx.x;
  {
    const int64_t blocks1 = (work1 + kXcds - 1) / kXcds * kXcds;
    const int64_t mq = ((blocks0 < blocks1 ? blocks0 : blocks1) / kMixChunk) * kMixChunk;
    if (b < 2 * mq) {
      const int64_t c = (b / (2 * kMixChunk)) * kMixChunk + b % kMixChunk;
      b = (b / kMixChunk) % 2 == 0 ? c : blocks0 + c;
    } else {
      const int64_t r = b - 2 * mq;
      b = r < blocks0 - mq ? mq + r : blocks0 + mq + (r - (blocks0 - mq));
    }
  }
  if (b < blocks0) {
    const int64_t per = blocks0 / kXcds;
    const int64_t L = (b % kXcds) * per + b / kXcds;
    if (L >= work0) return;
    lds_tile<HAS_ZP, BM, TN0>(smem, A16, codes, scales, zeros, Y, M, N, K, row_bytes, nb, bs_shift,
                              (L / tiles_n0) * BM, (L % tiles_n0) * (128 * TN0), 0, steps);
  } else {
    const int64_t b1 = b - blocks0;
    const int64_t per = (work1 + kXcds - 1) / kXcds;
    const int64_t L = (b1 % kXcds) * per + b1 / kXcds;
    if (L >= work1) return;
    lds_tile<HAS_ZP, BM, TN1>(smem, A16, codes, scales, zeros, Y, M, N, K, row_bytes, nb, bs_shift,
                              (L / tiles_n1) * BM, n_split + (L % tiles_n1) * (128 * TN1), 0, steps);
  }
}

template <bool HAS_ZP, int BM, int TN0, int TN1>
hipError_t launch_mix(const Sizes& s, const mnb_plan& p, int64_t M, const _Float16* A16, float* Y,
                      int64_t n_split, hipStream_t st) {
  using T0 = Tile<BM, TN0>;
  using T1 = Tile<BM, TN1>;
  const int64_t rows = (M + BM - 1) / BM;
  const int64_t tiles_n0 = n_split / T0::BN, work0 = rows * tiles_n0;
  const int64_t blocks0 = (work0 + kXcds - 1) / kXcds * kXcds;
  const int64_t tiles_n1 = (s.N - n_split + T1::BN - 1) / T1::BN, work1 = rows * tiles_n1;
  const int64_t blocks = blocks0 + (work1 + kXcds - 1) / kXcds * kXcds;
  if (blocks > 0x7FFFFFFF || n_split % T0::BN || n_split >= s.N) return hipErrorInvalidValue;
  const size_t l0 = (size_t)T0::Stages * T0::template stage_bytes<HAS_ZP>();
  const size_t l1 = (size_t)T1::Stages * T1::template stage_bytes<HAS_ZP>();
  hipLaunchKernelGGL((gemm_int4_lds_mix<HAS_ZP, BM, TN0, TN1>), dim3((unsigned)blocks), dim3(256),
                     l0 > l1 ? l0 : l1, st, A16, static_cast<const uint8_t*>(p.codes),
                     static_cast<const float*>(p.scales), static_cast<const uint32_t*>(p.zeros), Y,
                     M, s.N, s.K, s.row_bytes, s.nb, s.bs == 32 ? 0 : (s.bs == 64 ? 1 : 2), n_split,
                     tiles_n0, work0, blocks0, tiles_n1, work1);
  return hipGetLastError();
}

template <bool HAS_ZP, int BM, int TN>
hipError_t launch_tile(const Sizes& s, const mnb_plan& p, int64_t M, const _Float16* A16, float* Y,
                       float* part, int32_t splits, int64_t kc, hipStream_t st) {
  using T_ = Tile<BM, TN>;
  const int64_t tiles_n = (s.N + T_::BN - 1) / T_::BN;
  const int64_t work = ((M + BM - 1) / BM) * tiles_n * splits;
  const int64_t blocks = (work + kXcds - 1) / kXcds * kXcds;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const size_t lds = (size_t)T_::Stages * T_::template stage_bytes<HAS_ZP>();
  hipLaunchKernelGGL((gemm_int4_lds<HAS_ZP, BM, TN>), dim3((unsigned)blocks), dim3(256), lds, st,
                     A16, static_cast<const uint8_t*>(p.codes),
                     static_cast<const float*>(p.scales), static_cast<const uint32_t*>(p.zeros), Y,
                     part, M, s.N, s.K, s.row_bytes, s.nb, s.bs == 32 ? 0 : (s.bs == 64 ? 1 : 2),
                     tiles_n, work, splits, kc);
  return hipGetLastError();
}

template <int BM, int TN>
hipError_t launch_tile_zp(const Sizes& s, const mnb_plan& p, int64_t M, const _Float16* A16, float* Y,
                          float* part, int32_t splits, int64_t kc, hipStream_t st) {
  return s.zeros ? launch_tile<true, BM, TN>(s, p, M, A16, Y, part, splits, kc, st)
                 : launch_tile<false, BM, TN>(s, p, M, A16, Y, part, splits, kc, st);
}

}  // namespace

bool gemm_lds_supported(const Sizes& s, int64_t M) {
  return M > 0 && (s.K % kBK) == 0 && (uint64_t)M * (uint64_t)s.K < (1ull << 31);
}

uint64_t gemm_lds_a16_bytes(const Sizes& s, int64_t M) {
  return align256((uint64_t)M * (uint64_t)s.K * 2);
}

hipError_t launch_gemm_lds(const Sizes& s, const mnb_plan& p, int64_t M, const float* A,
                           void* ws, float* Y, float* part, int32_t splits, int64_t kc, int bm,
                           int tn, int64_t n_split, hipStream_t st) {
  _Float16* A16 = static_cast<_Float16*>(ws);
  const int64_t n8 = M * s.K / 8;
  hipLaunchKernelGGL(round_a_f16, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, A, A16,
                     n8);
  if (n_split > 0)  // 256 x 256 tiles up to column n_split, then 256 x 128
    return s.zeros ? launch_mix<true, 256, 2, 1>(s, p, M, A16, Y, n_split, st)
                   : launch_mix<false, 256, 2, 1>(s, p, M, A16, Y, n_split, st);
  if (bm == 128) return launch_tile_zp<128, 1>(s, p, M, A16, Y, part, splits, kc, st);
  if (bm == 256 && tn == 1) return launch_tile_zp<256, 1>(s, p, M, A16, Y, part, splits, kc, st);
  if (bm == 256) return launch_tile_zp<256, 2>(s, p, M, A16, Y, part, splits, kc, st);
  return hipErrorInvalidValue;
}

}  // namespace mnb
