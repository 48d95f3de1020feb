// TEST INFRASTRUCTURE ONLY -- fp64 CPU reference for MatMulNBits, the QMoE layer and the INT3 RTN quantizer.
//
// Plain, slow and meant to be read against the pages (see oracle.h for the
// source list).  Every quantity is computed in double precision and rounded
// once at the end.  No blocking, fusion or reordering beyond the definitions:
// each weight row is dequantized into an fp64 buffer and then used in plain
// sequential dot products.
//
// Readings taken where the pages are silent (each repeated where it is used):
//  * a 4-bit byte holds the even position in its low nibble (row-local
//    LSB-first packing at width 4);
//  * the implicit zero point is 2^(bits-1): 8 for INT4, 4 for INT3;
//  * explicit dense zero points are packed like the codes, one per block;
//  * positions k >= K in the last block are never read;
//  * FC1 rows alternate gate (even) and up (odd);
//  * SwiGLU is silu(g) * u with no extra constants;
//  * top-k ties go to the lower expert index.

#include "oracle.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <numeric>
#include <thread>
#include <vector>

namespace {

// Bit i of a row sits in byte i >> 3 at bit position i & 7; code j is the
// little-endian value of bits [bits*j, bits*j + bits) ([P0], row-local
// LSB-first UINT8 packing).
unsigned code_at(const uint8_t* row, int64_t j, int bits) {
  unsigned v = 0;
  for (int t = 0; t < bits; ++t) {
    const int64_t bit = (int64_t)bits * j + t;
    const unsigned b = (row[bit >> 3] >> (bit & 7)) & 1u;
    v |= b << t;
  }
  return v;
}

bool bits_ok(int bits) { return bits >= 1 && bits <= 8; }

template <class F>
void parallel_for(int64_t n, int nthreads, F f) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads == 1 || n < 2) {
    f(0, n);
    return;
  }
  const int64_t nt = std::min<int64_t>(nthreads, n);
  std::vector<std::thread> pool;
  for (int64_t t = 0; t < nt; ++t) {
    const int64_t lo = n * t / nt, hi = n * (t + 1) / nt;
    pool.emplace_back([=] { f(lo, hi); });
  }
  for (auto& th : pool) th.join();
}

double sigmoid(double v) { return 1.0 / (1.0 + std::exp(-v)); }

// Dense MatMulNBits row dequantization ([PLAN K01]): block b of row n holds
// bs codes in bs*bits/8 bytes; w = (q - z) * scale[n*nb + b], valid only for
// k < K.  The product of a small integer and an fp32 value is exact in fp64.
void dense_row(int64_t n, int64_t K, int bits, int bs, const uint8_t* B,
               const float* scales, const uint8_t* zp, double* w,
               uint8_t* codes_out, uint8_t* zeros_out) {
  const int64_t nb = (K + bs - 1) / bs;
  const int64_t block_bytes = (int64_t)bs * bits / 8;
  const int64_t zrow = (nb * bits + 7) / 8;
  for (int64_t b = 0; b < nb; ++b) {
    const uint8_t* blk = B + (n * nb + b) * block_bytes;
    const unsigned z = zp ? code_at(zp + n * zrow, b, bits) : (1u << (bits - 1));
    if (zeros_out) zeros_out[n * nb + b] = (uint8_t)z;
    const double s = scales ? (double)scales[n * nb + b] : 0.0;
    const int64_t valid = std::min<int64_t>(bs, K - b * bs);
    for (int64_t j = 0; j < valid; ++j) {
      const unsigned q = code_at(blk, j, bits);
      if (codes_out) codes_out[n * K + b * bs + j] = (uint8_t)q;
      if (w) w[b * bs + j] = ((double)q - (double)z) * s;
    }
  }
}

bool dense_args_ok(int64_t K, int64_t N, int bits, int bs) {
  return K >= 1 && N >= 1 && bits_ok(bits) && bs >= 1 && ((int64_t)bs * bits) % 8 == 0;
}

// INT3 QMoE row dequantization ([P0], [OLIVE]): a row of K codes is one
// row-local LSB-first bit stream of ceil(bits*K/8) bytes; block b of the row
// uses scale s[b]; w = (q - 2^(bits-1)) * s.
// A 16-bit activation / scale / bias value: IEEE binary16 (dtype 0) or
// bfloat16 (dtype 1), widened exactly.
double h16(uint16_t v, int dtype) { return dtype ? orc_bf16_to_f64(v) : orc_f16_to_f64(v); }

void moe_row(const uint8_t* row, const uint16_t* s, int64_t K, int bits, int bs, int dtype,
             double* w) {
  const double z = (double)(1u << (bits - 1));
  for (int64_t k = 0; k < K; ++k) {
    const double q = (double)code_at(row, k, bits);
    w[k] = (q - z) * h16(s[k / bs], dtype);
  }
}

}  // namespace

extern "C" {

int orc_unpack_bits(const uint8_t* row, int64_t n_codes, int bits, uint8_t* codes) {
  if (!bits_ok(bits) || n_codes < 0 || (n_codes && (!row || !codes))) return -1;
  for (int64_t j = 0; j < n_codes; ++j) codes[j] = (uint8_t)code_at(row, j, bits);
  return 0;
}

int orc_pack_bits(const uint8_t* codes, int64_t n_codes, int bits, uint8_t* row) {
  if (!bits_ok(bits) || n_codes < 0 || (n_codes && (!row || !codes))) return -1;
  const int64_t nbytes = (n_codes * bits + 7) / 8;
  std::memset(row, 0, (size_t)nbytes);
  for (int64_t j = 0; j < n_codes; ++j) {
    const unsigned c = codes[j];
    if (c >> bits) return -2;  // code does not fit the width
    for (int t = 0; t < bits; ++t) {
      const int64_t bit = (int64_t)bits * j + t;
      row[bit >> 3] = (uint8_t)(row[bit >> 3] | (((c >> t) & 1u) << (bit & 7)));
    }
  }
  return 0;
}

int orc_padding_is_canonical(const uint8_t* row, int64_t n_codes, int bits) {
  if (!bits_ok(bits) || n_codes < 0) return -1;
  const int64_t total = n_codes * bits;
  const int used = (int)(total % 8);
  if (used == 0) return 1;
  const uint8_t last = row[total / 8];
  return (last >> used) == 0 ? 1 : 0;
}

// IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
double orc_f16_to_f64(uint16_t h) {
  const int sign = h >> 15;
  const int e = (h >> 10) & 31;
  const int m = h & 1023;
  double v;
  if (e == 0)
    v = std::ldexp((double)m, -24);
  else if (e == 31)
    v = m ? std::nan("") : INFINITY;
  else
    v = std::ldexp((double)(1024 + m), e - 25);
  return sign ? -v : v;
}

// Round to nearest, ties to even, with overflow to infinity.
uint16_t orc_f64_to_f16(double x) {
  const uint16_t sign = std::signbit(x) ? 0x8000 : 0;
  if (std::isnan(x)) return (uint16_t)(sign | 0x7E00);
  const double a = std::fabs(x);
  if (a >= 65520.0) return (uint16_t)(sign | 0x7C00);  // halfway to 2^16 and beyond
  if (a < std::ldexp(1.0, -14)) {
    // subnormal: multiples of 2^-24; rounding up to 1024 yields the smallest normal
    const double q = std::nearbyint(std::ldexp(a, 24));
    return (uint16_t)(sign | (uint16_t)q);
  }
  int E;
  std::frexp(a, &E);  // a = f * 2^E, f in [0.5, 1)
  int exp = E - 1;    // a in [2^exp, 2^(exp+1))
  double m = std::nearbyint((std::ldexp(a, -exp) - 1.0) * 1024.0);
  if (m >= 1024.0) {
    m = 0.0;
    exp += 1;
  }
  if (exp > 15) return (uint16_t)(sign | 0x7C00);
  return (uint16_t)(sign | (uint16_t)((exp + 15) << 10) | (uint16_t)m);
}

// bfloat16: the top 16 bits of an IEEE binary32 (1 sign bit, 8 exponent bits,
// 7 fraction bits).
double orc_bf16_to_f64(uint16_t b) {
  const int sign = b >> 15;
  const int e = (b >> 7) & 255;
  const int m = b & 127;
  double v;
  if (e == 0)
    v = std::ldexp((double)m, -133);  // subnormal: m * 2^(1 - 127 - 7)
  else if (e == 255)
    v = m ? std::nan("") : INFINITY;
  else
    v = std::ldexp((double)(128 + m), e - 134);
  return sign ? -v : v;
}

// Round to nearest, ties to even, with overflow to infinity.
uint16_t orc_f64_to_bf16(double x) {
  const uint16_t sign = std::signbit(x) ? 0x8000 : 0;
  if (std::isnan(x)) return (uint16_t)(sign | 0x7FC0);
  const double a = std::fabs(x);
  // the largest finite bf16 is (2 - 2^-7) 2^127; halfway to 2^128 rounds up
  if (a >= std::ldexp(2.0 - std::ldexp(1.0, -8), 127)) return (uint16_t)(sign | 0x7F80);
  if (a < std::ldexp(1.0, -126)) {
    // subnormal: multiples of 2^-133; rounding up to 128 yields the smallest normal
    const double q = std::nearbyint(std::ldexp(a, 133));
    return (uint16_t)(sign | (uint16_t)q);
  }
  int E;
  std::frexp(a, &E);
  int exp = E - 1;
  double m = std::nearbyint((std::ldexp(a, -exp) - 1.0) * 128.0);
  if (m >= 128.0) {
    m = 0.0;
    exp += 1;
  }
  if (exp > 127) return (uint16_t)(sign | 0x7F80);
  return (uint16_t)(sign | (uint16_t)((exp + 127) << 7) | (uint16_t)m);
}

int orc_bf16_to_f64_array(const uint16_t* h, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_to_f64(h[i]);
  return 0;
}

int orc_f64_to_bf16_array(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f64_to_bf16(x[i]);
  return 0;
}

int orc_f16_to_f64_array(const uint16_t* h, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_to_f64(h[i]);
  return 0;
}

int orc_f64_to_f16_array(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f64_to_f16(x[i]);
  return 0;
}

int orc_mnb_codes(int64_t K, int64_t N, int bits, int bs, const uint8_t* B,
                  const uint8_t* zp, uint8_t* codes, uint8_t* zeros) {
  if (!dense_args_ok(K, N, bits, bs) || !B) return -1;
  for (int64_t n = 0; n < N; ++n)
    dense_row(n, K, bits, bs, B, nullptr, zp, nullptr, codes, zeros);
  return 0;
}

int orc_mnb_dequant(int64_t K, int64_t N, int bits, int bs, const uint8_t* B,
                    const float* scales, const uint8_t* zp, double* W) {
  if (!dense_args_ok(K, N, bits, bs) || !B || !scales || !W) return -1;
  for (int64_t n = 0; n < N; ++n)
    dense_row(n, K, bits, bs, B, scales, zp, W + n * K, nullptr, nullptr);
  return 0;
}

// Y[m,n] = sum_k A[m,k] * w[n,k] in fp64 ([PLAN K02] for M = 1, [PLAN K03]
// for M > 1: the same compressed weights).  Each row is dequantized once and
// reused across the M rows of A.
int orc_mnb_gemm(int64_t M, int64_t K, int64_t N, int bits, int bs,
                 const float* A, const uint8_t* B, const float* scales,
                 const uint8_t* zp, float* Y, double* Y64, double* S,
                 int nthreads) {
  if (M < 0 || !dense_args_ok(K, N, bits, bs) || !B || !scales || (M && !A)) return -1;
  parallel_for(N, nthreads, [&](int64_t lo, int64_t hi) {
    std::vector<double> w((size_t)K);
    for (int64_t n = lo; n < hi; ++n) {
      dense_row(n, K, bits, bs, B, scales, zp, w.data(), nullptr, nullptr);
      for (int64_t m = 0; m < M; ++m) {
        const float* a = A + m * K;
        double acc = 0.0, sabs = 0.0;
        for (int64_t k = 0; k < K; ++k) {
          const double p = (double)a[k] * w[(size_t)k];
          acc += p;
          sabs += std::fabs(p);
        }
        if (Y) Y[m * N + n] = (float)acc;
        if (Y64) Y64[m * N + n] = acc;
        if (S) S[m * N + n] = sabs;
      }
    }
  });
  return 0;
}

// [ROUTE]: fp32 softmax over E, top-k, renormalize.  Because softmax is
// monotone, the top-k of the probabilities is the top-k of the logits, and the
// renormalized probabilities equal a softmax over the selected logits, which
// is what is evaluated here (in fp64).
int orc_route(int64_t T, int E, int k, const float* logits, int32_t* ids,
              double* weights) {
  if (T < 0 || E < 1 || k < 1 || k > E || (T && (!logits || !ids || !weights))) return -1;
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * E;
    for (int e = 0; e < E; ++e)
      if (!std::isfinite(l[e])) return -2;
    std::vector<int> idx((size_t)E);
    std::iota(idx.begin(), idx.end(), 0);
    std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) { return l[a] > l[b]; });
    const double lmax = (double)l[idx[0]];
    double den = 0.0;
    for (int j = 0; j < k; ++j) den += std::exp((double)l[idx[(size_t)j]] - lmax);
    for (int j = 0; j < k; ++j) {
      ids[t * k + j] = idx[(size_t)j];
      weights[t * k + j] = std::exp((double)l[idx[(size_t)j]] - lmax) / den;
    }
  }
  return 0;
}

// INT3 QMoE layer ([P0], [P1], [OLIVE], [ROUTE]), token by token:
//   route -> for each selected expert e:
//     g_i = x . w1[e][2i],  u_i = x . w1[e][2i+1],  h_i = g_i * sigmoid(g_i) * u_i
//     y_e[n] = h . w2[e][n]
//   out[t][n] = sum_j r_j * y_{e_j}[n], rounded once to fp16.
// S is the first-order propagation of per-product rounding through SwiGLU:
//   S[t][n] = sum_j r_j sum_i |w2[n][i]| (|h_i| + |dh/dg| gs_i + |dh/du| us_i)
// with gs_i = sum_k |x_k w1[2i][k]| and us_i = sum_k |x_k w1[2i+1][k]|.
int orc_qmoe(int64_t T, int64_t H, int64_t I, int E, int k, int bits1,
             int bits2, int bs, int dtype, const uint16_t* x, const float* logits,
             const uint8_t* W1, const uint16_t* s1, const uint8_t* W2,
             const uint16_t* s2, const uint16_t* b1, const uint16_t* b2,
             uint16_t* out16, double* out64, double* S,
             int32_t* ids, double* r, double* g, double* u, double* h,
             double* gs, double* us, int nthreads) {
  if (T < 0 || H < 1 || I < 1 || E < 1 || k < 1 || k > E || !bits_ok(bits1) ||
      !bits_ok(bits2) || bs < 1 || H % bs || I % bs || (dtype != 0 && dtype != 1))
    return -1;
  if (T == 0) return 0;
  if (!x || !logits || !W1 || !s1 || !W2 || !s2) return -1;
  std::vector<int32_t> rid((size_t)(T * k));
  std::vector<double> rw((size_t)(T * k));
  const int rc = orc_route(T, E, k, logits, rid.data(), rw.data());
  if (rc) return rc;
  const int64_t rb1 = (bits1 * H + 7) / 8, rb2 = (bits2 * I + 7) / 8;
  const int64_t nb1 = H / bs, nb2 = I / bs;
  parallel_for(T, nthreads, [&](int64_t lo, int64_t hi) {
    std::vector<double> xd((size_t)H), wg((size_t)H), wu((size_t)H), w2((size_t)I);
    std::vector<double> gv((size_t)I), uv((size_t)I), hv((size_t)I), gsv((size_t)I), usv((size_t)I);
    std::vector<double> acc((size_t)H), sacc((size_t)H);
    for (int64_t t = lo; t < hi; ++t) {
      for (int64_t c = 0; c < H; ++c) xd[(size_t)c] = h16(x[t * H + c], dtype);
      std::fill(acc.begin(), acc.end(), 0.0);
      std::fill(sacc.begin(), sacc.end(), 0.0);
      for (int j = 0; j < k; ++j) {
        const int64_t e = rid[(size_t)(t * k + j)];
        const double rj = rw[(size_t)(t * k + j)];
        for (int64_t i = 0; i < I; ++i) {
          const int64_t rg = e * 2 * I + 2 * i, ru = rg + 1;
          moe_row(W1 + rg * rb1, s1 + rg * nb1, H, bits1, bs, dtype, wg.data());
          moe_row(W1 + ru * rb1, s1 + ru * nb1, H, bits1, bs, dtype, wu.data());
          // an optional bias is one more product term, 1 * b ([P1] optional biases)
          double gg = 0, uu = 0, sg = 0, su = 0;
          if (b1) {
            gg = h16(b1[rg], dtype);
            uu = h16(b1[ru], dtype);
            sg = std::fabs(gg);
            su = std::fabs(uu);
          }
          for (int64_t c = 0; c < H; ++c) {
            gg += xd[(size_t)c] * wg[(size_t)c];
            uu += xd[(size_t)c] * wu[(size_t)c];
            sg += std::fabs(xd[(size_t)c] * wg[(size_t)c]);
            su += std::fabs(xd[(size_t)c] * wu[(size_t)c]);
          }
          gv[(size_t)i] = gg;
          uv[(size_t)i] = uu;
          gsv[(size_t)i] = sg;
          usv[(size_t)i] = su;
          hv[(size_t)i] = gg * sigmoid(gg) * uu;
        }
        for (int64_t n = 0; n < H; ++n) {
          const int64_t row = e * H + n;
          moe_row(W2 + row * rb2, s2 + row * nb2, I, bits2, bs, dtype, w2.data());
          double y = 0, sy = 0;
          if (b2) {
            y = h16(b2[row], dtype);
            sy = std::fabs(y);
          }
          for (int64_t i = 0; i < I; ++i) {
            const double gi = gv[(size_t)i], ui = uv[(size_t)i];
            const double sgm = sigmoid(gi);
            const double dg = ui * sgm * (1.0 + gi * (1.0 - sgm));
            const double du = gi * sgm;
            y += hv[(size_t)i] * w2[(size_t)i];
            sy += std::fabs(w2[(size_t)i]) *
                  (std::fabs(hv[(size_t)i]) + std::fabs(dg) * gsv[(size_t)i] +
                   std::fabs(du) * usv[(size_t)i]);
          }
          acc[(size_t)n] += rj * y;
          sacc[(size_t)n] += rj * sy;
        }
        const size_t base = (size_t)((t * k + j) * I);
        for (int64_t i = 0; i < I; ++i) {
          if (g) g[base + (size_t)i] = gv[(size_t)i];
          if (u) u[base + (size_t)i] = uv[(size_t)i];
          if (h) h[base + (size_t)i] = hv[(size_t)i];
          if (gs) gs[base + (size_t)i] = gsv[(size_t)i];
          if (us) us[base + (size_t)i] = usv[(size_t)i];
        }
      }
      for (int64_t n = 0; n < H; ++n) {
        if (out64) out64[t * H + n] = acc[(size_t)n];
        if (out16)
          out16[t * H + n] = dtype ? orc_f64_to_bf16(acc[(size_t)n]) : orc_f64_to_f16(acc[(size_t)n]);
        if (S) S[t * H + n] = sacc[(size_t)n];
      }
    }
  });
  for (int64_t i = 0; i < T * k; ++i) {
    if (ids) ids[i] = rid[(size_t)i];
    if (r) r[i] = rw[(size_t)i];
  }
  return 0;
}

int orc_qmoe_fc2(int64_t T, int64_t H, int64_t I, int E, int k, int bits2,
                 int bs, int dtype, const int32_t* ids, const double* h, const uint8_t* W2,
                 const uint16_t* s2, const uint16_t* b2, double* y, double* yS,
                 int nthreads) {
  if (T < 0 || H < 1 || I < 1 || E < 1 || k < 1 || !bits_ok(bits2) || bs < 1 || I % bs ||
      (dtype != 0 && dtype != 1))
    return -1;
  if (T == 0) return 0;
  if (!ids || !h || !W2 || !s2 || !y) return -1;
  const int64_t rb2 = (bits2 * I + 7) / 8, nb2 = I / bs;
  for (int64_t i = 0; i < T * k; ++i)
    if (ids[i] < 0 || ids[i] >= E) return -2;
  parallel_for(T * k, nthreads, [&](int64_t lo, int64_t hi) {
    std::vector<double> w2((size_t)I);
    for (int64_t tj = lo; tj < hi; ++tj) {
      const int64_t e = ids[tj];
      const double* hv = h + tj * I;
      for (int64_t n = 0; n < H; ++n) {
        const int64_t row = e * H + n;
        moe_row(W2 + row * rb2, s2 + row * nb2, I, bits2, bs, dtype, w2.data());
        double acc = 0, sa = 0;
        if (b2) {
          acc = h16(b2[row], dtype);
          sa = std::fabs(acc);
        }
        for (int64_t i = 0; i < I; ++i) {
          acc += hv[i] * w2[(size_t)i];
          sa += std::fabs(hv[i] * w2[(size_t)i]);
        }
        y[tj * H + n] = acc;
        if (yS) yS[tj * H + n] = sa;
      }
    }
  });
  return 0;
}

}  // extern "C"

// INT3 RTN producer quantizer ([OLIVE]: scale max|w| / 3.5, zero point 4,
// all-zero group scale 1 / 3.5 with code 4, non-finite weights and scales
// that round to zero rejected; [P0]: stored-scale rounding).  The decisions
// (the scale's fp16 rounding and each code's rounding) are taken in fp32, as
// a producer working on fp32 weights does; see oracle.h.
int orc_rtn_int3(int64_t rows, int64_t K, int bs, int dtype, const float* W, uint8_t* B,
                 uint16_t* scales, uint8_t* status) {
  if (rows < 0 || K < 1 || bs < 1 || K % bs || (dtype != 0 && dtype != 1) ||
      (rows && (!W || !B || !scales || !status)))
    return -1;
  // the stored scale type: fp16 (exponent field 0x7C00) or bf16 (0x7F80)
  auto store = [dtype](float v) { return dtype ? orc_f64_to_bf16((double)v) : orc_f64_to_f16((double)v); };
  const uint16_t inf_bits = dtype ? 0x7F80 : 0x7C00;
  const int64_t nb = K / bs, rb = (3 * K + 7) / 8;
  std::vector<uint8_t> codes(K);
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const float* g = W + r * K + b * bs;
      bool finite = true;
      float amax = 0.0f;
      for (int j = 0; j < bs; ++j) {
        if (!std::isfinite(g[j]))
          finite = false;
        else
          amax = std::max(amax, std::fabs(g[j]));
      }
      uint8_t st = 0;
      uint16_t s16 = 0;
      if (!finite) {
        st = 1;
      } else if (amax == 0.0f) {
        s16 = store(1.0f / 3.5f);
      } else {
        const float s = amax / 3.5f;
        s16 = store(s);  // fp32 -> fp64 is exact: one rounding
        if ((s16 & 0x7FFF) == 0) st = 2;
        else if ((s16 & 0x7FFF) == inf_bits) st = 3;
      }
      if (st) s16 = 0;
      const float sd = (float)(dtype ? orc_bf16_to_f64(s16) : orc_f16_to_f64(s16));
      for (int j = 0; j < bs; ++j) {
        int q = 4;
        if (!st) {
          const float t = g[j] / sd;
          q = (int)std::nearbyint(t) + 4;
          q = std::min(7, std::max(0, q));
        }
        codes[b * bs + j] = (uint8_t)q;
      }
      scales[r * nb + b] = s16;
      status[r * nb + b] = st;
    }
    if (orc_pack_bits(codes.data(), K, 3, B + r * rb) != 0) return -2;
  }
  return 0;
}
