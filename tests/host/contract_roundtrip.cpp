// Host harness: descriptor checks, content validation, prepack into an
// exact-size buffer and unpack round trip over dense and QMoE shapes (run
// under AddressSanitizer / UBSan).
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>
#include "contract.h"
using namespace mnb;

static uint64_t g_checked = 0;

// code k of row r in the contract layout
static unsigned contract_code(const Sizes& s, const mnb_desc& d, const uint8_t* B, int64_t r, int64_t k) {
  const uint8_t* row = B + (uint64_t)r * s.row_bytes;
  if (d.row_layout == MNB_ROWS_BLOCKED) {
    const int64_t b = k / s.bs, j = k % s.bs;
    const uint8_t byte = row[b * (s.bs / 2) + j / 2];
    return (j & 1) ? (byte >> 4) : (byte & 15u);
  }
  unsigned q = 0;
  for (int t = 0; t < s.bits; ++t) {
    const int64_t bit = k * s.bits + t;
    q |= ((row[bit >> 3] >> (bit & 7)) & 1u) << t;
  }
  return q;
}

static int run(const mnb_desc& d, uint32_t seed) {
  Sizes s;
  int rc = check_desc(&d, &s);
  if (rc != MNB_OK) { printf("check_desc rc %d\n", rc); return 1; }
  std::mt19937 rng(seed);
  std::vector<uint8_t> B(s.codes);
  for (auto& x : B) x = (uint8_t)rng();
  // canonical padding of row-local rows
  if (d.row_layout == MNB_ROWS_ROW_LOCAL) {
    const int64_t used = (s.K * s.bits) % 8;
    if (used)
      for (int64_t r = 0; r < s.rows; ++r) B[(uint64_t)r * s.row_bytes + s.row_bytes - 1] &= (uint8_t)((1u << used) - 1);
  }
  std::vector<uint8_t> sc(s.scales);
  if (d.scale_dtype == MNB_DTYPE_F32) {
    for (size_t i = 0; i < sc.size() / 4; ++i) { float v = (float)(rng() % 1000) / 997.0f; std::memcpy(&sc[4 * i], &v, 4); }
  } else {
    for (size_t i = 0; i < sc.size() / 2; ++i) { uint16_t h = (uint16_t)(0x2000 + rng() % 0x3000); std::memcpy(&sc[2 * i], &h, 2); }
  }
  std::vector<uint8_t> zp;
  if (d.has_zero_points) {
    zp.assign((size_t)(s.kind == kMoe ? s.rows : s.N) * s.zrow, 0);
    if (s.kind == kMoe) {
      // every zero point 2^(bits-1), canonical padding
      for (int64_t r = 0; r < s.rows; ++r)
        for (int64_t b = 0; b < s.nb; ++b)
          for (int t = 0; t < s.bits; ++t) {
            const int64_t bit = b * s.bits + t;
            if (((1u << (s.bits - 1)) >> t) & 1u) zp[(uint64_t)r * s.zrow + (bit >> 3)] |= (uint8_t)(1u << (bit & 7));
          }
    } else {
      for (auto& x : zp) x = (uint8_t)rng();
      if (s.nb % 2)  // the unused high nibble of the last byte
        for (int64_t r = 0; r < s.N; ++r) zp[(uint64_t)r * s.zrow + s.zrow - 1] &= 15u;
    }
  }
  rc = validate_content(&d, s, B.data(), sc.data(), zp.empty() ? nullptr : zp.data());
  if (rc != MNB_OK) { printf("validate rc %d\n", rc); return 1; }
  std::vector<uint8_t> dst(s.total);  // exact size: any write past it is caught
  prepack(s, B.data(), sc.data(), zp.empty() ? nullptr : zp.data(), dst.data());
  mnb_plan p;
  fill_plan(&d, s, dst.data(), 0, &p);
  Sizes s2;
  if (check_plan(&p, &s2) != MNB_OK) { printf("check_plan failed\n"); return 1; }
  // round trip of a few rows of every expert (all rows for small shapes)
  const int64_t step = s.N <= 64 ? 1 : s.N / 17 + 1;
  std::vector<uint8_t> codes(s.K), zeros(s.nb), scl(s.nb * (d.scale_dtype == MNB_DTYPE_F32 ? 4 : 2));
  for (int64_t e = 0; e < s.E; ++e)
    for (int64_t n = 0; n < s.N; n += step) {
      unpack_host(s, &p, e, n, 1, codes.data(), zeros.data(), scl.data());
      const int64_t r = e * s.N + n;
      for (int64_t k = 0; k < s.K; ++k)
        if (codes[k] != contract_code(s, d, B.data(), r, k)) { printf("code mismatch e%ld n%ld k%ld\n", (long)e, (long)n, (long)k); return 1; }
      if (std::memcmp(scl.data(), sc.data() + (uint64_t)r * scl.size(), scl.size())) { printf("scale mismatch\n"); return 1; }
      if (d.has_zero_points && s.kind == kDenseInt4)
        for (int64_t b = 0; b < s.nb; ++b) {
          const uint8_t zb = zp[(uint64_t)n * s.zrow + b / 2];
          const unsigned want = (b & 1) ? (zb >> 4) : (zb & 15u);
          if (zeros[b] != want) { printf("zero mismatch\n"); return 1; }
        }
      ++g_checked;
    }
  return 0;
}

int main() {
  int fails = 0, cases = 0;
  // dense INT4 (blocked rows, fp32 scales), ragged K, zero points, threaded sizes
  const int64_t Ks[] = {1, 34, 100, 2050, 4096};
  const int64_t Ns[] = {1, 7, 129, 40000};
  const int bss[] = {32, 64, 128};
  for (int64_t K : Ks) for (int64_t N : Ns) for (int bs : bss) for (int zpf = 0; zpf < 2; ++zpf) {
    if (N == 40000 && K > 2050) continue;
    mnb_desc d{}; d.abi_version = MNB_ABI_VERSION; d.bits = 4; d.block_size = bs; d.K = K; d.N = N;
    d.scale_dtype = MNB_DTYPE_F32; d.has_zero_points = zpf; d.row_layout = MNB_ROWS_BLOCKED; d.num_experts = 1;
    ++cases; if (run(d, (uint32_t)(K * 131 + N * 7 + bs + zpf))) { ++fails; printf("dense K%ld N%ld bs%d zp%d failed\n", (long)K, (long)N, bs, zpf); }
  }
  // QMoE INT3 / INT4 (row-local rows, fp16 / bf16 scales), K block-aligned
  const int64_t mK[] = {32, 64, 96, 768, 2048};
  const int64_t mN[] = {32, 48, 96, 1536};
  const int64_t mE[] = {1, 3, 16};
  for (int bits = 3; bits <= 4; ++bits) for (int64_t K : mK) for (int64_t N : mN) for (int64_t E : mE)
    for (int bs : bss) for (int dt = 1; dt <= 2; ++dt) for (int zpf = 0; zpf < 2; ++zpf) {
      if (K % bs) continue;
      if (E == 16 && N == 1536 && K == 2048 && bs != 64) continue;
      mnb_desc d{}; d.abi_version = MNB_ABI_VERSION; d.bits = bits; d.block_size = bs; d.K = K; d.N = N;
      d.scale_dtype = dt; d.has_zero_points = zpf; d.row_layout = MNB_ROWS_ROW_LOCAL; d.num_experts = E;
      ++cases; if (run(d, (uint32_t)(bits * 1000003 + K * 131 + N * 7 + E * 3 + bs + dt + zpf))) {
        ++fails; printf("moe bits%d K%ld N%ld E%ld bs%d dt%d zp%d failed\n", bits, (long)K, (long)N, (long)E, bs, dt, zpf); }
    }
  printf("cases %d failures %d rows checked %llu\n", cases, fails, (unsigned long long)g_checked);
  return fails ? 1 : 0;
}
