// Host contract of the mnb library (see contract.h).
//
// Sources: "Qwen3 Missing-Kernel Implementation Plan", section "PR sequence",
// step K01 (validate the FP32/UINT8/FP32 contract, packed layout, implicit
// zero points, scale indexing and padding; reject unsupported variants
// explicitly); onnxruntime PR "INT3 QMoE CUDA correctness baseline and Qwen
// experimental results", embedded P0/P1 body, sections "P0: Portable Format
// and Numerical References" (checked size arithmetic, canonical padding) and
// "P1: Compatible QMoE v1 Extension" (block sizes 32/64/128, block-aligned K
// but any N, exact buffer sizes, finite nonnegative FP16 scales).

#include "contract.h"

#include <cstring>
#include <thread>
#include <vector>

namespace mnb {
namespace {

bool mul_ok(uint64_t a, uint64_t b, uint64_t* r) { return !__builtin_mul_overflow(a, b, r); }
bool add_ok(uint64_t a, uint64_t b, uint64_t* r) { return !__builtin_add_overflow(a, b, r); }

bool align_up(uint64_t v, uint64_t* r) {
  uint64_t t;
  if (!add_ok(v, kSectionAlign - 1, &t)) return false;
  *r = t / kSectionAlign * kSectionAlign;
  return true;
}

uint16_t load_u16(const void* p, uint64_t i) {
  uint16_t v;
  std::memcpy(&v, static_cast<const uint8_t*>(p) + 2 * i, 2);
  return v;
}

}  // namespace

int32_t check_desc(const mnb_desc* d, Sizes* s) {
  if (!d || !s) return MNB_ERR_INVALID_ARG;
  if (d->abi_version != MNB_ABI_VERSION) return MNB_ERR_INVALID_ARG;
  if (d->K < 1 || d->N < 1 || d->num_experts < 1) return MNB_ERR_INVALID_ARG;
  if (d->accuracy_level < 0 || d->accuracy_level > 4) return MNB_ERR_INVALID_ARG;
  if (d->has_zero_points != 0 && d->has_zero_points != 1) return MNB_ERR_INVALID_ARG;
  if (d->scale_dtype != MNB_DTYPE_F32 && d->scale_dtype != MNB_DTYPE_F16 &&
      d->scale_dtype != MNB_DTYPE_BF16)
    return MNB_ERR_INVALID_ARG;
  if (d->row_layout != MNB_ROWS_BLOCKED && d->row_layout != MNB_ROWS_ROW_LOCAL) return MNB_ERR_INVALID_ARG;
  if (d->bits < 1 || d->bits > 8) return MNB_ERR_INVALID_ARG;
  if (d->block_size < 1) return MNB_ERR_INVALID_ARG;
  if (d->block_size != 32 && d->block_size != 64 && d->block_size != 128) return MNB_ERR_UNSUPPORTED;

  Sizes z{};
  z.E = d->num_experts;
  z.N = d->N;
  z.K = d->K;
  z.bs = d->block_size;
  z.bits = d->bits;
  z.nb = d->K / d->block_size + (d->K % d->block_size ? 1 : 0);

  if (d->bits == 4 && d->scale_dtype == MNB_DTYPE_F32) {
    // dense MatMulNBits profile
    if (d->row_layout != MNB_ROWS_BLOCKED || d->num_experts != 1) return MNB_ERR_UNSUPPORTED;
    z.kind = kDenseInt4;
  } else if (d->bits == 3 || d->bits == 4) {
    // QMoE v1 projection profile: INT3, or INT4 for the mixed (3,4) / (4,3)
    // width pairs and the all-INT4 layer; explicit zero points are accepted
    // only as the implicit value (checked with the content)
    if ((d->scale_dtype != MNB_DTYPE_F16 && d->scale_dtype != MNB_DTYPE_BF16) ||
        d->row_layout != MNB_ROWS_ROW_LOCAL)
      return MNB_ERR_UNSUPPORTED;
    if (d->K % d->block_size) return MNB_ERR_UNSUPPORTED;  // block-aligned K
    z.kind = kMoe;
  } else {
    return MNB_ERR_UNSUPPORTED;
  }

  uint64_t rows, t;
  if (!mul_ok((uint64_t)z.E, (uint64_t)z.N, &rows) || rows > (uint64_t)INT64_MAX)
    return MNB_ERR_SIZE_OVERFLOW;
  z.rows = (int64_t)rows;
  if (d->row_layout == MNB_ROWS_BLOCKED) {
    // nb * bs * bits / 8, bs * bits divisible by 8 for bs in {32, 64, 128}
    if (!mul_ok((uint64_t)z.nb, (uint64_t)(z.bs * z.bits / 8), &t) || t > (uint64_t)INT64_MAX)
      return MNB_ERR_SIZE_OVERFLOW;
  } else {
    uint64_t bitsrow;
    if (!mul_ok((uint64_t)z.K, (uint64_t)z.bits, &bitsrow) || !add_ok(bitsrow, 7, &t))
      return MNB_ERR_SIZE_OVERFLOW;
    t /= 8;
  }
  z.row_bytes = (int64_t)t;
  if (!mul_ok(rows, (uint64_t)z.row_bytes, &z.codes)) return MNB_ERR_SIZE_OVERFLOW;
  uint64_t nscale;
  if (!mul_ok(rows, (uint64_t)z.nb, &nscale)) return MNB_ERR_SIZE_OVERFLOW;
  if (!mul_ok(nscale, d->scale_dtype == MNB_DTYPE_F32 ? 4 : 2, &z.scales)) return MNB_ERR_SIZE_OVERFLOW;
  if (d->has_zero_points && z.kind == kMoe) {
    // packed per-row block zero points, a row-local LSB-first stream of nb
    // codes per row [E*N, ceil(nb*bits/8)]; validated, then implied (no
    // prepacked section)
    uint64_t zb, zt;
    if (!mul_ok((uint64_t)z.nb, (uint64_t)z.bits, &zb) || !add_ok(zb, 7, &zb)) return MNB_ERR_SIZE_OVERFLOW;
    z.zrow = zb / 8;
    if (!mul_ok(rows, z.zrow, &zt)) return MNB_ERR_SIZE_OVERFLOW;
  } else if (d->has_zero_points) {
    z.zrow = (uint64_t)(z.nb / 2 + (z.nb % 2));
    uint64_t zt;
    if (!mul_ok((uint64_t)z.N, z.zrow, &zt)) return MNB_ERR_SIZE_OVERFLOW;  // contract bytes
    const uint64_t groups = (uint64_t)z.N / 8 + (z.N % 8 ? 1 : 0);
    if (!mul_ok(groups, (uint64_t)z.nb, &zt) || !mul_ok(zt, 4, &z.zeros)) return MNB_ERR_SIZE_OVERFLOW;
  }
  uint64_t a, b, c;
  if (!align_up(z.codes, &a)) return MNB_ERR_SIZE_OVERFLOW;
  z.off_scales = a;
  if (!add_ok(a, z.scales, &b) || !align_up(b, &b)) return MNB_ERR_SIZE_OVERFLOW;
  z.off_zeros = b;
  if (!add_ok(b, z.zeros, &c) || !align_up(c, &c)) return MNB_ERR_SIZE_OVERFLOW;
  z.total = c;
  *s = z;
  return MNB_OK;
}

int32_t validate_content(const mnb_desc* d, const Sizes& s, const uint8_t* B,
                         const void* scales, const uint8_t* zp) {
  if (s.kind != kMoe) return MNB_OK;
  // explicit zero points must all be the implicit 2^(bits-1) ([P1]: all-4
  // explicit zero points for INT3), with canonical padding
  if (d->has_zero_points) {
    if (!zp) return MNB_ERR_INVALID_ARG;
    const unsigned want = 1u << (s.bits - 1);
    const int64_t zbits = s.nb * s.bits, zused = zbits % 8;
    for (int64_t r = 0; r < s.rows; ++r) {
      const uint8_t* zr = zp + (uint64_t)r * s.zrow;
      for (int64_t b = 0; b < s.nb; ++b) {
        unsigned z = 0;
        for (int64_t t = 0; t < s.bits; ++t) {
          const int64_t bit = b * s.bits + t;
          z |= (unsigned)((zr[bit >> 3] >> (bit & 7)) & 1u) << t;
        }
        if (z != want) return MNB_ERR_CONTENT;
      }
      if (zused && (zr[s.zrow - 1] >> zused)) return MNB_ERR_CONTENT;
    }
  }
  // finite, nonnegative FP16 / BF16 scales: an all-ones exponent is Inf/NaN
  // (fp16 0x7C00, bf16 0x7F80); a set sign bit is only allowed on zero
  const uint16_t expo = d->scale_dtype == MNB_DTYPE_BF16 ? 0x7F80u : 0x7C00u;
  const uint64_t n = s.scales / 2;
  for (uint64_t i = 0; i < n; ++i) {
    const uint16_t h = load_u16(scales, i);
    if ((h & expo) == expo) return MNB_ERR_CONTENT;
    if ((h & 0x8000u) && (h & 0x7FFFu)) return MNB_ERR_CONTENT;
  }
  // canonical padding: bits after K*bits in the last byte of a row are zero
  const int64_t used = (s.K * s.bits) % 8;
  if (used) {
    for (int64_t r = 0; r < s.rows; ++r) {
      const uint8_t last = B[(uint64_t)r * (uint64_t)s.row_bytes + (uint64_t)s.row_bytes - 1];
      if (last >> used) return MNB_ERR_CONTENT;
    }
  }
  return MNB_OK;
}

namespace {

// Runs f(lo, hi) over [0, items) on up to 16 host threads when the work is
// large enough to pay for them (bytes: the data the items cover).
template <typename F>
void parallel_items(int64_t items, uint64_t bytes, F&& f) {
  unsigned nt = std::thread::hardware_concurrency();
  nt = nt < 1 ? 1 : (nt > 16 ? 16 : nt);
  if (bytes < (uint64_t(8) << 20) || items < 2 * (int64_t)nt) nt = 1;
  if (nt == 1) {
    f(int64_t(0), items);
    return;
  }
  std::vector<std::thread> pool;
  pool.reserve(nt);
  for (unsigned t = 0; t < nt; ++t) {
    const int64_t lo = items * t / nt, hi = items * (t + 1) / nt;
    try {
      pool.emplace_back([&f, lo, hi] { f(lo, hi); });
    } catch (...) {
      f(lo, hi);  // no thread available: this range runs here
    }
  }
  for (auto& th : pool) th.join();
}

// The 32 three-bit codes of contract bytes src[0..12) (row-local, LSB-first:
// code i at bits [3i, 3i + 3)) as the three pair-interleaved words of the
// private layout: word m takes codes 10m .. 10m + 9, the even ones in its low
// half and the odd ones in its high half (3 bits each); bit t of codes 30 and
// 31 goes to bits 15 and 31 of word t.
inline void int3_group_words(const uint8_t* src, uint32_t w[3]) {
  uint64_t lo = 0;
  uint32_t hi = 0;
  std::memcpy(&lo, src, 8);
  std::memcpy(&hi, src + 8, 4);
  const unsigned __int128 v = (unsigned __int128)lo | ((unsigned __int128)hi << 64);
  for (int m = 0; m < 3; ++m) {
    const uint32_t x = (uint32_t)(v >> (30 * m)) & 0x3FFFFFFFu;
    uint32_t ev = 0, od = 0;
    for (int p = 0; p < 5; ++p) {
      ev |= ((x >> (6 * p)) & 7u) << (3 * p);
      od |= ((x >> (6 * p + 3)) & 7u) << (3 * p);
    }
    w[m] = ev | (od << 16);
  }
  const uint32_t c30 = (uint32_t)(v >> 90) & 7u, c31 = (uint32_t)(v >> 93) & 7u;
  for (int t = 0; t < 3; ++t) w[t] |= (((c30 >> t) & 1u) << 15) | (((c31 >> t) & 1u) << 31);
}

// The 32 four-bit codes of contract bytes src[0..16) (code i in byte i / 2,
// low nibble for even i) as four words: word m takes codes 8m .. 8m + 7, the
// even ones in its low half and the odd ones in its high half.
inline void int4_group_words(const uint8_t* src, uint32_t w[4]) {
  for (int m = 0; m < 4; ++m) {
    uint32_t x;
    std::memcpy(&x, src + 4 * m, 4);
    const uint32_t ev = (x & 0xFu) | ((x >> 4) & 0xF0u) | ((x >> 8) & 0xF00u) | ((x >> 12) & 0xF000u);
    const uint32_t od = ((x >> 4) & 0xFu) | ((x >> 8) & 0xF0u) | ((x >> 12) & 0xF00u) |
                        ((x >> 16) & 0xF000u);
    w[m] = ev | (od << 16);
  }
}

// Writes the tile-major groups of rows [16 rt, 16 rt + rcnt) of expert e: the
// tile's chunks of 4 groups in K order, each chunk row by row, which is the
// order of moe_group_offset, so the tile's bytes are written front to back.
void pack_moe_tile(const Sizes& s, const uint8_t* B, uint8_t* codes, int64_t e, int64_t rt) {
  const int64_t GB = 4 * s.bits, ng = s.K / 32;
  const int64_t rcnt = (s.N - 16 * rt) < 16 ? (s.N - 16 * rt) : 16;
  const int64_t row0 = e * s.N + 16 * rt;
  uint8_t* out = codes + moe_group_offset(s.N, s.K, GB, e, 16 * rt, 0);
  for (int64_t c = 0; c < ng; c += 4) {
    const int64_t gic = (ng - c) < 4 ? (ng - c) : 4;
    for (int64_t r = 0; r < rcnt; ++r) {
      const uint8_t* src = B + (uint64_t)(row0 + r) * (uint64_t)s.row_bytes + (uint64_t)(c * GB);
      for (int64_t g = 0; g < gic; ++g, out += GB, src += GB) {
        uint32_t w[4];
        if (s.bits == 4)
          int4_group_words(src, w);
        else
          int3_group_words(src, w);
        std::memcpy(out, w, (size_t)GB);
      }
    }
  }
}

}  // namespace

void prepack(const Sizes& s, const uint8_t* B, const void* scales,
             const uint8_t* zp, uint8_t* dst) {
  // every byte of the sections is written below; only the alignment gaps
  // between and after them are cleared here
  std::memset(dst + s.codes, 0, s.off_scales - s.codes);
  std::memset(dst + s.off_scales + s.scales, 0, s.off_zeros - s.off_scales - s.scales);
  std::memset(dst + s.off_zeros + s.zeros, 0, s.total - s.off_zeros - s.zeros);
  uint8_t* codes = dst;
  if (s.kind == kDenseInt4) {
    // Store each code as (q - 8) in 4-bit two's complement: nibble XOR 8.
    // Pad positions k >= K of the last block are written as 0.
    const int64_t half = s.bs / 2;
    const int64_t valid_last = s.K - (s.nb - 1) * s.bs;
    parallel_items(s.N, s.codes, [&](int64_t lo, int64_t hi) {
      for (int64_t n = lo; n < hi; ++n) {
        const uint8_t* src = B + (uint64_t)n * (uint64_t)s.row_bytes;
        uint8_t* out = codes + (uint64_t)n * (uint64_t)s.row_bytes;
        for (int64_t i = 0; i < s.row_bytes; ++i) out[i] = (uint8_t)(src[i] ^ 0x88u);
        if (valid_last < s.bs) {
          uint8_t* last = out + (s.nb - 1) * half;
          for (int64_t j = valid_last; j < s.bs; ++j) {
            if (j & 1)
              last[j >> 1] &= 0x0Fu;
            else
              last[j >> 1] &= 0xF0u;
          }
        }
      }
    });
  } else {
    // contract rows are LSB-first bit streams; regroup every 32 codes into
    // the pair-interleaved words, stored tile-major (same byte count).  Each
    // (expert, 16-row tile) writes one contiguous piece of the code section,
    // so the tiles are spread over host threads.
    const int64_t tiles = (s.N + 15) / 16, items = s.E * tiles;
    parallel_items(items, (uint64_t)s.codes, [&](int64_t lo, int64_t hi) {
      for (int64_t it = lo; it < hi; ++it) pack_moe_tile(s, B, codes, it / tiles, it % tiles);
    });
  }
  parallel_items(64, s.scales, [&](int64_t lo, int64_t hi) {
    const uint64_t a = s.scales * (uint64_t)lo / 64, b = s.scales * (uint64_t)hi / 64;
    std::memcpy(dst + s.off_scales + a, static_cast<const uint8_t*>(scales) + a, b - a);
  });
  if (s.zeros) {
    // word (g, b): nibble r = zero point of row 8g + r, block b; rows past N
    // hold 8 (never read)
    const int64_t groups = s.N / 8 + (s.N % 8 ? 1 : 0);
    // (8 strided byte reads and a word write per (group, block): weighed as
    // 64 bytes of streaming work each when choosing the thread count)
    parallel_items(groups, s.zeros * 16, [&](int64_t lo, int64_t hi) {
      for (int64_t g = lo; g < hi; ++g) {
        for (int64_t b = 0; b < s.nb; ++b) {
          uint32_t w = 0;
          for (int r = 0; r < 8; ++r) {
            const uint64_t n = 8 * (uint64_t)g + (uint64_t)r;
            uint32_t z = 8;
            if (n < (uint64_t)s.N) {
              const uint8_t byte = zp[n * s.zrow + (uint64_t)(b / 2)];
              z = (b & 1) ? (byte >> 4) : (byte & 15u);
            }
            w |= z << (4 * r);
          }
          std::memcpy(dst + s.off_zeros + ((uint64_t)g * (uint64_t)s.nb + (uint64_t)b) * 4, &w, 4);
        }
      }
    });
  }
}

void fill_plan(const mnb_desc* d, const Sizes& s, void* base, int32_t device,
               mnb_plan* p) {
  std::memset(p, 0, sizeof(*p));
  p->desc = *d;
  p->magic = kPlanMagic;
  p->layout_version = kLayoutVersion;
  p->n_blocks = s.nb;
  p->row_bytes = s.row_bytes;
  p->codes_bytes = s.codes;
  p->scales_bytes = s.scales;
  p->zeros_bytes = s.zeros;
  p->total_bytes = s.total;
  uint8_t* b = static_cast<uint8_t*>(base);
  p->codes = b;
  p->scales = b + s.off_scales;
  p->zeros = s.zeros ? b + s.off_zeros : nullptr;
  p->device = device;
}

int32_t check_plan(const mnb_plan* p, Sizes* s) {
  if (!p || !s) return MNB_ERR_INVALID_ARG;
  if (p->magic != kPlanMagic || p->layout_version != kLayoutVersion) return MNB_ERR_STALE_PLAN;
  const int32_t rc = check_desc(&p->desc, s);
  if (rc != MNB_OK) return MNB_ERR_STALE_PLAN;
  if (p->codes_bytes != s->codes || p->scales_bytes != s->scales || p->zeros_bytes != s->zeros ||
      p->total_bytes != s->total || p->n_blocks != s->nb || p->row_bytes != s->row_bytes)
    return MNB_ERR_STALE_PLAN;
  if (!p->codes || !p->scales || (s->zeros && !p->zeros)) return MNB_ERR_STALE_PLAN;
  return MNB_OK;
}

void unpack_host(const Sizes& s, const mnb_plan* p, int64_t expert,
                 int64_t row0, int64_t nrows, uint8_t* codes, uint8_t* zeros,
                 void* scales) {
  const uint8_t* base = static_cast<const uint8_t*>(p->codes);
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t row = expert * s.N + row0 + r;
    const uint8_t* src = base + (uint64_t)row * (uint64_t)s.row_bytes;
    if (codes) {
      for (int64_t k = 0; k < s.K; ++k) {
        unsigned q;
        if (s.kind == kDenseInt4) {
          const int64_t b = k / s.bs, j = k % s.bs;
          const uint8_t byte = src[b * (s.bs / 2) + j / 2];
          q = ((j & 1) ? (byte >> 4) : (byte & 15u)) ^ 8u;
        } else {
          uint32_t w[4];
          const int64_t GB = 4 * s.bits;
          std::memcpy(w, base + moe_group_offset(s.N, s.K, GB, row / s.N, row % s.N, k / 32),
                      (size_t)GB);
          const int i = (int)(k % 32);
          if (s.bits == 4) {
            q = (w[int4_word(i)] >> int4_bit(i)) & 15u;
          } else if (i < 30) {
            q = (w[int3_word(i)] >> int3_bit(i)) & 7u;
          } else {
            q = 0;
            for (int t = 0; t < 3; ++t) q |= ((w[t] >> (i == 30 ? 15 : 31)) & 1u) << t;
          }
        }
        codes[(uint64_t)r * (uint64_t)s.K + (uint64_t)k] = (uint8_t)q;
      }
    }
    if (zeros) {
      for (int64_t b = 0; b < s.nb; ++b) {
        unsigned z = 1u << (s.bits - 1);
        if (s.zeros) {
          uint32_t w;
          std::memcpy(&w, static_cast<const uint8_t*>(p->zeros) +
                              ((uint64_t)(row / 8) * (uint64_t)s.nb + (uint64_t)b) * 4, 4);
          z = (w >> (4 * (row % 8))) & 15u;
        }
        zeros[(uint64_t)r * (uint64_t)s.nb + (uint64_t)b] = (uint8_t)z;
      }
    }
    if (scales) {
      const uint64_t esz = s.kind == kDenseInt4 ? 4 : 2;
      std::memcpy(static_cast<uint8_t*>(scales) + (uint64_t)r * (uint64_t)s.nb * esz,
                  static_cast<const uint8_t*>(p->scales) + (uint64_t)row * (uint64_t)s.nb * esz,
                  (uint64_t)s.nb * esz);
    }
  }
}

}  // namespace mnb
