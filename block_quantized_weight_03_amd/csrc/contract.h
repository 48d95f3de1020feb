// Host-side contract of the mnb library: descriptor checks, overflow-checked
// sizes, content validation and the private prepacked layout.  Plain C++17,
// no HIP dependency, so all of it runs (and is tested) without a GPU.
#pragma once

#include <cstdint>

#include "../../include/mnb.h"

namespace mnb {

constexpr uint32_t kPlanMagic = 0x4D4E4250u;  // "MNBP"
// Version of the private prepacked layout (bumped whenever it changes):
//  dense INT4: codes [N][nb][bs/2] with every nibble stored as (q - 8) in
//              4-bit two's complement (byte XOR 0x88) and pad nibbles zero;
//              scales fp32 [N][nb]; zero points (if explicit) as uint32 words
//              [ceil(N/8)][nb], nibble r of word (g, b) holding the zero point
//              of row 8g + r, block b (one load gives a row group's points).
//  QMoE (INT3 or INT4 projections): codes: the same bytes per row as the
//              contract, bits*K/8, regrouped for the matrix-core
//              dequantization.  Each group of 32 codes c0..c31 (k = 32G + i)
//              of a row is GB = 4*bits bytes:
//              INT3: three 32-bit words w0, w1, w2; word m holds the pairs
//              (c[10m+2p], c[10m+2p+1]) for p = 0..4 at bits [3p, 3p+3) and
//              [16+3p, 16+3p+3), so (w >> 3p) & 0x00070007 puts a pair in the
//              two 16-bit halves; bit t of c30 is bit 15 of w_t and bit t of
//              c31 is bit 31 of w_t.
//              INT4: four 32-bit words; word m holds the pairs (c[8m+2p],
//              c[8m+2p+1]) for p = 0..3 at bits [4p, 4p+4) and [16+4p,
//              16+4p+4), so (w >> 4p) & 0x000F000F puts a pair in the halves.
//              The groups are stored tile-major: the rows of an expert in
//              tiles of 16 (the last may hold fewer), each tile as a sequence
//              of K chunks of 4 groups (128 codes; the last may hold fewer),
//              each chunk as its rows' groups row by row; so one chunk of one
//              tile is 16 x 4 GB contiguous bytes.  Scales fp16 [E*N][K/bs].
constexpr uint32_t kLayoutVersion = 5;
constexpr uint64_t kSectionAlign = 256;

enum Kind : int32_t { kDenseInt4 = 1, kMoe = 2 };

// Word (within its group of three) and bit offset of INT3 code i (0..31) of a
// group, for the codes stored in one 3-bit field (i < 30).
constexpr int int3_word(int i) { return i / 10; }
constexpr int int3_bit(int i) { return 3 * ((i % 10) / 2) + 16 * (i % 2); }

// Word (within its group of four) and bit offset of INT4 code i (0..31) of a
// group.
constexpr int int4_word(int i) { return i / 8; }
constexpr int int4_bit(int i) { return 4 * ((i % 8) / 2) + 16 * (i % 2); }

// Byte offset, inside the code section, of 32-code group G of row n_local of
// expert e (tile-major QMoE layout with GB-byte groups; K is a multiple of 32).
inline uint64_t moe_group_offset(int64_t N, int64_t K, int64_t GB, int64_t e, int64_t n_local,
                                 int64_t G) {
  const int64_t ng = K / 32, rt = n_local / 16, r = n_local % 16;
  const int64_t rcnt = (N - 16 * rt) < 16 ? (N - 16 * rt) : 16;
  const int64_t c = G / 4, g = G % 4;
  const int64_t gic = (ng - 4 * c) < 4 ? (ng - 4 * c) : 4;
  return (uint64_t)(e * N + 16 * rt) * (uint64_t)(ng * GB) +
         (uint64_t)(rcnt * 4 * GB * c + r * gic * GB + g * GB);
}

struct Sizes {
  Kind kind;
  int64_t E, N, K, nb, bs, bits;
  int64_t rows;         // E * N
  int64_t row_bytes;    // contract bytes per B row
  uint64_t codes;       // contract (= prepacked) code bytes
  uint64_t scales;      // scale bytes
  uint64_t zeros;       // prepacked zero-point bytes (0 if implicit)
  uint64_t zrow;        // contract zero-point bytes per row (ceil(nb/2))
  uint64_t off_scales;  // offsets of the sections in the prepacked buffer
  uint64_t off_zeros;
  uint64_t total;       // prepacked bytes
};

// Checks a descriptor and fills every size with overflow-checked arithmetic.
int32_t check_desc(const mnb_desc* d, Sizes* s);

// Validates the host content of the weights (QMoE projections: finite
// nonnegative fp16 scales and canonical row padding).  Dense INT4 content is
// not checked.
int32_t validate_content(const mnb_desc* d, const Sizes& s, const uint8_t* B,
                         const void* scales, const uint8_t* zp);

// Writes the private layout (s.total bytes) into dst.
void prepack(const Sizes& s, const uint8_t* B, const void* scales,
             const uint8_t* zp, uint8_t* dst);

// Fills a plan whose sections start at base (host or device address).
void fill_plan(const mnb_desc* d, const Sizes& s, void* base, int32_t device,
               mnb_plan* plan);

// Checks that a plan was produced by this library and rebuilds its sizes.
int32_t check_plan(const mnb_plan* p, Sizes* s);

// Reads logical codes / zero points / scales back from a host-resident
// prepacked layout.
void unpack_host(const Sizes& s, const mnb_plan* p, int64_t expert,
                 int64_t row0, int64_t nrows, uint8_t* codes, uint8_t* zeros,
                 void* scales);

}  // namespace mnb
