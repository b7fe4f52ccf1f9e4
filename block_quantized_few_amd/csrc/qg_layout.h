// qg_layout.h -- byte layout of the library's device images and workspaces.
//
// Internal to libqgemv; both the host packing code and the kernels include it.
//
// Weight image of an n x k matrix (k % 32 == 0), kb = k/32 blocks per row,
// padded to kbp = roundup(kb, 16) blocks with zero blocks:
//   Q8_0 code plane: n * kbp * 32 bytes.  Row o starts at o*kbp*32; its blocks
//        come in groups of 16 (512 bytes): the first 256 bytes hold the low
//        halves (codes 0..15) of the group's 16 blocks, 16 bytes each, the next
//        256 bytes the high halves (codes 16..31).  A 16-lane row group then
//        reads a whole group with two fully coalesced 256-byte loads, each lane
//        holding one complete block.
//   Q4_0 code plane: n * kbp * 16 bytes, block b of row o at (o*kbp + b)*16,
//        the canonical nibble order kept (byte j: code j low, code j+16 high),
//        so low nibbles give codes 0..15 and high nibbles codes 16..31.
//   Scale plane: fp16 [n][kbp] at the next 256-byte boundary after the codes.
//
// Prepared activation rows (workspace of `rows` rows of length k):
//   codes  int8  [rows][kbp*32] in the same low/high half grouping as Q8_0;
//   dx     fp32  [rows][kbp] block scales;
//   nsx    int32 [rows][kbp] = -8 * (sum of the block's codes), the start value
//          of a Q4_0 block dot (sum (c-8) q = sum c q - 8 sum q).
//   Each plane starts on a 256-byte boundary; pad blocks are all zero.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define QG_HD __host__ __device__ inline

namespace qg {

constexpr int QK = 32;           // weights per block
constexpr int GROUP = 16;        // blocks per interleave group
constexpr int Q8_CANON = 34;     // canonical block bytes
constexpr int Q4_CANON = 18;

QG_HD int64_t kb_of(int64_t k) { return k / QK; }
QG_HD int64_t kbp_of(int64_t k) { return ((k / QK + GROUP - 1) / GROUP) * GROUP; }
QG_HD size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

QG_HD size_t code_bytes_per_block(int fmt) { return fmt == 1 ? 32 : 16; }

QG_HD size_t image_code_bytes(int fmt, int64_t n, int64_t k) {
  return (size_t)n * (size_t)kbp_of(k) * code_bytes_per_block(fmt);
}
QG_HD size_t image_scale_offset(int fmt, int64_t n, int64_t k) { return align256(image_code_bytes(fmt, n, k)); }
QG_HD size_t image_total_bytes(int fmt, int64_t n, int64_t k) {
  return image_scale_offset(fmt, n, k) + align256((size_t)n * (size_t)kbp_of(k) * 2);
}

// Offset of the low half (Q8_0) of block b in row o; the high half is +256.
QG_HD size_t q8_lo_offset(int64_t o, int64_t b, int64_t kbp) {
  return (size_t)o * (size_t)kbp * 32 + (size_t)(b / GROUP) * 512 + (size_t)(b % GROUP) * 16;
}
QG_HD size_t q4_offset(int64_t o, int64_t b, int64_t kbp) { return ((size_t)o * (size_t)kbp + (size_t)b) * 16; }

// Workspace of prepared rows.
struct PrepLayout {
  size_t codes, dx, nsx, total;
};
QG_HD PrepLayout prep_layout(int64_t rows, int64_t k) {
  PrepLayout L;
  int64_t kbp = kbp_of(k);
  L.codes = 0;
  L.dx = align256((size_t)rows * (size_t)kbp * 32);
  L.nsx = L.dx + align256((size_t)rows * (size_t)kbp * 4);
  L.total = L.nsx + align256((size_t)rows * (size_t)kbp * 4);
  return L;
}

// Workspace of a grouped call: header, sorted assignment list, work items,
// then the prepared rows.
struct GroupedLayout {
  size_t header, sorted, items, prep, total;
};
QG_HD GroupedLayout grouped_layout(int64_t x_rows, int64_t k, int64_t m) {
  GroupedLayout G;
  G.header = 0;  // int32 [0] = work items, [1] = skipped assignments
  G.sorted = 256;
  G.items = G.sorted + align256((size_t)(m > 0 ? m : 1) * 4);
  G.prep = G.items + align256((size_t)(m > 0 ? m : 1) * 12);
  G.total = G.prep + prep_layout(x_rows, k).total;
  return G;
}

}  // namespace qg
