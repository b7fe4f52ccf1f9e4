// qg_layout.h -- byte layout of the library's device images and workspaces,
// and the fixed partition of a row's blocks into partial sums.
//
// Internal to libqgemv; the host packer and the kernels both include it.
//
// Weight image of an n x k matrix (k % 32 == 0).  kb = k/32 blocks per row,
// padded to kbp = roundup(kb, 16) with zero blocks; rows padded to
// np = roundup(n, 16) with zero rows.  Rows are grouped in tiles of 16, and a
// tile stores its blocks one after another, each block holding the 16 rows:
//   Q8_0 codes: tile t, block b at (t*kbp + b)*512: the low halves (codes
//        0..15) of rows 0..15 at 16*i, then the high halves (codes 16..31) at
//        256 + 16*i.  16 lanes that own 16 rows read 256 contiguous bytes, and
//        one MFMA operand fragment (8 codes of each of 16 rows) is 512
//        contiguous bytes.
//   Q4_0 codes: tile t, block b at (t*kbp + b)*256: row i's 16 packed bytes at
//        16*i in the canonical nibble order (byte j: code j low, code j+16
//        high).
//   Scales (fp16) at the next 256-byte boundary: (t*kbp + b)*16 + i.
// For n % 16 == 0 and k % 512 == 0 the image holds exactly the canonical bytes
// per weight.
//   Q4_K (k % 256 == 0): the code plane of Q4_0, sub-block b of a row (32
//        weights, sub-block b % 8 of superblock b / 8) in one 16-byte cell with
//        the Q4_0 nibble order (byte l: code l low, code l + 16 high); in place
//        of the fp16 scales, the superblocks' 16-byte headers (fp16 d, fp16
//        dmin, the twelve bytes of 6-bit sub-scales and sub-mins, as in the
//        canonical block): tile t, superblock s, row i at byte
//        ((t*(kbp/8) + s)*16 + i)*16 of that plane -- the same 2 bytes per
//        32 weights, so the image also holds 144 bytes per 256 weights.
//
// Prepared activation rows (workspace of `rows` rows of length k), each plane
// on a 256-byte boundary, pad blocks zero, in one of two orders:
//   row order (1..2 rows, and the grouped path):
//     codes int8 [rows][kbp*32] in element order;
//     dx    fp32 [rows][kbp] block scales;
//     nsx   int32 [rows][kbp] = -8 * (sum of the block's codes), the start
//           value of a Q4_0 block dot (sum (c-8) q = sum c q - 8 sum q).
//   pair order (3..16 rows; the operand order of the K=64 int8 MFMA): blocks
//     in pairs p = (2p, 2p+1), rows in groups g of eight (G = ceil(rows/8)
//     groups; rows past `rows` are zero).  Chunk (p, g) is 1 KB of codes: 64
//     lanes x 16 bytes, lane l = 16*q + i (i < 16, q < 4) holding, when
//     (i < 8) == (q < 2), codes 16*(q%2) .. 16*(q%2)+15 of row 8g + i%8 of
//     block 2p + i/8, and zeros otherwise; then dx and nsx [p][g][16] for
//     (row 8g + i%8, block 2p + i/8) at index i.
// Partition of a row's kbp blocks (depends on kbp only, never on the number of
// activation rows, so a row's fp32 result is the same in every launch): P parts
// (a power of two up to 32, about 8 blocks each) of BS = kbp/P blocks, grouped
// as S (<= 4) "wave parts" of H (<= 8) "lane parts".  Wave part s covers blocks
// [s*H*BS, (s+1)*H*BS); inside it lane part h takes the blocks s*H*BS + H*u + h,
// u = 0..BS-1, accumulated in that order.  Lane parts are summed by a fixed
// pairwise tree (((h0 + h1) + (h2 + h3)) + ...), wave parts left to right.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define QG_HD __host__ __device__ inline

namespace qg {

constexpr int QK = 32;     // weights per block
constexpr int GROUP = 16;  // block padding unit
constexpr int TILE = 16;   // rows per tile
constexpr int Q8_CANON = 34;
constexpr int Q4_CANON = 18;
constexpr int QK_K = 256;       // weights per K-quant superblock
constexpr int Q4K_CANON = 144;  // canonical Q4_K superblock bytes
constexpr int FMT_ID_Q4K = 5;   // QG_FMT_Q4_K

QG_HD int64_t kb_of(int64_t k) { return k / QK; }
QG_HD int64_t kbp_of(int64_t k) { return ((k / QK + GROUP - 1) / GROUP) * GROUP; }
QG_HD int64_t np_of(int64_t n) { return ((n + TILE - 1) / TILE) * TILE; }
QG_HD size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Bytes of one (tile, block) cell of the code plane.
QG_HD size_t cell_bytes(int fmt) { return fmt == 1 ? 512 : 256; }

QG_HD size_t image_code_bytes(int fmt, int64_t n, int64_t k) {
  return (size_t)(np_of(n) / TILE) * (size_t)kbp_of(k) * cell_bytes(fmt);
}
QG_HD size_t image_scale_offset(int fmt, int64_t n, int64_t k) { return align256(image_code_bytes(fmt, n, k)); }
QG_HD size_t image_total_bytes(int fmt, int64_t n, int64_t k) {
  return image_scale_offset(fmt, n, k) + align256((size_t)np_of(n) * (size_t)kbp_of(k) * 2);
}

// F16 image: 16-row tiles of 32-column steps, 1 KB per (tile, step).
QG_HD int64_t f16_steps(int64_t k) { return (k + 31) / 32; }
QG_HD int64_t f16_tiles(int64_t n) { return (n + 15) / 16; }
QG_HD int64_t f16_image_bytes(int64_t n, int64_t k) { return f16_tiles(n) * f16_steps(k) * 1024; }

// FP8 image: 16-row tiles of 128-column groups, 2 KB per (tile, group), then
// (256-byte aligned) the fp32 scales of 128 x 128 blocks [ceil(n/128)][k/128].
// FP8 workspace: codes [rows][k], then (aligned) fp32 scales [rows][k/128].
QG_HD size_t fp8_scale_offset(int64_t n, int64_t k) { return align256((size_t)f16_tiles(n) * (size_t)(k / 128) * 2048); }
QG_HD size_t fp8_image_bytes(int64_t n, int64_t k) {
  return fp8_scale_offset(n, k) + align256((size_t)((n + 127) / 128) * (size_t)(k / 128) * 4);
}
QG_HD size_t fp8_ws_scale_offset(int64_t rows, int64_t k) { return align256((size_t)rows * (size_t)k); }
QG_HD size_t fp8_ws_bytes(int64_t rows, int64_t k) {
  return fp8_ws_scale_offset(rows, k) + align256((size_t)rows * (size_t)(k / 128) * 4);
}

// Byte offset of row o's part of block b (Q8_0: its low half; the high half
// is 256 bytes further).
QG_HD size_t cell_row_offset(int fmt, int64_t o, int64_t b, int64_t kbp) {
  return ((size_t)(o / TILE) * (size_t)kbp + (size_t)b) * cell_bytes(fmt) + (size_t)(o % TILE) * 16;
}
// Index (in fp16 units) of row o's scale of block b.
QG_HD size_t scale_index(int64_t o, int64_t b, int64_t kbp) {
  return ((size_t)(o / TILE) * (size_t)kbp + (size_t)b) * TILE + (size_t)(o % TILE);
}
// Q4_K: byte offset, inside the scale plane, of row o's header of superblock s.
QG_HD size_t q4k_header_offset(int64_t o, int64_t s, int64_t kbp) {
  return (((size_t)(o / TILE) * (size_t)(kbp / 8) + (size_t)s) * TILE + (size_t)(o % TILE)) * 16;
}

struct PrepLayout {
  size_t codes, dx, nsx, total;
  bool pairs;  // pair order
  int groups;  // row groups of eight (pair order)
};
QG_HD bool prep_pairs(int64_t rows) { return rows >= 3 && rows <= 16; }
QG_HD PrepLayout prep_layout_rows(int64_t rows, int64_t k) {
  PrepLayout L;
  const int64_t kbp = kbp_of(k);
  L.codes = 0;
  L.dx = align256((size_t)rows * (size_t)kbp * 32);
  L.nsx = L.dx + align256((size_t)rows * (size_t)kbp * 4);
  L.total = L.nsx + align256((size_t)rows * (size_t)kbp * 4);
  L.pairs = false;
  L.groups = 0;
  return L;
}
QG_HD PrepLayout prep_layout_pairs(int64_t rows, int64_t k) {
  PrepLayout L;
  const size_t chunks = (size_t)(kbp_of(k) / 2) * (size_t)((rows + 7) / 8);
  L.codes = 0;
  L.dx = align256(chunks * 1024);
  L.nsx = L.dx + align256(chunks * 64);
  L.total = L.nsx + align256(chunks * 64);
  L.pairs = true;
  L.groups = (int)((rows + 7) / 8);
  return L;
}
// The order a GEMV of `rows` rows reads.
QG_HD PrepLayout prep_layout(int64_t rows, int64_t k) {
  return prep_pairs(rows) ? prep_layout_pairs(rows, k) : prep_layout_rows(rows, k);
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
  G.total = G.prep + prep_layout_rows(x_rows, k).total;
  return G;
}

// Workspace of the FP8 lane's grouped call: the same plan, then the FP8
// activation groups of the x_rows rows (fp8_ws_bytes).
QG_HD GroupedLayout grouped_fp8_layout(int64_t x_rows, int64_t k, int64_t m) {
  GroupedLayout G = grouped_layout(x_rows, k, m);
  G.total = G.prep + fp8_ws_bytes(x_rows, k);
  return G;
}

// Workspace of a fused routed-MoE step (qg_moe_step): rows <= 16 input rows,
// m = rows * slots assignments, slots = topk (+1 with a shared expert).
constexpr int QG_MOE_MAX_M = 16 * 33;
struct MoeLayout {
  size_t header, expert, weight, x_index, sorted, items, ditems, logits, xprep, gu, hprep, o, total;
};
// fp8: the input rows and h in FP8 groups (fp8_ws_bytes) instead of q8 rows.
QG_HD MoeLayout moe_layout(int64_t rows, int64_t n_experts, int64_t hidden, int64_t ffn, int64_t slots,
                           bool fp8 = false) {
  const int64_t m = rows * slots;
  MoeLayout M;
  M.header = 0;
  M.expert = 256;
  M.weight = M.expert + align256((size_t)m * 4);
  M.x_index = M.weight + align256((size_t)m * 4);
  M.sorted = M.x_index + align256((size_t)m * 4);
  M.items = M.sorted + align256((size_t)m * 4);
  M.ditems = M.items + align256((size_t)m * 12);
  M.logits = M.ditems + align256((size_t)m * 12);
  M.xprep = M.logits + align256((size_t)rows * n_experts * 4);
  M.gu = M.xprep + (fp8 ? fp8_ws_bytes(rows, hidden) : prep_layout_rows(rows, hidden).total);
  M.hprep = M.gu + align256((size_t)m * 2 * ffn * 4);
  M.o = M.hprep + (fp8 ? fp8_ws_bytes(m, ffn) : prep_layout_rows(m, ffn).total);
  M.total = M.o + align256((size_t)m * hidden * 4);
  return M;
}

struct PartPlan {
  int P, H, S, BS;
  int lgP, lgH, lgS;  // log2 of the powers of two P, H, S
};
QG_HD int ilog2(int v) {
  int l = 0;
  while ((1 << (l + 1)) <= v) l++;
  return l;
}
QG_HD PartPlan part_plan(int kbp) {
  const int m = kbp / 8;  // parts of about eight blocks
  int P = 1;
  while (P * 2 <= m && P < 32 && kbp % (P * 2) == 0) P *= 2;
  PartPlan pl;
  pl.P = P;
  pl.S = P < 4 ? P : 4;
  pl.H = P / pl.S;
  pl.BS = kbp / P;
  pl.lgP = ilog2(pl.P);
  pl.lgH = ilog2(pl.H);
  pl.lgS = ilog2(pl.S);
  return pl;
}

}  // namespace qg
