// qg_q8.hip -- the q8 lane: Q8_0 / Q4_0 weights against q8 activation rows,
// 1..16 rows per call, for one projection, a set of projections, or the
// routed experts of a MoE layer.
//
// Rows past eight never get a launch of their own: every launch takes all of
// its 1..16 rows in one pass over the weights (the tiling of the dasLLAMA
// pages -- router-GEMV commit of the audio-towers page, commit 16880fe of the
// llama-leg page -- done inside the kernel).
//
// Two kernels share one weight layout (16-row tiles, block-major; see
// qg_layout.h) and one partition of each row's blocks, so they produce the
// same bits for a row:
//   * RL ("lanes own rows", 1..2 rows and the grouped path): a lane owns one
//     weight row and streams its blocks with 16-byte loads; the integer dot of
//     each block is exact inside the lane (v_dot4_i32_i8); activation blocks
//     are read from LDS by the whole lane group at once (broadcast).  At 1..2
//     rows the launch quantizes its fp32 rows itself.
//   * MP ("pairs", 3..16 rows): one v_mfma_i32_16x16x64_i8 gives the exact
//     dots of two blocks of 16 weight rows against 8 activation rows (two for
//     16 rows); the lanes then scale and accumulate in fp32.
// Both accumulate, per row and activation row, acc = fma(isum, dw * dx, acc)
// over the blocks of each part in the partition's order, then add lane parts
// by a fixed tree and wave parts left to right.
#include <hip/hip_runtime.h>
#include <string.h>

#include "qg_device.h"
#include "qg_internal.h"
#include "qg_launch.h"
#include "qg_route.h"

namespace qg {

constexpr int WG = 512;
constexpr int WAVES = WG / WAVE;
constexpr int LDS_X_RL = 80 * 1024;   // staged rows, RL (leaves room for 2+ workgroups per CU)
constexpr int FUSE_MAX_ROWS = 2;      // rows quantized inside the GEMV launch

__host__ __device__ inline int x_block_bytes(int fmt) { return nibble_fmt(fmt) ? 40 : 36; }

// Block index of staged slot `slot` of a chunk that starts at in-part index u0.
// Slots are ordered (u, wave part, lane part), so lanes that step together read
// neighbouring slots.
__device__ __forceinline__ int slot_block(const PartPlan& pl, int u0, int slot) {
  const int u = u0 + (slot >> pl.lgP), part = slot & (pl.P - 1);
  return (part & ~(pl.H - 1)) * pl.BS + pl.H * u + (part & (pl.H - 1));
}

// Blocks per part per staging round of an RL tile whose R rows get lds_x bytes
// of LDS: all BS at once, or a multiple of four (a round then starts on the
// block that the lane's first register set holds).  lds_x always holds four
// rounds' worth for any plan (P <= 32, R <= 16: 4 * 16 * 32 * 40 bytes).
__host__ __device__ inline int rl_round(int lds_x, int R, const PartPlan& pl, int fmt) {
  const int uc_max = lds_x / (R * pl.P * x_block_bytes(fmt));
  return uc_max >= pl.BS ? pl.BS : (uc_max & ~3);
}

// Blocks a lane keeps in flight (memory parallelism comes from the many waves).
__host__ __device__ constexpr int rl_lookahead(bool, int) { return 2; }

// ------------------------------------------------------------- staging ---

// RL layout: codes [R][nslot][32], dx [R][nslot], nsx [R][nslot].
template <int FMT, int R>
__device__ void stage_rl(uint8_t* lds, const Prep& prep, const int* s_src, int kbp, const PartPlan& pl, int u0,
                         int nslot) {
  const int tid = threadIdx.x;
  uint4* lc = reinterpret_cast<uint4*>(lds);
  float* ld = reinterpret_cast<float*>(lds + (size_t)R * nslot * 32);
  int* ln = reinterpret_cast<int*>(lds + (size_t)R * nslot * 36);
#pragma unroll
  for (int r = 0; r < R; r++) {
    const size_t src = (size_t)s_src[r] * kbp;
    for (int e = tid; e < nslot * 2; e += WG) {
      const int b = slot_block(pl, u0, e >> 1);
      lc[r * nslot * 2 + e] = ld16(prep.codes + (src + b) * 32 + (e & 1) * 16);
    }
    for (int e = tid; e < nslot; e += WG) {
      const int b = slot_block(pl, u0, e);
      ld[r * nslot + e] = prep.dx[src + b];
      if (FMT != FMT_Q8) ln[r * nslot + e] = prep.nsx[src + b];
    }
  }
}

// RL layout, quantizing fp32 rows on the way (all of kbp staged): four lanes per
// block (work item e: quarter e & 3 of staged block e >> 2), the same
// arithmetic as the stand-alone quantizer.  The start values are written for
// Q4_0 only (the Q8_0 staging area has no room for them).
//
// Split in two so that a caller can issue its weight loads in between: the
// memory counter a wave waits on retires loads in issue order, so activation
// values loaded first can be quantized while the weight loads are in flight.
constexpr int XQ_FIRST = 1;  // work items per thread whose loads are issued first

// One work item's loaded values: eight consecutive columns of a row (a, c),
// and with GLU the matching up values (ua, uc) of an interleaved gate/up row.
template <bool GLU>
struct XQuarterT {
  float4 a, c;
};
template <>
struct XQuarterT<true> {
  float4 a, c, ua, uc;
};
using XQuarter = XQuarterT<false>;

// Work item e of R <= 2 rows: row r = e / (4 * nslot), without a division.
__device__ __forceinline__ int xq_row(int e, int nslot) { return e >= 4 * nslot ? 1 : 0; }

// Row r of the fused staging is row r of x (rows k apart), or with GLU row
// s_src[r] of gu (rows 2k apart: the gate values, then the up values), whose
// SwiGLU the store takes.
template <bool GLU = false>
__device__ __forceinline__ XQuarterT<GLU> xq_load(const float* __restrict__ x, int64_t k, int kb, int nslot,
                                                  const PartPlan& pl, int e, int total, const int* s_src = nullptr) {
  const int q = e & 3, blk = e >> 2;
  const int r = xq_row(e, nslot), slot = blk - r * nslot;
  const int b = slot_block(pl, 0, slot);
  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
  XQuarterT<GLU> v;
  v.a = z;
  v.c = z;
  if constexpr (GLU) {
    v.ua = z;
    v.uc = z;
  }
  if (e < total) {  // uniform over a wave: total is a multiple of 64
    // pad blocks read the row's first quarter and use zeros
    const bool ok = b < kb;
    const int64_t row = GLU ? (int64_t)s_src[r] * 2 * k : (int64_t)r * k;
    const float4* src = reinterpret_cast<const float4*>(x + row + (ok ? (int64_t)b * QK + q * 8 : 0));
    const float4 a = src[0], c = src[1];
    v.a = ok ? a : z;
    v.c = ok ? c : z;
    if constexpr (GLU) {
      const float4* up = src + k / 4;
      const float4 ua = up[0], uc = up[1];
      v.ua = ok ? ua : z;
      v.uc = ok ? uc : z;
    }
  }
  return v;
}

template <int FMT, bool GLU = false>
__device__ __forceinline__ void xq_store(const XQuarterT<GLU>& xv, uint8_t* lds, int R, int nslot, int e, int total) {
  if (e >= total) return;  // whole quads leave together: total and the stride are multiples of 4
  const int q = e & 3, blk = e >> 2;
  const int r = xq_row(e, nslot), slot = blk - r * nslot;
  float v[8] = {xv.a.x, xv.a.y, xv.a.z, xv.a.w, xv.c.x, xv.c.y, xv.c.z, xv.c.w};
  if constexpr (GLU) {
    // h = silu(g) * u, the arithmetic of the stand-alone SwiGLU quantization
    // (two values at a time: all eight at once held 44 more registers, a
    // workgroup per CU fewer in the grouped launch)
    const float u[8] = {xv.ua.x, xv.ua.y, xv.ua.z, xv.ua.w, xv.uc.x, xv.uc.y, xv.uc.z, xv.uc.w};
#pragma unroll 2
    for (int i = 0; i < 8; i++) v[i] = v[i] / (1.0f + expf(-v[i])) * u[i];
  }
  unsigned lo, hi;
  float d;
  int sum;
  quantize_quarter(v, lo, hi, d, sum);
  *reinterpret_cast<uint2*>(lds + ((size_t)r * nslot + slot) * 32 + q * 8) = make_uint2(lo, hi);
  if (q == 0) {
    reinterpret_cast<float*>(lds + (size_t)R * nslot * 32)[r * nslot + slot] = d;
    if (FMT != FMT_Q8) reinterpret_cast<int*>(lds + (size_t)R * nslot * 36)[r * nslot + slot] = -8 * sum;
  }
}

// First part: load this thread's first XQ_FIRST work items.
template <bool GLU = false>
__device__ __forceinline__ void stage_quantize_begin(XQuarterT<GLU> (&xv)[XQ_FIRST], const float* __restrict__ x,
                                                     int64_t k, int kb, int R, int kbp, const PartPlan& pl,
                                                     const int* s_src = nullptr) {
  const int total = R * kbp * 4;
#pragma unroll
  for (int j = 0; j < XQ_FIRST; j++) xv[j] = xq_load<GLU>(x, k, kb, kbp, pl, threadIdx.x + j * WG, total, s_src);
}

// Second part: quantize them into LDS, then the rest of the work items.
template <int FMT, bool GLU = false>
__device__ __forceinline__ void stage_quantize_end(const XQuarterT<GLU> (&xv)[XQ_FIRST], uint8_t* lds,
                                                   const float* __restrict__ x, int64_t k, int kb, int R, int kbp,
                                                   const PartPlan& pl, const int* s_src = nullptr) {
  const int total = R * kbp * 4;
#pragma unroll
  for (int j = 0; j < XQ_FIRST; j++) xq_store<FMT, GLU>(xv[j], lds, R, kbp, threadIdx.x + j * WG, total);
  for (int e = threadIdx.x + XQ_FIRST * WG; e < total; e += WG) {
    xq_store<FMT, GLU>(xq_load<GLU>(x, k, kb, kbp, pl, e, total, s_src), lds, R, kbp, e, total);
  }
}

// ------------------------------------------------------------- RL tile ---

struct TileArgs {
  const uint8_t* code;
  const uint16_t* scale;
  int64_t n;
  int kbp, kb;
  int64_t k;
  int64_t row0;     // first weight row of the tile
  Prep prep;        // prepared rows
  const float* xf;  // fp32 rows (fused quantization) or null
  const int* s_src; // prepared row of each activation row (LDS)
  float* y;
  int64_t ldy;
  const int* s_dst; // output row of each activation row (LDS)
  int lds_x;        // LDS bytes for staged rows
  PartPlan pl;      // partition of kbp
  int ucx;          // RL staging round (rl_round)
};

// One weight block of one row as a lane holds it.
template <int FMT>
struct WBlock {
  uint4 lo;
  uint4 hi;  // Q8_0 high half
  uint16_t sc;
  uint4 hdr;  // Q4_K: the 16-byte header of the block's superblock
};

// Block b of the lane's row.  The address is the tile's base (uniform) plus a
// 32-bit lane offset, so the loads take the scalar-base form.  Q4_K: soff
// points at the row's header of superblock 0 (fp16 units), superblocks 128
// units apart; the lane parts of a row that step through one superblock read
// the same 16 bytes.
template <int FMT>
__device__ __forceinline__ WBlock<FMT> load_block(const uint8_t* __restrict__ tcode, uint32_t woff,
                                                  const uint16_t* __restrict__ tscale, uint32_t soff, int b) {
  constexpr uint32_t CB = FMT == FMT_Q8 ? 512 : 256;
  WBlock<FMT> w;
  w.lo = ld16_stream(tcode + (woff + (uint32_t)b * CB));
  if (FMT == FMT_Q8) w.hi = ld16_stream(tcode + (woff + (uint32_t)b * CB + 256));
  if (FMT == FMT_Q4K) w.hdr = ld16_stream(tscale + (soff + (uint32_t)(b >> 3) * 128));
  else w.sc = ld2_stream(tscale + (soff + (uint32_t)b * TILE));
  return w;
}

// acc[r] = fma(isum, dw * dx, acc[r]) for one block, its activation blocks at
// staged slot `slot` (Q4_K: q4k_acc of sub-block `sub` of its superblock).
template <int FMT, int R>
__device__ __forceinline__ void compute_block(float (&acc)[R], const WBlock<FMT>& w, const uint8_t* lds, int nslot,
                                              int slot, int sub) {
  const float* ld = reinterpret_cast<const float*>(lds + (size_t)R * nslot * 32);
  const int* ln = reinterpret_cast<const int*>(lds + (size_t)R * nslot * 36);
  if constexpr (FMT == FMT_Q4K) {
    float D, M;
    q4k_dm(w.hdr, sub, D, M);
#pragma unroll
    for (int r = 0; r < R; r++) {
      const uint8_t* xb = lds + ((size_t)r * nslot + slot) * 32;
      const uint4 xl = ld16(xb), xh = ld16(xb + 16);
      const int isum = dot_q4(w.lo, xl, xh, 0);
      acc[r] = q4k_acc(acc[r], isum, -(ln[r * nslot + slot] / 8), D, M, ld[r * nslot + slot]);
    }
    return;
  }
  const float dw = h2f(w.sc);
#pragma unroll
  for (int r = 0; r < R; r++) {
    const uint8_t* xb = lds + ((size_t)r * nslot + slot) * 32;
    const uint4 xl = ld16(xb), xh = ld16(xb + 16);
    const float dxr = ld[r * nslot + slot];
    if constexpr (FMT == FMT_Q8) {
      acc[r] = __builtin_fmaf((float)dot_q8(w.lo, w.hi, xl, xh), dw * dxr, acc[r]);
    } else {
      // sixteen times the dot against dx / 16: the product and the sum are those of the dot against dx
      acc[r] = __builtin_fmaf((float)dot_q4s16(w.lo, xl, xh), dw * (dxr * 0.0625f), acc[r]);
    }
  }
}

// One RL tile: weight rows row0 .. row0 + WG/P - 1.  `stage`: the activation
// rows are not in LDS yet.  Returns whether LDS now holds all of them (so the
// next tile of the same rows may skip staging).
//
// A lane streams its part's blocks u = 0 .. BS-1 with LA blocks in flight:
// the load of block u+LA is issued as block u is used.  The first LA are
// issued before the activation rows are staged (and, when they are quantized
// here, after their fp32 loads, which the wave's in-order memory counter then
// returns first).
// GLU (with FUSED): the fp32 rows are the SwiGLU of interleaved gate/up rows
// ta.xf picked by ta.s_src (see xq_load).
template <int FMT, int R, bool FUSED, int LA = rl_lookahead(FUSED, R), bool GLU = false>
__device__ bool rl_tile(const TileArgs& ta, uint8_t* lds, float* red, int parity, bool stage) {
  static_assert(!FUSED || R <= FUSE_MAX_ROWS, "fused quantization stages at most two rows");
  const PartPlan& pl = ta.pl;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & (WAVE - 1);
  const int lg_rpw = 6 - pl.lgH, rpw = 1 << lg_rpw;  // rows per wave
  const int g = wave >> pl.lgS, s = wave & (pl.S - 1), h = lane >> lg_rpw, rl = lane & (rpw - 1);
  const int64_t row = ta.row0 + g * rpw + rl;
  const bool valid = row < ta.n;
  const int64_t rc = valid ? row : ta.n - 1;  // out-of-range lanes read a real row, store nothing
  // tile base (uniform) + lane offset (< 2^32: a tile spans WG/P rows of kbp blocks)
  const int64_t t0 = ta.row0 >> 4;
  const uint8_t* tcode = ta.code + cell_row_offset(FMT, t0 * TILE, 0, ta.kbp);
  const uint16_t* tscale = ta.scale + scale_index(t0 * TILE, 0, ta.kbp);
  const uint32_t woff = (uint32_t)((rc >> 4) - t0) * (uint32_t)ta.kbp * (FMT == FMT_Q8 ? 512u : 256u) +
                        (uint32_t)(rc & 15) * 16u;
  const uint32_t soff = (uint32_t)((rc >> 4) - t0) * (uint32_t)ta.kbp * 16u + (uint32_t)(rc & 15) * (FMT == FMT_Q4K ? 8u : 1u);

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; r++) acc[r] = 0.0f;
  const int ucx = ta.ucx;
  const bool full = ucx == pl.BS;          // every block staged at once
  const int bpart = s * pl.H * pl.BS + h;  // this lane's block at u = 0
  const int sbase = s * pl.H + h;          // its slot at u = 0 of a round

  XQuarterT<GLU> xv[XQ_FIRST];
  if (FUSED && stage) stage_quantize_begin<GLU>(xv, ta.xf, ta.k, ta.kb, R, ta.kbp, pl, ta.s_src);
  WBlock<FMT> w[LA];
#pragma unroll
  for (int j = 0; j < LA; j++) w[j] = load_block<FMT>(tcode, woff, tscale, soff, bpart + pl.H * j);  // BS >= 8
  __builtin_amdgcn_sched_barrier(0);
  int u0 = 0, nslot = ucx << pl.lgP;
  int next_round = (!full || stage) ? 0 : pl.BS;  // u at which activation rows are (re)staged
  auto restage = [&](int u) {
    if (u == next_round) {
      u0 = u;
      nslot = min(ucx, pl.BS - u) << pl.lgP;
      next_round = full ? pl.BS : u + ucx;
      __syncthreads();
      if (FUSED) stage_quantize_end<FMT, GLU>(xv, lds, ta.xf, ta.k, ta.kb, R, ta.kbp, pl, ta.s_src);
      else stage_rl<FMT, R>(lds, ta.prep, ta.s_src, ta.kbp, pl, u0, nslot);
      __syncthreads();
    }
  };
  int u = 0;
  // Rounds whose every block has a next block to load: no branch around the
  // loads, so the block registers need no copies at a join (a copy would
  // wait for the load just issued and leave one block in flight).  (Q4_K,
  // whose header decode holds more registers, spilled with the second loop
  // at two rows: it keeps the one loop below.)
  for (; FMT != FMT_Q4K && u + 2 * LA <= pl.BS; u += LA) {
    restage(u);
    const int slot = ((u - u0) << pl.lgP) + sbase;
#pragma unroll
    for (int j = 0; j < LA; j++) {
      compute_block<FMT, R>(acc, w[j], lds, nslot, slot + (j << pl.lgP), (bpart + pl.H * (u + j)) & 7);
      w[j] = load_block<FMT>(tcode, woff, tscale, soff, bpart + pl.H * (u + j + LA));
    }
  }
  // the last fewer than 2 LA blocks
  for (; u < pl.BS; u += LA) {
    restage(u);
    const int slot = ((u - u0) << pl.lgP) + sbase;
#pragma unroll
    for (int j = 0; j < LA; j++) {
      if (u + j < pl.BS) {
        compute_block<FMT, R>(acc, w[j], lds, nslot, slot + (j << pl.lgP), (bpart + pl.H * (u + j)) & 7);
        if (u + j + LA < pl.BS) w[j] = load_block<FMT>(tcode, woff, tscale, soff, bpart + pl.H * (u + j + LA));
      }
    }
  }
  // lane parts: ((h0 + h1) + (h2 + h3)) + ...; every lane of the row gets the same bits
  for (int off = rpw; off < WAVE; off <<= 1)
#pragma unroll
    for (int r = 0; r < R; r++) acc[r] += __shfl_xor(acc[r], off);
  if (pl.S == 1) {
    if (valid && h == 0)
#pragma unroll
      for (int r = 0; r < R; r++) ta.y[(int64_t)ta.s_dst[r] * ta.ldy + row] = acc[r];
  } else {
    float* rb = red + parity * (WAVES * WAVE * R);
    if (h == 0)
#pragma unroll
      for (int r = 0; r < R; r++) rb[(wave * WAVE + rl) * R + r] = acc[r];
    __syncthreads();
    if (s == 0 && h == 0) {
#pragma unroll
      for (int r = 0; r < R; r++) {
        float v = rb[((g * pl.S) * WAVE + rl) * R + r];
        for (int s2 = 1; s2 < pl.S; s2++) v += rb[((g * pl.S + s2) * WAVE + rl) * R + r];
        if (valid) ta.y[(int64_t)ta.s_dst[r] * ta.ldy + row] = v;
      }
    }
  }
  return full;
}

// ------------------------------------------------------------- MP tile ---
//
// "Pair" kernel for 3..16 rows: one v_mfma_i32_16x16x64_i8 takes two weight
// blocks (b, b+1) of 16 rows against 8 activation rows.  A lane (i, q) feeds
// the weights of row i: half q%2 of block b + q/2 (for a Q8_0 cell that is 16
// contiguous bytes, so the wave reads the two cells, 1 KB, at once).  The
// prepared activation chunk puts row j's codes of block b in the columns
// j < 8 and of block b+1 in the columns 8 + j, with zeros where the other
// block's weights would meet them, so column j holds the exact int32 dot of
// block b and column 8 + j that of block b+1.
//
// With H >= 2 lane parts, blocks b and b+1 at the same u are lane parts h and
// h+1 (h even): columns j and 8 + j accumulate the two lane parts, and the
// first level of the lane-part tree adds lanes i and i^8.  With H == 1 they
// are u and u+1 of the one lane part: lane i adds its own block, then its
// partner's, in that order.

// Split of a tile's work over waves (H >= 2 means S == 4): W2 waves share a
// wave part, each taking PPW lane-part pairs, and NT 16-row image tiles that
// share each step's activation chunk.  Two widths: narrow (more, smaller
// tiles: more waves to hide latency) and wide (NT as large as 128 registers
// allow without spilling: the activation chunk is loaded once per NT KB of
// weights, and fewer tiles fit the workgroups resident at once).
__host__ __device__ constexpr int mp_w2(int H) { return H >= 4 ? 2 : 1; }
__host__ __device__ constexpr int mp_nt_base(int H, int G, bool wide) {
  return wide ? (H == 2 || H == 4 ? (G == 2 ? 2 : 3) : (G == 2 ? 1 : 2)) : (H == 8 || G == 2 ? 1 : 2);
}
// Q4_K decodes each tile's sub-block scales and offsets in registers as well:
// its wide tiles take one tile fewer (as many would spill).
__host__ __device__ constexpr int mp_nt(int H, int G, bool wide, int fmt = FMT_Q8) {
  return fmt == FMT_Q4K && wide && mp_nt_base(H, G, wide) > 1 ? mp_nt_base(H, G, wide) - 1
                                                              : mp_nt_base(H, G, wide);
}
// block-pair steps in flight per wave (even: step j's lane-part pair is j & 1)
__host__ __device__ constexpr int mp_la(int NT, int G) { return NT * G == 1 ? 4 : 2; }
constexpr int MP_NV_MAX = 16;  // floats per lane a wave passes to the combine (NT * G * 4)

__device__ __forceinline__ float lane_xor8(float v) {
  // DPP row_ror:8 within each row of 16 lanes: lane i reads lane i ^ 8
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
}

// One step: one block pair for NT tiles and G row groups.
template <int NT, int G>
struct MpStep {
  uint4 a[NT];  // weight codes (16 bytes)
  uint4 x[G];   // activation chunk (16 bytes)
  float dx[G];
  int ns[G];
  int b;  // first block of the pair
};

template <int NT>
struct MpAddr {
  const uint8_t* code[NT];  // tile code planes (wave-uniform)
  uint32_t aoff;            // lane offset: bytes in a cell pair
  const uint8_t* xc;        // pair-order chunks (uniform)
  const float* xd;
  const int* xn;
  int groups;               // row groups in the workspace
  const uint16_t* sl[NT];   // the wave's staged scales of each tile (LDS), from block sb0 on
  int sb0;
  int mplane;               // Q4_K: fp16 units from the staged (sc, m) plane to the (d, dmin) plane
  uint32_t soff;            // lane offset in a staged block pair (fp16 units)
  // Gathered row order (rows picked by the tile's s_src map): this lane's
  // element (row * kbp + its block's offset in the pair) per row group, and
  // whether its bytes meet its column's block (else they are zero).
  int64_t gsrc[2];
  bool xon;   // the lane's 16 bytes of a pair-order chunk are codes, not the zeros (not loaded)
  int ghalf;  // 0 or 16: the half of the block's codes
  bool gon;
  // The activation codes as a raw buffer from xc: a lane whose 16 bytes are
  // the zeros adds XOFF_ZERO to its offsets, past the buffer's range, and the
  // load returns zeros (no branch around the loads, so the waits before a
  // step's compute can count the loads issued after its own).
  __amdgpu_buffer_rsrc_t xr;
  uint32_t xlane;  // the lane's byte offset in a chunk, or XOFF_ZERO (pair order); ghalf or XOFF_ZERO (gathered)
};
constexpr uint32_t XOFF_ZERO = 0x80000000u;
constexpr int XBUF_RECORDS = 0x7FFFFFF0;  // the buffer's byte range: every real offset is below it
constexpr int XBUF_WORD3 = 0x00020000;    // raw (untyped) buffer, 32-bit data format

// The exact int32 dots of one pair step: lane (i, q) holds 16 bytes of weight
// codes (araw: Q8_0 codes, or Q4_0 packed nibbles whose half sh = 0 / 4 it
// feeds) and 16 bytes of the activation chunk; c[v] is the dot of weight row
// 4q + v with column i, starting from ns (Q4_0: -8 * sum of that column's
// activation codes).
template <int FMT>
__device__ __forceinline__ v4i pair_dots(uint4 araw, uint4 x, int ns, int sh) {
  uint4 av = araw;
  if constexpr (FMT == FMT_Q4) {
    // codes kept as c XOR 8: the lane's nibble to the high half of each byte
    // (a 64-bit shift moves two words; the mask clears what crosses), the int8
    // 16 (c - 8), so the product is sixteen times the dot and needs no start value
    const uint64_t lo = ((uint64_t)av.y << 32 | av.x) << (4 - sh), hi = ((uint64_t)av.w << 32 | av.z) << (4 - sh);
    av.x = (uint32_t)lo & 0xF0F0F0F0u;
    av.y = (uint32_t)(lo >> 32) & 0xF0F0F0F0u;
    av.z = (uint32_t)hi & 0xF0F0F0F0u;
    av.w = (uint32_t)(hi >> 32) & 0xF0F0F0F0u;
  } else if constexpr (FMT == FMT_Q4K) {
    av.x = (av.x >> sh) & 0x0F0F0F0Fu;
    av.y = (av.y >> sh) & 0x0F0F0F0Fu;
    av.z = (av.z >> sh) & 0x0F0F0F0Fu;
    av.w = (av.w >> sh) & 0x0F0F0F0Fu;
  }
  const v4i a = {(int)av.x, (int)av.y, (int)av.z, (int)av.w};
  const v4i bx = {(int)x.x, (int)x.y, (int)x.z, (int)x.w};
  v4i c = {ns, ns, ns, ns};
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bx, c, 0, 0, 0);
}

// Lane offset of a pair step's weight bytes inside the two cells of blocks
// (b, b + 1): Q8_0 lane (i, q) reads half q % 2 of block b + q / 2 of row i;
// Q4_0 lanes q = 0, 1 read block b's 16 bytes of row i, q = 2, 3 block b + 1's.
template <int FMT>
__device__ __forceinline__ uint32_t pair_aoff(int i, int q) {
  return FMT == FMT_Q8 ? (uint32_t)(q * 256 + i * 16) : (uint32_t)((q >> 1) * 256 + i * 16);
}

template <int NT>
__device__ __forceinline__ uint4 xbuf_load(const MpAddr<NT>& ad, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(ad.xr, (int)off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int FMT, int NT, int G, bool GATHER>
__device__ __forceinline__ void mp_load(MpStep<NT, G>& st, const MpAddr<NT>& ad, int lane, int b) {
  constexpr int CB = FMT == FMT_Q8 ? 512 : 256;
  // (offsets from the tile's uniform base fit 32 bits: the scalar-base load
  // form; Q4_K, whose decode holds more registers, measured slower with it)
#pragma unroll
  for (int t = 0; t < NT; t++)
    st.a[t] = FMT == FMT_Q4K ? ld16_stream(ad.code[t] + (size_t)b * CB + ad.aoff)
                             : ld16_stream(ad.code[t] + (uint32_t)(b * CB + (int)ad.aoff));
  st.b = b;
  if (GATHER) {
#pragma unroll
    for (int g = 0; g < G; g++) {
      const int64_t e = ad.gsrc[g] + b;
      st.x[g] = xbuf_load(ad, (uint32_t)e * 32u + ad.xlane);
      st.dx[g] = ad.xd[e];
      st.ns[g] = FMT == FMT_Q4K ? ad.xn[e] : 0;
    }
    return;
  }
  const uint32_t chunk0 = (uint32_t)(b >> 1) * (uint32_t)ad.groups;
#pragma unroll
  for (int g = 0; g < G; g++) {
    st.x[g] = xbuf_load(ad, (chunk0 + g) * 1024u + ad.xlane);
    st.dx[g] = ad.xd[(chunk0 + g) * 16 + (lane & 15)];
    st.ns[g] = FMT == FMT_Q4K ? ad.xn[(chunk0 + g) * 16 + (lane & 15)] : 0;
  }
}

template <int FMT, int NT, int G, int PP, bool SEQ>
__device__ __forceinline__ void mp_compute(float (&acc)[NT][PP][G][4], int pp, const MpStep<NT, G>& st,
                                           const MpAddr<NT>& ad, int sh) {
  if constexpr (FMT == FMT_Q4K) {
    // rows 4q .. 4q+3 of the lane's block bb from the wave's staged copy: their
    // 6-bit (sc, m) pairs ([block][16 rows] of sc | m << 8), and the fp32 d and
    // dmin of bb's superblock ([superblock][16 rows] of (d, dmin))
    const int bb = st.b + ((threadIdx.x & 15) >> 3);
#pragma unroll
    for (int t = 0; t < NT; t++) {
      const uint2 sm = *reinterpret_cast<const uint2*>(ad.sl[t] + (st.b - ad.sb0) * TILE + ad.soff);
      const float* ddp = reinterpret_cast<const float*>(ad.sl[t] + ad.mplane) +
                         (((bb >> 3) - (ad.sb0 >> 3)) * TILE + (int)(ad.soff & 15u)) * 2;
      const float4 d01 = *reinterpret_cast<const float4*>(ddp), d23 = *reinterpret_cast<const float4*>(ddp + 4);
      const unsigned s4[4] = {sm.x & 0xffffu, sm.x >> 16, sm.y & 0xffffu, sm.y >> 16};
      const float dv[4] = {d01.x, d01.z, d23.x, d23.z}, mv[4] = {d01.y, d01.w, d23.y, d23.w};
      float D[4], M[4];
#pragma unroll
      for (int v = 0; v < 4; v++) {
        D[v] = dv[v] * (float)(s4[v] & 255u);
        M[v] = mv[v] * (float)(s4[v] >> 8);
      }
#pragma unroll
      for (int g = 0; g < G; g++) {
        const v4i c = pair_dots<FMT>(st.a[t], st.x[g], 0, sh);
        const int xsum = -(st.ns[g] / 8);
        const float dx = st.dx[g];
#pragma unroll
        for (int v = 0; v < 4; v++) {
          float& r = acc[t][PP == 1 ? 0 : pp][g][v];
          const float tv = __builtin_fmaf((float)c[v], D[v], -((float)xsum * M[v]));
          if (SEQ) {
            // block b (this lane), then block b+1 (lane i ^ 8)
            const float pt = lane_xor8(tv), pdx = lane_xor8(dx);
            r = __builtin_fmaf(tv, dx, r);
            r = __builtin_fmaf(pt, pdx, r);
          } else {
            r = __builtin_fmaf(tv, dx, r);
          }
        }
      }
    }
    return;
  }
#pragma unroll
  for (int t = 0; t < NT; t++) {
    // fp16 scales of rows 4q .. 4q+3 of the lane's block, from the wave's staged copy
    const uint2 wv = *reinterpret_cast<const uint2*>(ad.sl[t] + (st.b - ad.sb0) * TILE + ad.soff);
#pragma unroll
    for (int g = 0; g < G; g++) {
      const v4i c = pair_dots<FMT>(st.a[t], st.x[g], st.ns[g], sh);
      // Q4_0: sixteen times the dots against dx / 16 (the same products and sums)
      const float dxg = FMT == FMT_Q4 ? st.dx[g] * 0.0625f : st.dx[g];
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const float f = (float)c[v], m = mul_h_f(v < 2 ? wv.x : wv.y, v & 1, dxg);
        float& r = acc[t][PP == 1 ? 0 : pp][g][v];
        if (SEQ) {
          // block b (this lane), then block b+1 (lane i ^ 8)
          const float pf = lane_xor8(f), pm = lane_xor8(m);
          r = __builtin_fmaf(f, m, r);
          r = __builtin_fmaf(pf, pm, r);
        } else {
          r = __builtin_fmaf(f, m, r);
        }
      }
    }
  }
}

// LDS of the pair kernel: the combine area (red; a wave's slice at wave * NV *
// 64 floats) and the waves' staged scales (scl; a wave's NT tiles from
// wave * NT * sc_stride).  Q4_K stages more (a (sc, m) pair per row and
// block, fp32 d and dmin per row and superblock), so its set kernels give a
// wave one region for both (red_ws
// floats = scl_ws / 2 fp16 units apart): a wave writes its combine values only
// after its own step loop, and stages the next tile's scales only after the
// combine's last barrier, so a workgroup needs the larger of the two per wave,
// not their sum.
struct MpLds {
  float* red;
  int red_ws;
  uint16_t* scl;
  int scl_ws;
};

// One MP tile: groups of S*W2 waves, each group NT 16-row image tiles; G
// groups of eight activation rows from the pair-order workspace, or (GATHER)
// from a row-order workspace through the tile's s_src map.
template <int FMT, int H, int G, int NT, bool GATHER, bool PF = false>
__device__ void mp_tile(const TileArgs& ta, int R, const MpLds& ml, int count = 1, int64_t row_stride = 0) {
  constexpr int CB = FMT == FMT_Q8 ? 512 : 256;
  constexpr bool SEQ = H == 1;
  constexpr int W2 = mp_w2(H);
  constexpr int PPW = SEQ ? 1 : H / 2 / W2;  // lane-part pairs per wave (1 or 2)
  const PartPlan& pl = ta.pl;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & (WAVE - 1);
  const int gw = pl.S * W2;  // waves per group
  const int g = wave / gw, wg = wave - g * gw, s = wg / W2, hw = wg - s * W2;
  const int i = lane & 15, q = lane >> 4;
  const int64_t ntiles = np_of(ta.n) / TILE;
  // staged scales of one tile's wave part, in fp16 units: fp16 per (row, block); Q4_K a (sc, m) byte pair per
  // (row, block), then fp32 (d, dmin) per (row, superblock touched: at most H*BS/8 + 2)
  const int sc_stride = pl.H * pl.BS * TILE + (FMT == FMT_Q4K ? (pl.H * pl.BS / 8 + 2) * TILE * 4 : 0);
  MpAddr<NT> ad;
  const uint16_t* scale[NT];
#pragma unroll
  for (int t = 0; t < NT; t++)
    ad.sl[t] = FMT == FMT_Q4K ? ml.scl + wave * ml.scl_ws + t * sc_stride : ml.scl + (wave * NT + t) * sc_stride;
  float* red = ml.red;
  ad.aoff = pair_aoff<FMT>(i, q);
  ad.soff = (uint32_t)((i >> 3) * 16 + 4 * q);
  ad.mplane = pl.H * pl.BS * TILE;  // Q4_K: fp16 units from the (sc, m) plane to the (d, dmin) plane
  ad.xc = reinterpret_cast<const uint8_t*>(ta.prep.codes);
  ad.xd = ta.prep.dx;
  ad.xn = ta.prep.nsx;
  ad.groups = (R + 7) >> 3;
  ad.xon = (i < 8) == (q < 2);
  ad.xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(ad.xc), 0, XBUF_RECORDS, XBUF_WORD3);
  ad.xlane = ad.xon ? (uint32_t)lane * 16u : XOFF_ZERO;
  if (GATHER) {
#pragma unroll
    for (int gg = 0; gg < G; gg++) {
      const int ar = min(gg * 8 + (i & 7), R - 1);  // columns past R read a real row, store nothing
      ad.gsrc[gg] = (int64_t)ta.s_src[ar] * ta.kbp + (i >> 3);
    }
    ad.ghalf = (q & 1) * 16;
    ad.gon = (i < 8) == (q < 2);
    ad.xlane = ad.gon ? (uint32_t)ad.ghalf : XOFF_ZERO;
  }
  const int sh = (q & 1) * 4;

  const int BS = pl.BS;
  const int nsteps = SEQ ? BS / 2 : BS * PPW;  // >= 4 (BS >= 8, even when H == 1)
  const int bs0 = s * H * BS + 2 * hw * PPW;
  // first block of step j
  auto blk = [&](int j) {
    if (SEQ) return bs0 + 2 * j;
    const int u = PPW == 2 ? j >> 1 : j, pp = PPW == 2 ? j & 1 : 0;
    return bs0 + H * u + 2 * pp;
  };
  // The weight scales of the wave part's blocks [sb0, sb0 + H*BS) of each tile
  // go to the wave's own LDS region once per tile (16 lanes would otherwise
  // load the same four scales every step).  Their loads are issued first, then
  // the first steps', so waiting for them waits for nothing else.
  ad.sb0 = s * H * pl.BS;
  const int nsv = H * pl.BS * 2;  // 16-byte pieces per tile (kbp/S blocks x 32 bytes)
  constexpr int MP_LA = mp_la(NT, G);
  uint4 sv[NT];
  MpStep<NT, G> st[MP_LA];
  int64_t wrow0 = 0;  // first row of this group's tiles
  // Points the wave at the tile group starting at row0 and issues its scale
  // loads and its first MP_LA steps.
  auto start = [&](int64_t row0) {
    wrow0 = row0 + (int64_t)g * TILE * NT;
#pragma unroll
    for (int t = 0; t < NT; t++) {
      const int64_t it0 = (wrow0 >> 4) + t;
      const int64_t it = it0 < ntiles ? it0 : ntiles - 1;  // past the last tile: reread it, store nothing
      ad.code[t] = ta.code + ((size_t)it * ta.kbp) * CB;
      scale[t] = ta.scale + ((size_t)it * ta.kbp) * TILE;
    }
    if constexpr (FMT != FMT_Q4K) {
#pragma unroll
      for (int t = 0; t < NT; t++)
        if (lane < nsv) sv[t] = ld16(scale[t] + (size_t)ad.sb0 * TILE + lane * 8);
    }
    // (nsteps >= 4 >= MP_LA: no bounds branch here, which would leave a path
    // on which the first step's loads are the last issued, and the step loop
    // would then wait for every load in flight before each round)
#pragma unroll
    for (int jj = 0; jj < MP_LA; jj++) mp_load<FMT, NT, G, GATHER>(st[jj], ad, lane, blk(jj));
  };
  // The started tile's scales into the wave's LDS region (the wave is done
  // reading the previous tile's).
  auto stage = [&]() {
    if constexpr (FMT == FMT_Q4K) {
      // the headers of the superblocks the wave part touches: each block's
      // (sc, m) pair per row, and each superblock's fp32 (d, dmin) per row
      const int nblk = pl.H * pl.BS, sb_lo = ad.sb0 >> 3, nsb = ((ad.sb0 + nblk - 1) >> 3) - sb_lo + 1;
#pragma unroll
      for (int t = 0; t < NT; t++) {
        const uint8_t* hb = reinterpret_cast<const uint8_t*>(scale[t]);
        uint16_t* smd = const_cast<uint16_t*>(ad.sl[t]);
        float2* ddd = reinterpret_cast<float2*>(smd + ad.mplane);
        for (int e = lane; e < nsb * TILE; e += WAVE) {
          const int sbi = sb_lo + (e >> 4), row = e & 15;
          const uint4 h = ld16(hb + ((size_t)sbi * TILE + row) * 16);
          ddd[e] = make_float2(h2f((uint16_t)(h.x & 0xffffu)), h2f((uint16_t)(h.x >> 16)));
#pragma unroll
          for (int j = 0; j < 8; j++) {
            const int b = sbi * 8 + j - ad.sb0;
            if (b >= 0 && b < nblk) {
              unsigned sc, m;
              q4k_scm(h, j, sc, m);
              smd[b * TILE + row] = (uint16_t)(sc | (m << 8));
            }
          }
        }
      }
      return;
    }
#pragma unroll
    for (int t = 0; t < NT; t++) {
      uint4* dst = reinterpret_cast<uint4*>(const_cast<uint16_t*>(ad.sl[t]));
      if (lane < nsv) dst[lane] = sv[t];
      for (int e = lane + WAVE; e < nsv; e += WAVE) dst[e] = ld16(scale[t] + (size_t)ad.sb0 * TILE + e * 8);
    }
  };
  start(ta.row0);
  stage();
  // The workgroup's tiles of this projection: row0, row0 + row_stride, ...
  // (PF: the next one's loads are in flight while this one is combined and
  // stored; otherwise one tile per call).
  for (int c = 0; c < (PF ? count : 1); c++) {
    float acc[NT][PPW][G][4];
#pragma unroll
    for (int t = 0; t < NT; t++)
#pragma unroll
      for (int p = 0; p < PPW; p++)
#pragma unroll
        for (int gg = 0; gg < G; gg++)
#pragma unroll
          for (int v = 0; v < 4; v++) acc[t][p][gg][v] = 0.0f;
    int j = 0;
    // steps whose every slot has a next step to load: no branch around the
    // loads, so the wait before a step's compute counts only the loads issued
    // after its own (a branch there makes it wait for every load in flight)
    for (; j + 2 * MP_LA <= nsteps; j += MP_LA) {
#pragma unroll
      for (int jj = 0; jj < MP_LA; jj++) {
        mp_compute<FMT, NT, G, PPW, SEQ>(acc, jj & 1, st[jj], ad, sh);
        mp_load<FMT, NT, G, GATHER>(st[jj], ad, lane, blk(j + jj + MP_LA));
        // keep each step's loads ahead of the next step's compute (moved after it,
        // every compute of the round would wait for all of the round's loads;
        // Q8_0's two-group steps measured 0.6 % faster without)
        if constexpr (G == 1 || FMT != FMT_Q8) __builtin_amdgcn_sched_barrier(0);
      }
    }
    for (; j < nsteps; j += MP_LA) {
#pragma unroll
      for (int jj = 0; jj < MP_LA; jj++) {
        if (j + jj < nsteps) {
          mp_compute<FMT, NT, G, PPW, SEQ>(acc, jj & 1, st[jj], ad, sh);
          if (j + jj + MP_LA < nsteps) mp_load<FMT, NT, G, GATHER>(st[jj], ad, lane, blk(j + jj + MP_LA));
        }
      }
    }
    // the wave's pairs by the lane-part tree: (h + h^1) across lanes i, i^8, then pair + pair
    float res[NT][G][4];
#pragma unroll
    for (int t = 0; t < NT; t++)
#pragma unroll
      for (int gg = 0; gg < G; gg++)
#pragma unroll
        for (int v = 0; v < 4; v++) {
          float val = acc[t][0][gg][v];
          if (!SEQ) {
            val = val + lane_xor8(val);
            if (PPW == 2) val = val + (acc[t][PPW - 1][gg][v] + lane_xor8(acc[t][PPW - 1][gg][v]));
          }
          res[t][gg][v] = val;
        }
    const int64_t row_out = wrow0;
    const bool more = PF && c + 1 < count;
    if (more) start(ta.row0 + (int64_t)(c + 1) * row_stride);
    if (gw > 1) {
      // the wave's values to the combine area
      constexpr int NV = NT * G * 4;
      const int ws = FMT == FMT_Q4K ? ml.red_ws : NV * WAVE;
#pragma unroll
      for (int t = 0; t < NT; t++)
#pragma unroll
        for (int gg = 0; gg < G; gg++)
#pragma unroll
          for (int v = 0; v < 4; v++) red[wave * ws + ((t * G + gg) * 4 + v) * WAVE + lane] = res[t][gg][v];
      __syncthreads();
      // One output per thread, over all groups of the workgroup: value o of
      // lane li + 16 lq (li < 8) of each wave of the group, summed as the W2
      // pair groups of a wave part (the tree's upper level), then the wave
      // parts left to right.
      constexpr int OUT = NV * 32;
      const int ngroups = WAVES / gw;
      // (the thread index through an opaque copy: the indexes below are then
      // formed here, not hoisted out of the tile loops, where they would hold
      // registers through the step loop)
      int e0;
      asm volatile("v_mov_b32 %0, %1" : "=v"(e0) : "v"((int)threadIdx.x));
#pragma unroll 1
      for (int e = e0; e < ngroups * OUT; e += WG) {
        const int gi = e / OUT, r = e - gi * OUT, o = r >> 5, li = r & 7, lq = (r >> 3) & 3;
        const int t = o / (G * 4), gg = (o >> 2) % G, v = o & 3;
        const int ar = gg * 8 + li;  // activation row of the output's column
        const int64_t row = row_out + (int64_t)(gi - g) * TILE * NT + t * TILE + 4 * lq + v;
        if (ar >= R || row >= ta.n) continue;
        const int w0 = gi * gw, off = o * WAVE + lq * 16 + li;
        float x = 0.0f;
        for (int s2 = 0; s2 < pl.S; s2++) {
          float part = red[(w0 + s2 * W2) * ws + off];
          if (W2 == 2) part = part + red[(w0 + s2 * W2 + 1) * ws + off];
          x = s2 == 0 ? part : x + part;
        }
        ta.y[(int64_t)ta.s_dst[ar] * ta.ldy + row] = x;
      }
      __syncthreads();  // the combine area is free for the next tile
    } else {
      if (i < 8) {
#pragma unroll
        for (int gg = 0; gg < G; gg++) {
          const int ar = gg * 8 + i;  // activation row of this lane's column
          if (ar < R) {
#pragma unroll
            for (int t = 0; t < NT; t++)
#pragma unroll
              for (int v = 0; v < 4; v++) {
                const int64_t row = row_out + t * TILE + 4 * q + v;
                if (row < ta.n) ta.y[(int64_t)ta.s_dst[ar] * ta.ldy + row] = res[t][gg][v];
              }
          }
        }
      }
    }
    if (more) stage();
  }
}

// ----------------------------------------------------------- set kernels ---

struct ProjDev {
  const uint8_t* code;
  const uint16_t* scale;
  Prep prep;
  const float* xf;
  float* y;
  int64_t n, k;
  int kb, kbp;
  int tiles;
  int rows_per_tile;
  PartPlan pl;
  int ucx;   // RL staging round
  int wide;  // pair kernel, per-projection width (MP_MIXED launches)
};
struct SetArgs {
  ProjDev p[QG_MAX_SET];
  int count;
  int total_tiles;
  int wave_lds;  // pair kernel: bytes of LDS per wave (combine slice and staged scales)
};

__device__ __forceinline__ void identity_map(int* s_map) {
  if (threadIdx.x < QG_MAX_ROWS) {
    s_map[threadIdx.x] = threadIdx.x;
    s_map[QG_MAX_ROWS + threadIdx.x] = threadIdx.x;
  }
  __syncthreads();
}

__device__ __forceinline__ TileArgs tile_args(const ProjDev& d, int64_t row0, const int* s_map, int lds_x) {
  TileArgs ta;
  ta.code = d.code;
  ta.scale = d.scale;
  ta.n = d.n;
  ta.kbp = d.kbp;
  ta.kb = d.kb;
  ta.k = d.k;
  ta.row0 = row0;
  ta.prep = d.prep;
  ta.xf = d.xf;
  ta.s_src = s_map;
  ta.y = d.y;
  ta.ldy = d.n;
  ta.s_dst = s_map + QG_MAX_ROWS;
  ta.lds_x = lds_x;
  ta.pl = d.pl;
  ta.ucx = d.ucx;
  return ta;
}

// Tiles are numbered projection by projection; workgroup w takes tiles w,
// w + G, w + 2G, ... and keeps a projection's activation rows in LDS while its
// tiles last.
// LA: blocks in flight per lane -- 2 when the launch fills the GPU (the many
// waves give the memory parallelism; at most 80 registers, 96 for two Q8_0
// rows, which would spill, so that three 512-thread workgroups fit a CU and a
// layer's tiles are resident at once), 8 with one workgroup per CU (a
// lane's blocks all in flight at once: launches of at most one tile per CU,
// which are latency-bound, and one row over many rounds of tiles).
template <int FMT, int R, bool FUSED, int LA>
__global__ __launch_bounds__(WG) __attribute__((amdgpu_waves_per_eu(LA > 2 ? 2 : (FMT == FMT_Q8 && R == 2 ? 5 : 6))))
void rl_set_kernel(SetArgs a, int lds_x) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int s_map[2 * QG_MAX_ROWS];
  identity_map(s_map);
  float* red = reinterpret_cast<float*>(lds + lds_x);
  int staged = -1, parity = 0;
  for (int tile = blockIdx.x; tile < a.total_tiles; tile += gridDim.x) {
    int p = 0, t0 = tile;
    while (p + 1 < a.count && t0 >= a.p[p].tiles) t0 -= a.p[p++].tiles;
    const ProjDev& d = a.p[p];
    const TileArgs ta = tile_args(d, (int64_t)t0 * d.rows_per_tile, s_map, lds_x);
    const bool full = rl_tile<FMT, R, FUSED, LA>(ta, lds, red, parity, p != staged);
    staged = full ? p : -1;
    // the combine area alternates only between tiles that pass its barrier, so
    // a buffer is rewritten only after everyone has read it
    if (d.pl.S > 1) parity ^= 1;
  }
}

// Width of a pair-kernel launch: every projection on narrow tiles, every one
// on wide tiles, or each on its own (ProjDev::wide).
enum { MP_NARROW = 0, MP_WIDE = 1, MP_MIXED = 2 };

// The workgroup's tiles of one projection at width W (tiles row0, row0 +
// stride, ...: cnt of them, one unless PF).
template <int FMT, int G, bool W, bool PF>
__device__ __forceinline__ void mp_tiles(const TileArgs& ta, int R, const MpLds& ml, int cnt,
                                         int64_t stride) {
  const int H = ta.pl.H;
  if (H == 1) mp_tile<FMT, 1, G, mp_nt(1, G, W, FMT), false, PF>(ta, R, ml, cnt, stride);
  else if (H == 2) mp_tile<FMT, 2, G, mp_nt(2, G, W, FMT), false, PF>(ta, R, ml, cnt, stride);
  else if (H == 4) mp_tile<FMT, 4, G, mp_nt(4, G, W, FMT), false, PF>(ta, R, ml, cnt, stride);
  else mp_tile<FMT, 8, G, mp_nt(8, G, W, FMT), false, PF>(ta, R, ml, cnt, stride);
}

// PF: each workgroup's narrow tiles of a projection in one mp_tile call, the
// next tile's loads in flight while a tile is combined (for launches of
// several rounds; it costs registers, so Q8_0 only).
template <int FMT, int G, int WIDTH, bool PF>
__global__ __launch_bounds__(WG) __attribute__((amdgpu_waves_per_eu(4))) void mp_set_kernel(SetArgs a, int R) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int s_map[2 * QG_MAX_ROWS];
  identity_map(s_map);
  // Q4_K: one region of a.wave_lds bytes per wave for its combine slice and its staged scales; otherwise the
  // combine area, then the staged scales
  const MpLds ml = FMT == FMT_Q4K
                       ? MpLds{reinterpret_cast<float*>(lds), a.wave_lds / 4, reinterpret_cast<uint16_t*>(lds),
                               a.wave_lds / 2}
                       : MpLds{reinterpret_cast<float*>(lds), 0,
                               reinterpret_cast<uint16_t*>(lds + WAVES * WAVE * MP_NV_MAX * 4), 0};
  constexpr bool MP_PF = PF && WIDTH == MP_NARROW && FMT == FMT_Q8;
  for (int tile = blockIdx.x; tile < a.total_tiles;) {
    int p = 0, t0 = tile;
    while (p + 1 < a.count && t0 >= a.p[p].tiles) t0 -= a.p[p++].tiles;
    const ProjDev& d = a.p[p];
    const TileArgs ta = tile_args(d, (int64_t)t0 * d.rows_per_tile, s_map, 0);
    // this workgroup's tiles of the projection, t0, t0 + G, ..., in one call
    // (narrow Q8_0 tiles; the others have no registers to spare for it)
    const int cnt = MP_PF ? (d.tiles - 1 - t0) / (int)gridDim.x + 1 : 1;
    const int64_t stride = (int64_t)gridDim.x * d.rows_per_tile;
    if constexpr (WIDTH == MP_NARROW) {
      mp_tiles<FMT, G, false, MP_PF>(ta, R, ml, cnt, stride);
    } else if constexpr (WIDTH == MP_WIDE) {
      mp_tiles<FMT, G, true, false>(ta, R, ml, cnt, stride);
    } else {
      if (d.wide) mp_tiles<FMT, G, true, false>(ta, R, ml, cnt, stride);
      else mp_tiles<FMT, G, false, false>(ta, R, ml, cnt, stride);
    }
    tile += cnt * (int)gridDim.x;
  }
}

// ------------------------------------------------------------- grouped ---

// One workgroup: the valid assignments ordered by (expert, index), then work
// items of at most 16 assignments of one expert.
__global__ __launch_bounds__(1024) void grouped_plan_kernel(const int32_t* __restrict__ expert,
                                                            const int32_t* __restrict__ x_index, int m,
                                                            int64_t n_experts, int x_rows, int* __restrict__ header,
                                                            int* __restrict__ sorted, int* __restrict__ items,
                                                            const float* __restrict__ x, int64_t k,
                                                            int8_t* __restrict__ xq, float* __restrict__ xd,
                                                            int* __restrict__ xn, uint8_t* __restrict__ fcodes,
                                                            float* __restrict__ fscales) {
  if (blockIdx.x > 0) {  // the input rows' quantization
    if (fcodes) plan_prepare_fp8(x, x_rows, k, fcodes, fscales, blockIdx.x - 1);
    else plan_prepare_q8(x, x_rows, k, xq, xd, xn, blockIdx.x - 1);
    return;
  }
  __shared__ int s_e[QG_MAX_ASSIGN];
  __shared__ int s_pos[QG_MAX_ASSIGN];  // sorted position -> assignment
  __shared__ int s_start[QG_MAX_ASSIGN];  // 1 where a work item starts
  __shared__ int s_ie[QG_MAX_ASSIGN], s_is[QG_MAX_ASSIGN], s_ic[QG_MAX_ASSIGN];  // work items
  __shared__ int s_bad, s_valid, s_cnt[2];
  const int tid = threadIdx.x, nt = blockDim.x;
  if (tid == 0) {
    s_bad = 0;
    s_valid = 0;
  }
  __syncthreads();
  for (int j = tid; j < m; j += nt) {
    const int e = expert[j], xi = x_index[j];
    const bool ok = e >= 0 && e < n_experts && xi >= 0 && xi < x_rows;
    s_e[j] = ok ? e : 0x7fffffff;
    atomicAdd(ok ? &s_valid : &s_bad, 1);
  }
  __syncthreads();
  for (int j = tid; j < m; j += nt) {
    const int e = s_e[j];
    if (e == 0x7fffffff) continue;
    int rank = 0, within = 0;
    for (int i = 0; i < m; i++) {
      const int f = s_e[i];
      rank += (f < e) || (f == e && i < j);
      within += (f == e && i < j);
    }
    s_pos[rank] = j;
    s_start[rank] = (within % QG_MAX_ROWS) == 0;
    sorted[rank] = j;
  }
  __syncthreads();
  const int nv = s_valid;
  // inclusive scan of the item starts (Hillis-Steele over <= QG_MAX_ASSIGN entries)
  for (int off = 1; off < nv; off <<= 1) {
    int vals[QG_MAX_ASSIGN / 1024];
    for (int p = tid, c = 0; p < nv; p += nt, c++) vals[c] = s_start[p] + (p >= off ? s_start[p - off] : 0);
    __syncthreads();
    for (int p = tid, c = 0; p < nv; p += nt, c++) s_start[p] = vals[c];
    __syncthreads();
  }
  for (int p = tid; p < nv; p += nt) {
    const int item = s_start[p] - 1;
    const bool first = p == 0 || s_start[p - 1] != s_start[p];
    if (first) {
      int cnt = 1;
      while (p + cnt < nv && s_start[p + cnt] == s_start[p]) cnt++;
      s_ie[item] = s_e[s_pos[p]];
      s_is[item] = p;
      s_ic[item] = cnt;
    }
  }
  if (tid == 0) header[1] = s_bad;
  __syncthreads();
  store_items_small_first(s_ie, s_is, s_ic, nv ? s_start[nv - 1] : 0, s_pos, s_cnt, items, header);
}

// Blocks in flight per lane in the small-item kernel: 4, or 8 (a lane's whole
// chain: the partition gives every lane part at least 8 blocks) when there
// are no more units than CUs, so each has a workgroup of its own and latency,
// not occupancy, bounds the launch.
constexpr int GROUPED_LA = 4;
constexpr int GROUPED_LA_FEW = 8;

// GLU: the rows are the SwiGLU of gate/up rows ta.xf, quantized while staged
// (all of kbp fits: the launcher checks).
template <int R, bool GLU, int LA>
__device__ __forceinline__ void grouped_rows(TileArgs ta, uint8_t* lds, float* red) {
  ta.ucx = rl_round(ta.lds_x, R, ta.pl, FMT_Q8);
  rl_tile<FMT_Q8, R, GLU, LA, GLU>(ta, lds, red, 0, true);
}

// Unit (item, tile) of an item of at most GROUPED_SMALL_ROWS rows:
// lanes-own-rows tiles.  Every thread calls it.  GLU: the activation row of
// assignment a is the SwiGLU of row a of glu (gate values, then up values;
// rows 2k wide), quantized in the tile's staging; prep is not read.
template <bool GLU, int LA = GROUPED_LA>
__device__ __forceinline__ void grouped_small_unit(const uint8_t* __restrict__ images, int64_t expert_bytes,
                                                   size_t scale_off, int64_t n, int64_t k, int kbp, const PartPlan& pl,
                                                   const Prep& prep, const int* __restrict__ sorted,
                                                   const int* __restrict__ items, const int32_t* __restrict__ x_index,
                                                   float* y, int lds_x, int item, int tile, uint8_t* lds, int* s_map,
                                                   const float* glu) {
  float* red = reinterpret_cast<float*>(lds + lds_x);
  const int e = items[3 * item], start = items[3 * item + 1], cnt = items[3 * item + 2];
  __syncthreads();  // the previous unit is done with s_map and LDS
  if ((int)threadIdx.x < cnt) {
    const int a = sorted[start + threadIdx.x];
    s_map[threadIdx.x] = x_index ? x_index[a] : a;
    s_map[QG_MAX_ROWS + threadIdx.x] = a;
  }
  __syncthreads();
  const uint8_t* img = images + (size_t)e * expert_bytes;
  TileArgs ta;
  ta.code = img;
  ta.scale = reinterpret_cast<const uint16_t*>(img + scale_off);
  ta.n = n;
  ta.kbp = kbp;
  ta.kb = (int)kb_of(k);
  ta.k = k;
  ta.row0 = (int64_t)tile * (WG >> pl.lgP);
  ta.prep = prep;
  ta.xf = glu;
  ta.s_src = s_map;
  ta.y = y;
  ta.ldy = n;
  ta.s_dst = s_map + QG_MAX_ROWS;
  ta.lds_x = lds_x;
  ta.pl = pl;
  ta.ucx = 0;  // set per row count
  if (cnt == 1) grouped_rows<1, GLU, LA>(ta, lds, red);
  else if (cnt == 2) grouped_rows<2, GLU, LA>(ta, lds, red);
}

// Items of at most GROUPED_SMALL_ROWS rows (the plan puts them first), when
// no item can have more: persistent over the (item, tile) units.
template <bool GLU, int LA>
__global__ __launch_bounds__(WG) void grouped_kernel(const uint8_t* __restrict__ images, int64_t expert_bytes,
                                                     size_t scale_off, int64_t n, int64_t k, int kbp, PartPlan pl,
                                                     Prep prep,
                                                     const int* __restrict__ header, const int* __restrict__ sorted,
                                                     const int* __restrict__ items,
                                                     const int32_t* __restrict__ x_index, float* y, int lds_x,
                                                     int tiles, const float* glu) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int s_map[2 * QG_MAX_ROWS];
  const int units = header[2] * tiles;
  for (int u = blockIdx.x; u < units; u += gridDim.x)  // uniform over the workgroup
    grouped_small_unit<GLU, LA>(images, expert_bytes, scale_off, n, k, kbp, pl, prep, sorted, items, x_index, y,
                                lds_x, u / tiles, u % tiles, lds, s_map, glu);
}

// Rows of a grouped item in the pair kernel's tiles (one 16-row image tile per
// wave group), the activation rows gathered from the row-order workspace.
template <int G>
__device__ __forceinline__ void grouped_mp_tile(const TileArgs& ta, int R, const MpLds& ml) {
  switch (ta.pl.H) {
    case 1: mp_tile<FMT_Q8, 1, G, 1, true>(ta, R, ml); break;
    case 2: mp_tile<FMT_Q8, 2, G, 1, true>(ta, R, ml); break;
    case 4: mp_tile<FMT_Q8, 4, G, 1, true>(ta, R, ml); break;
    default: mp_tile<FMT_Q8, 8, G, 1, true>(ta, R, ml); break;
  }
}

// Rows per pair-tile unit of a grouped launch.
static inline int grouped_mp_rows(const PartPlan& pl) { return (WAVES / (pl.S * mp_w2(pl.H))) * TILE; }

// Unit (item, tile) of an item of more than GROUPED_SMALL_ROWS rows: the pair
// tile, activation rows gathered.  Every thread calls it.
__device__ __forceinline__ void grouped_big_unit(const uint8_t* __restrict__ images, int64_t expert_bytes,
                                                 size_t scale_off, int64_t n, int64_t k, int kbp, const PartPlan& pl,
                                                 const Prep& prep, const int* __restrict__ sorted,
                                                 const int* __restrict__ items, const int32_t* __restrict__ x_index,
                                                 float* y, int item, int tile, uint8_t* lds, int* s_map) {
  // combine area, then the waves' staged scales
  const MpLds ml{reinterpret_cast<float*>(lds), 0, reinterpret_cast<uint16_t*>(lds + WAVES * WAVE * MP_NV_MAX * 4),
                 0};
  const int rpt = (WAVES / (pl.S * mp_w2(pl.H))) * TILE;
  const int e = items[3 * item], start = items[3 * item + 1], cnt = items[3 * item + 2];
  __syncthreads();  // the previous unit is done with s_map and LDS
  if ((int)threadIdx.x < cnt) {
    const int a = sorted[start + threadIdx.x];
    s_map[threadIdx.x] = x_index ? x_index[a] : a;
    s_map[QG_MAX_ROWS + threadIdx.x] = a;
  }
  __syncthreads();
  const uint8_t* img = images + (size_t)e * expert_bytes;
  TileArgs ta;
  ta.code = img;
  ta.scale = reinterpret_cast<const uint16_t*>(img + scale_off);
  ta.n = n;
  ta.kbp = kbp;
  ta.kb = (int)kb_of(k);
  ta.k = k;
  ta.row0 = (int64_t)tile * rpt;
  ta.prep = prep;
  ta.xf = nullptr;
  ta.s_src = s_map;
  ta.y = y;
  ta.ldy = n;
  ta.s_dst = s_map + QG_MAX_ROWS;
  ta.lds_x = 0;
  ta.pl = pl;
  ta.ucx = 0;
  if (cnt > 8) grouped_mp_tile<2>(ta, cnt, ml);
  else grouped_mp_tile<1>(ta, cnt, ml);
}

// Items of every size in one launch, persistent over the (item, tile) units:
// those of the items of more than GROUPED_SMALL_ROWS rows (pair tiles, the
// longer ones) first, then those of the small items (lanes-own-rows tiles).
// The two kinds of unit share the dynamic LDS (max of their needs); the
// small items' staged rows start at byte 0.
__global__ __launch_bounds__(WG) __attribute__((amdgpu_waves_per_eu(4))) void grouped_all_kernel(
    const uint8_t* __restrict__ images, int64_t expert_bytes, size_t scale_off, int64_t n, int64_t k, int kbp,
    PartPlan pl, Prep prep, const int* __restrict__ header, const int* __restrict__ sorted,
    const int* __restrict__ items, const int32_t* __restrict__ x_index, float* y, int lds_x, int tiles_s,
    int tiles_b) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int s_map[2 * QG_MAX_ROWS];
  const int nsmall = header[2];
  const int ub = (header[0] - nsmall) * tiles_b, units = ub + nsmall * tiles_s;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {  // uniform over the workgroup
    if (u < ub)
      grouped_big_unit(images, expert_bytes, scale_off, n, k, kbp, pl, prep, sorted, items, x_index, y,
                       nsmall + u / tiles_b, u % tiles_b, lds, s_map);
    else
      grouped_small_unit<false>(images, expert_bytes, scale_off, n, k, kbp, pl, prep, sorted, items, x_index, y,
                                lds_x, (u - ub) / tiles_s, (u - ub) % tiles_s, lds, s_map, nullptr);
  }
}

// ------------------------------------------------- routed MoE gate/up ---

static_assert(MOE_UP_PLAN_ROWS <= WAVES, "the gate/up launch routes a row a wave");

// The gate/up launch of a routed MoE step: every workgroup computes the
// step's plan from the router logits (moe_plan_block: the same plan in each),
// workgroup 0 stores it for the later launches, and the workgroups take the
// (item, tile) units as the grouped kernels do, the plan read from LDS.  The
// activation row of assignment j is row j / slots of the prepared input.
template <int LA>
__global__ __launch_bounds__(WG) void moe_up_small_kernel(const uint8_t* __restrict__ images, int64_t expert_bytes,
                                                          size_t scale_off, int64_t n, int64_t k, int kbp,
                                                          PartPlan pl, Prep prep, float* y, int lds_x, int tiles,
                                                          MoeUp up) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int s_map[2 * QG_MAX_ROWS];
  const int m = up.rows * (up.topk + up.shared);
  const PlanLds P = plan_carve(lds + up.plan_off, m, up.E);
  moe_plan_block<WG>(up.logits, up.rows, up.E, up.topk, up.shared != 0, P);
  if (blockIdx.x == 0) plan_store<WG>(P, m, up.expert, up.weight, up.x_index, up.header, up.sorted, up.items, up.dheader,
                                     up.ditems);
  const int units = P.misc[1] * tiles;  // every item is small (rows <= 2)
  for (int u = blockIdx.x; u < units; u += gridDim.x)
    grouped_small_unit<false, LA>(images, expert_bytes, scale_off, n, k, kbp, pl, prep, P.sorted, P.items, P.xi, y,
                                  lds_x, u / tiles, u % tiles, lds, s_map, nullptr);
}

__global__ __launch_bounds__(WG) __attribute__((amdgpu_waves_per_eu(4))) void moe_up_all_kernel(
    const uint8_t* __restrict__ images, int64_t expert_bytes, size_t scale_off, int64_t n, int64_t k, int kbp,
    PartPlan pl, Prep prep, float* y, int lds_x, int tiles_s, int tiles_b, MoeUp up) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int s_map[2 * QG_MAX_ROWS];
  const int m = up.rows * (up.topk + up.shared);
  const PlanLds P = plan_carve(lds + up.plan_off, m, up.E);
  moe_plan_block<WG>(up.logits, up.rows, up.E, up.topk, up.shared != 0, P);
  if (blockIdx.x == 0) plan_store<WG>(P, m, up.expert, up.weight, up.x_index, up.header, up.sorted, up.items, up.dheader,
                                     up.ditems);
  const int nsmall = P.misc[1];
  const int ub = (P.misc[0] - nsmall) * tiles_b, units = ub + nsmall * tiles_s;
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    if (u < ub)
      grouped_big_unit(images, expert_bytes, scale_off, n, k, kbp, pl, prep, P.sorted, P.items, P.xi, y,
                       nsmall + u / tiles_b, u % tiles_b, lds, s_map);
    else
      grouped_small_unit<false>(images, expert_bytes, scale_off, n, k, kbp, pl, prep, P.sorted, P.items, P.xi, y,
                                lds_x, (u - ub) / tiles_s, (u - ub) % tiles_s, lds, s_map, nullptr);
  }
}

// ------------------------------------------------ MoE down and combine ---
//
// One or two rows: the down projection of every assignment and the weighted
// combine in one launch.  Workgroup w takes output rows RT w .. RT w + RT - 1
// (RT = 8 or 16: half an image tile or one) of every assignment.  A wave task
// is NA = (64/H)/RT assignments and one wave part s; lane h * (64/H) + RT j + i
// is lane part h of row i for the task's assignment j.  The activation row of assignment a is the SwiGLU of its
// gate/up row, quantized in staging as the grouped launch's staging does it.
// A lane sums its blocks in order, the lane parts and then the wave parts
// follow the lanes-own-rows kernel's tree, so each assignment's output has the
// bits of the one-row dense call; the slots then add up in the combine
// kernel's order (fma of weight and output, slot by slot from zero).
struct DownCombine {
  const uint8_t* images;
  int64_t expert_bytes;
  size_t scale_off;
  int n_images;
  int64_t n;  // hidden: output rows, a multiple of 16
  int kbp;
  PartPlan pl;
  const float* gu;  // [m][2 ffn]: gate values, then up values
  int64_t ffn;
  const int32_t* expert;
  const float* weight;
  int rows, slots;
  int tasks;  // ceil(m / NA) * S
  int waves;  // of the workgroup: the tasks', or more for the staging
  int qpt;    // staging quarters per thread (1 or 2)
  float* y;
};

constexpr int MDC_LA = 8;          // blocks in flight per lane
constexpr int MDC_MAX_WAVES = 12;  // one wave task per wave; three waves a SIMD (170 registers)
// output rows a workgroup: half an image tile at one row (twice the
// workgroups over the CUs; at two rows each would stage twice the SwiGLU
// values for as many weights), the whole tile at two
__host__ __device__ constexpr int mdc_lgrt(int rows) { return rows == 1 ? 3 : 4; }

template <int LG>  // rows per workgroup: 1 << LG (8 or 16) of an image tile
__global__ __launch_bounds__(MDC_MAX_WAVES * WAVE) void moe_down_combine_kernel(DownCombine a) {
  constexpr int RT = 1 << LG;
  extern __shared__ __align__(16) uint8_t lds[];
  const int m = a.rows * a.slots, kbp = a.kbp;
  const PartPlan& pl = a.pl;
  uint8_t* xq = lds;                                                  // [m][kbp] x 32 codes
  float* xd = reinterpret_cast<float*>(lds + (size_t)m * kbp * 32);  // [m][kbp] scales
  float* red = xd + (size_t)m * kbp;                                  // [m][RT][S] wave-part sums
  const int nt = (int)blockDim.x, tid = (int)threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & (WAVE - 1);
  const int lg_rpw = 6 - pl.lgH, na = 1 << (lg_rpw - LG);
  const int h = lane >> lg_rpw, j = (lane >> LG) & (na - 1), i = lane & (RT - 1);
  const int s = wave & (pl.S - 1), ag = wave >> pl.lgS;
  const int aa = ag * na + j;
  const bool on = wave < a.tasks && aa < m;
  // the lane's expert (the plan's), then the staging's gate/up values, then the weights
  int e = a.expert[on ? aa : 0];
  const int nq = m * kbp * 4;  // staging quarters: (assignment, block, quarter)
  const int64_t nblk = a.ffn / QK;
  // quarter t's eight gate and eight up values (zeros past the rows' blocks):
  // four 16-byte loads, always issued (a quarter past the rows reads row 0's),
  // so the expert's load before them is waited for alone
  auto gu_load = [&](int t, float (&gv)[8], float (&uv)[8]) {
    const int blk = t >> 2, q = t & 3, ai = blk / kbp, b = blk - ai * kbp;
    const bool ld = t < nq && b < nblk;
    const float* g = a.gu + ((int64_t)(ld ? ai : 0) * 2 * a.ffn + (int64_t)(ld ? b : 0) * QK + q * 8);
    const float4 g0 = *reinterpret_cast<const float4*>(g), g1 = *reinterpret_cast<const float4*>(g + 4);
    const float4 u0 = *reinterpret_cast<const float4*>(g + a.ffn), u1 = *reinterpret_cast<const float4*>(g + a.ffn + 4);
    const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const float uu[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
    for (int v = 0; v < 8; v++) {
      gv[v] = ld ? gg[v] : 0.0f;
      uv[v] = ld ? uu[v] : 0.0f;
    }
  };
  // SwiGLU, then the q8 block (four lanes a block, as the SwiGLU kernel)
  auto stage = [&](int t, const float (&gv)[8], const float (&uv)[8]) {
    float v[8];
#pragma unroll
    for (int x = 0; x < 8; x++) v[x] = gv[x] / (1.0f + expf(-gv[x])) * uv[x];
    unsigned lo, hi;
    float d;
    int sum;
    quantize_quarter(v, lo, hi, d, sum);  // whole quads: nt is a multiple of 64
    if (t < nq) {
      *reinterpret_cast<uint2*>(xq + (size_t)(t >> 2) * 32 + (t & 3) * 8) = make_uint2(lo, hi);
      if ((t & 3) == 0) xd[t >> 2] = d;
    }
  };
  float gv[8], uv[8], gv2[8], uv2[8];
  gu_load(tid, gv, uv);
  gu_load(tid + nt, gv2, uv2);  // a second round's (two rows), always loaded: no branch around loads
  const bool ev = (unsigned)e < (unsigned)a.n_images;  // a plan entry out of range adds nothing
  e = ev ? e : 0;
  const int64_t row0 = (int64_t)blockIdx.x * RT;
  const uint8_t* img = a.images + (size_t)e * (size_t)a.expert_bytes;
  const size_t c0 = (size_t)(row0 >> 4) * (size_t)kbp;  // the tile's first cell
  const uint8_t* tcode = img + c0 * 512;
  const uint16_t* tscale = reinterpret_cast<const uint16_t*>(img + a.scale_off) + c0 * TILE;
  const int ti = (int)(row0 & 15) + i;  // the lane's row in the image tile
  const uint32_t woff = (uint32_t)ti * 16u, soff = (uint32_t)ti;
  const int bpart = s * pl.H * pl.BS + h;
  const bool task = wave < a.tasks;  // uniform: waves past the tasks only stage
  WBlock<FMT_Q8> w[MDC_LA];
  if (task) {
#pragma unroll
    for (int u = 0; u < MDC_LA; u++)
      if (u < pl.BS) w[u] = load_block<FMT_Q8>(tcode, woff, tscale, soff, bpart + pl.H * u);
  }
  // (the quarters' values were loaded before the weights)
  stage(tid, gv, uv);
  if (a.qpt > 1) stage(tid + nt, gv2, uv2);
  __syncthreads();
  float acc = 0.0f;
  const int ac = on ? aa : 0;
  const uint8_t* xa = xq + (size_t)ac * kbp * 32;
  const float* da = xd + (size_t)ac * kbp;
  for (int u = 0; task && u < pl.BS; u += MDC_LA) {
#pragma unroll
    for (int v = 0; v < MDC_LA; v++) {
      if (u + v < pl.BS) {
        const int b = bpart + pl.H * (u + v);
        const uint4 xl = ld16(xa + (size_t)b * 32), xh = ld16(xa + (size_t)b * 32 + 16);
        const int isum = dot_q8(w[v].lo, w[v].hi, xl, xh);
        acc = __builtin_fmaf((float)isum, h2f(w[v].sc) * da[b], acc);
        if (u + v + MDC_LA < pl.BS) w[v] = load_block<FMT_Q8>(tcode, woff, tscale, soff, b + pl.H * MDC_LA);
      }
    }
  }
  // lane parts: ((h0 + h1) + (h2 + h3)); then the wave parts through LDS
  for (int off = 1 << lg_rpw; off < WAVE; off <<= 1) acc += __shfl_xor(acc, off);
  if (on && h == 0) red[((size_t)aa * RT + i) * pl.S + s] = ev ? acc : 0.0f;
  __syncthreads();
  if (tid < a.rows * RT) {
    const int r = tid >> LG, ri = tid & (RT - 1);
    float y = 0.0f;
    for (int sl = 0; sl < a.slots; sl++) {
      const int as = r * a.slots + sl;
      const float* rp = red + ((size_t)as * RT + ri) * pl.S;
      float v = rp[0];
      for (int s2 = 1; s2 < pl.S; s2++) v += rp[s2];
      y = __builtin_fmaf(a.weight[as], v, y);
    }
    a.y[(int64_t)r * a.n + row0 + ri] = y;
  }
}

// Whether the one-launch down projection and combine takes this step, and its
// launch shape.
static bool down_combine_shape(int rows, int slots, int64_t hidden, int64_t ffn, DownCombine& dc, size_t& lds) {
  if (rows < 1 || rows > 2 || hidden % TILE) return false;
  const int rt = 1 << mdc_lgrt(rows);
  const int kbp = (int)kbp_of(ffn);
  const PartPlan pl = part_plan(kbp);
  if (pl.H > 4) return false;  // rows of a wave part (64 / H) at least 16
  const int m = rows * slots, na = (WAVE / pl.H) / rt;
  const int tasks = (m + na - 1) / na * pl.S;
  const int quads = (m * kbp * 4 + WAVE - 1) / WAVE;  // staging waves at one quarter a thread
  const int waves = tasks > (quads + 1) / 2 ? tasks : (quads + 1) / 2;
  if (waves > MDC_MAX_WAVES) return false;
  lds = (size_t)m * kbp * 36 + (size_t)m * rt * pl.S * 4;
  if (lds > 64 * 1024) return false;
  dc.n = hidden;
  dc.kbp = kbp;
  dc.pl = pl;
  dc.ffn = ffn;
  dc.rows = rows;
  dc.slots = slots;
  dc.tasks = tasks;
  dc.waves = waves;
  dc.qpt = waves * WAVE >= m * kbp * 4 ? 1 : 2;
  return true;
}

bool moe_down_combine_fits(int rows, int slots, int64_t hidden, int64_t ffn) {
  DownCombine dc;
  size_t lds = 0;
  return down_combine_shape(rows, slots, hidden, ffn, dc, lds);
}

int launch_moe_down_combine(const void* images, int n_images, int64_t hidden, int64_t ffn, const float* gu,
                            const int32_t* expert, const float* weight, int rows, int slots, float* y,
                            hipStream_t s) {
  DownCombine dc;
  size_t lds = 0;
  if (!down_combine_shape(rows, slots, hidden, ffn, dc, lds))
    return fail(QG_ELAUNCH, "no one-launch down projection for rows=%d slots=%d ffn=%lld", rows, slots,
                (long long)ffn);
  dc.images = (const uint8_t*)images;
  dc.expert_bytes = (int64_t)image_total_bytes(QG_FMT_Q8_0, hidden, ffn);
  dc.scale_off = image_scale_offset(QG_FMT_Q8_0, hidden, ffn);
  dc.n_images = n_images;
  dc.gu = gu;
  dc.expert = expert;
  dc.weight = weight;
  dc.y = y;
  const int lg = mdc_lgrt(rows);
  auto kern = lg == 3 ? moe_down_combine_kernel<3> : moe_down_combine_kernel<4>;
  if (lds > 48 * 1024)
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL(kern, dim3((unsigned)(hidden >> lg)), dim3(dc.waves * WAVE), lds, s, dc);
  return hip_status(hipGetLastError(), "moe_down_combine_kernel");
}

// ------------------------------------------------------ pair-dot hook ---

// Test hook: the int32 dots of every (activation row, weight row, block) as the
// pair kernel forms them -- the same weight and chunk operands, the same
// matrix product (pair_dots) -- written out instead of scaled and summed.
// One wave per (16-row tile, block pair, group of eight activation rows) of a
// pair-order workspace; isum [rows][n][kb].
template <int FMT>
__global__ __launch_bounds__(256) void pair_blockdots_kernel(const uint8_t* __restrict__ code, int64_t n, int kbp,
                                                             int kb, Prep prep, int groups, int rows,
                                                             int* __restrict__ isum) {
  constexpr int CB = FMT == FMT_Q8 ? 512 : 256;
  const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  const int64_t pairs = kbp / 2, ntiles = np_of(n) / TILE;
  if (wave >= ntiles * pairs * groups) return;  // whole waves leave together
  const int lane = threadIdx.x & (WAVE - 1), i = lane & 15, q = lane >> 4;
  const int g = (int)(wave % groups), p = (int)((wave / groups) % pairs);
  const int64_t t = wave / (groups * pairs);
  const uint4 a = ld16(code + ((size_t)t * kbp + 2 * p) * CB + pair_aoff<FMT>(i, q));
  const size_t chunk = (size_t)p * groups + g;
  const bool xon = (i < 8) == (q < 2);
  const uint4 x = xon ? ld16(reinterpret_cast<const uint8_t*>(prep.codes) + (chunk * 64 + lane) * 16)
                      : make_uint4(0u, 0u, 0u, 0u);
  const v4i c = pair_dots<FMT>(a, x, 0, (q & 1) * 4);  // Q4_0: sixteen times the dots
  const int r = g * 8 + (i & 7), b = 2 * p + (i >> 3);
  if (r >= rows || b >= kb) return;
#pragma unroll
  for (int v = 0; v < 4; v++) {
    const int64_t o = t * TILE + 4 * q + v;
    if (o < n) isum[((int64_t)r * n + o) * kb + b] = FMT == FMT_Q4 ? c[v] >> 4 : c[v];
  }
}

int launch_pair_blockdots(int fmt, const void* image, int64_t n, int64_t k, const void* ws, int rows, int32_t* isum,
                          hipStream_t s) {
  const PrepLayout L = prep_layout(rows, k);
  const Prep pv = prep_view(ws, L);
  const int kbp = (int)kbp_of(k), kb = (int)kb_of(k);
  const int64_t waves = (np_of(n) / TILE) * (kbp / 2) * L.groups;
  const unsigned g = (unsigned)((waves * WAVE + 255) / 256);
  if (fmt == QG_FMT_Q8_0)
    hipLaunchKernelGGL(pair_blockdots_kernel<FMT_Q8>, dim3(g), dim3(256), 0, s, (const uint8_t*)image, n, kbp, kb, pv,
                       L.groups, rows, isum);
  else if (fmt == QG_FMT_Q4_K)
    hipLaunchKernelGGL(pair_blockdots_kernel<FMT_Q4K>, dim3(g), dim3(256), 0, s, (const uint8_t*)image, n, kbp, kb,
                       pv, L.groups, rows, isum);
  else
    hipLaunchKernelGGL(pair_blockdots_kernel<FMT_Q4>, dim3(g), dim3(256), 0, s, (const uint8_t*)image, n, kbp, kb, pv,
                       L.groups, rows, isum);
  return hip_status(hipGetLastError(), "pair_blockdots_kernel");
}

// ------------------------------------------------------------- launchers ---

int device_cus() {
  static int cus = 0;
  if (!cus) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      cus = v;
    else
      cus = 256;
  }
  return cus;
}

// Workgroups to launch: no more than the device holds at once (the kernels
// loop over the remaining tiles) and no more than there are tiles.
template <typename K>
static unsigned persistent_grid(K kernel, size_t lds, int64_t tiles) {
  // a failure here makes the launch itself fail, which its caller reports
  if (lds > 48 * 1024)
    (void)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, WG, lds) != hipSuccess || per_cu < 1) per_cu = 1;
  const int64_t g = (int64_t)device_cus() * per_cu;
  return (unsigned)(tiles < g ? tiles : g);
}

bool fuses_quantization(int fmt, int rows, int64_t k) {
  return rows >= 1 && rows <= FUSE_MAX_ROWS && (size_t)rows * kbp_of(k) * x_block_bytes(fmt) <= (size_t)LDS_X_RL;
}

template <int FMT, int R, bool FUSED>
static void launch_rl(const SetArgs& a, int lds_x, hipStream_t s) {
  const size_t lds = (size_t)lds_x + 2 * WAVES * WAVE * R * 4;
  bool whole = true;  // every projection staged whole (LA need not divide a staging round)
  for (int i = 0; i < a.count; i++) whole = whole && a.p[i].ucx == a.p[i].pl.BS;
  // A lane's whole chain in flight, one workgroup per CU: for launches of at
  // most one tile per CU, and for one row over four or more tiles per CU (one
  // row of 128256 x 4096: 87 -> 85 us, of 65536 x 4096: 46.7 -> 45.0; equal at
  // two tiles per CU; at two rows slower at every size).
  const bool small = whole && (a.total_tiles <= device_cus() || (R == 1 && a.total_tiles >= 4 * device_cus()));
  if (small) {
    // Q4_K holds each block's 16-byte superblock header too: six blocks in flight keep it within the
    // registers of two workgroups per CU, where eight would leave one
    auto kern = rl_set_kernel<FMT, R, FUSED, FMT == FMT_Q4K ? 6 : 8>;
    hipLaunchKernelGGL(kern, dim3(persistent_grid(kern, lds, a.total_tiles)), dim3(WG), lds, s, a, lds_x);
  } else {
    auto kern = rl_set_kernel<FMT, R, FUSED, 2>;
    hipLaunchKernelGGL(kern, dim3(persistent_grid(kern, lds, a.total_tiles)), dim3(WG), lds, s, a, lds_x);
  }
}

template <int FMT>
static void launch_rl_rows(const SetArgs& a, int rows, bool fused, int lds_x, hipStream_t s) {
  if (fused) {
    if (rows == 1) launch_rl<FMT, 1, true>(a, lds_x, s);
    else launch_rl<FMT, 2, true>(a, lds_x, s);
    return;
  }
  if (rows == 1) launch_rl<FMT, 1, false>(a, lds_x, s);
  else launch_rl<FMT, 2, false>(a, lds_x, s);
}

// Tiles of the pair kernel at width `wide`; returns the LDS bytes it needs:
// the combine area (MP_NV_MAX floats per lane), then each wave's staged
// scales (NT tiles of kbp/S blocks x 16 fp16); Q4_K (a 6-bit (sc, m) pair per
// row and block, fp32 (d, dmin) per row and superblock) one region per wave
// for either, whichever is larger.
static size_t mp_fill(SetArgs& a, int G, int width, int fmt) {
  int64_t tiles = 0;
  size_t sc = 0;
  for (int i = 0; i < a.count; i++) {
    ProjDev& d = a.p[i];
    if (width != MP_MIXED) d.wide = width == MP_WIDE;
    const int nt = mp_nt(d.pl.H, G, d.wide != 0, fmt);
    d.rows_per_tile = (WAVES / (d.pl.S * mp_w2(d.pl.H))) * TILE * nt;
    d.tiles = (int)((d.n + d.rows_per_tile - 1) / d.rows_per_tile);
    tiles += d.tiles;
    // fp16 per (row, block); Q4_K a (sc, m) pair per (row, block) and fp32 (d, dmin) per (row, superblock)
    const size_t hbs = (size_t)(d.kbp / d.pl.S);
    const size_t v = (size_t)nt * (hbs * TILE * 2 + (fmt == FMT_Q4K ? (hbs / 8 + 2) * TILE * 8 : 0));
    sc = v > sc ? v : sc;
  }
  a.total_tiles = (int)tiles;
  const size_t red = (size_t)MP_NV_MAX * WAVE * 4;
  if (fmt != FMT_Q4K) {
    a.wave_lds = 0;
    return WAVES * red + WAVES * sc;
  }
  const size_t region = ((sc > red ? sc : red) + 15) / 16 * 16;
  a.wave_lds = (int)region;
  return (size_t)WAVES * region;
}

// Weight bytes one wave of projection d streams per tile group on wide tiles.
static int64_t mp_wide_wave_bytes(const ProjDev& d, int fmt, int G) {
  return (int64_t)mp_nt(d.pl.H, G, true, fmt) * (d.kbp / (d.pl.S * mp_w2(d.pl.H))) * (fmt == FMT_Q8 ? 512 : 256);
}

// The pair kernel runs in rounds of the workgroups resident at once; a round
// costs about a tile's latency chain.  At 9-16 rows every projection takes
// wide tiles when that needs fewer rounds (half the activation-chunk loads).
// At 3-8 rows, when narrow tiles overflow one round, projections move to
// wide tiles one at a time, those whose waves then stream the least first,
// until the launch fits one round (a wave's stream is the latency chain that
// ends the launch).  Narrow Q8_0 tiles over several rounds take the kernel
// that prefetches across a workgroup's tiles.
template <int FMT, int G>
static void launch_mp(SetArgs a, int rows, hipStream_t s) {
  auto kn = mp_set_kernel<FMT, G, MP_NARROW, false>;
  auto kw = mp_set_kernel<FMT, G, MP_WIDE, false>;
  SetArgs aw = a;
  const size_t ln = mp_fill(a, G, MP_NARROW, FMT), lw = mp_fill(aw, G, MP_WIDE, FMT);
  const unsigned gn = persistent_grid(kn, ln, a.total_tiles), gw = persistent_grid(kw, lw, aw.total_tiles);
  const int64_t rn = (a.total_tiles + gn - 1) / gn, rw = (aw.total_tiles + gw - 1) / gw;
  if (G == 2 && rw < rn) {
    hipLaunchKernelGGL(kw, dim3(gw), dim3(WG), lw, s, aw, rows);
    return;
  }
  if constexpr (G == 1) {
    // Widen projections, those whose waves then stream the least first,
    // until the launch fits one round of resident workgroups.
    auto km = mp_set_kernel<FMT, G, MP_MIXED, false>;
    SetArgs am = a;
    int order[QG_MAX_SET];
    for (int i = 0; i < am.count; i++) order[i] = i;
    for (int i = 1; i < am.count; i++)
      for (int j = i; j > 0 && mp_wide_wave_bytes(am.p[order[j]], FMT, G) <
                                   mp_wide_wave_bytes(am.p[order[j - 1]], FMT, G); j--) {
        const int t = order[j];
        order[j] = order[j - 1];
        order[j - 1] = t;
      }
    for (int i = 0; i < am.count && rn > 1; i++) {
      am.p[order[i]].wide = 1;
      const size_t lm = mp_fill(am, G, MP_MIXED, FMT);
      const unsigned gm = persistent_grid(km, lm, am.total_tiles);
      if (am.total_tiles <= (int64_t)gm) {
        hipLaunchKernelGGL(km, dim3(gm), dim3(WG), lm, s, am, rows);
        return;
      }
    }
  }
  if constexpr (FMT == FMT_Q8) {
    if (rn > 1) {
      auto kp = mp_set_kernel<FMT, G, MP_NARROW, true>;  // the occupancy of kn (128 registers at most)
      if (ln > 48 * 1024)
        (void)hipFuncSetAttribute((const void*)kp, hipFuncAttributeMaxDynamicSharedMemorySize, (int)ln);
      hipLaunchKernelGGL(kp, dim3(gn), dim3(WG), ln, s, a, rows);
      return;
    }
  }
  hipLaunchKernelGGL(kn, dim3(gn), dim3(WG), ln, s, a, rows);
}

// Launch order of a set's projections on the 1-2-row kernel: longer lane
// chains (blocks per lane part) first, then longer rows.
static bool rl_before(int64_t ka, int64_t kb) {
  const int ba = part_plan((int)kbp_of(ka)).BS, bb = part_plan((int)kbp_of(kb)).BS;
  return ba != bb ? ba > bb : ka > kb;
}

int launch_qgemv_set(int fmt, const ProjArg* projs, int count, int rows, hipStream_t s) {
  SetArgs a;
  memset(&a, 0, sizeof a);
  a.count = count;
  const bool mf = prep_pairs(rows);  // 3..16 rows: the pair kernel
  // Tiles of projections with longer rows come first: their workgroups stage
  // the most activation blocks, so they get the earliest start; on the
  // 1-2-row kernel those whose lanes walk more blocks come before them (the
  // longest chains start first).  The order changes no result (each
  // projection has its own output).
  int order[QG_MAX_SET];
  for (int i = 0; i < count; i++) order[i] = i;
  auto before = [&](int64_t ka, int64_t kb) { return mf ? ka > kb : rl_before(ka, kb); };
  for (int i = 1; i < count; i++)
    for (int j = i; j > 0 && before(projs[order[j]].k, projs[order[j - 1]].k); j--) {
      const int t = order[j];
      order[j] = order[j - 1];
      order[j - 1] = t;
    }
  bool fused = true;
  int64_t tiles = 0;
  size_t need = 0;
  for (int i = 0; i < count; i++) {
    const ProjArg& pa = projs[order[i]];
    ProjDev& d = a.p[i];
    const uint8_t* img = (const uint8_t*)pa.image;
    d.code = img;
    d.scale = (const uint16_t*)(img + image_scale_offset(fmt, pa.n, pa.k));
    d.prep = pa.ws ? prep_view(pa.ws, prep_layout(rows, pa.k)) : Prep{nullptr, nullptr, nullptr};
    d.xf = pa.x;
    d.y = pa.y;
    d.n = pa.n;
    d.k = pa.k;
    d.kb = (int)kb_of(pa.k);
    d.kbp = (int)kbp_of(pa.k);
    const PartPlan pl = part_plan(d.kbp);
    d.pl = pl;
    d.rows_per_tile = WG / pl.P;  // RL tiles; the pair kernel sets its own
    d.tiles = (int)((pa.n + d.rows_per_tile - 1) / d.rows_per_tile);
    tiles += d.tiles;
    const size_t x = (size_t)rows * d.kbp * x_block_bytes(fmt);
    need = x > need ? x : need;
    fused = fused && pa.x != nullptr;
  }
  a.total_tiles = (int)tiles;
  const size_t cap = LDS_X_RL;
  fused = fused && !mf && need <= cap;  // the fused path stages every row whole
  const int lds_x = (int)((need < cap ? need : cap) + 15) / 16 * 16;
  for (int i = 0; i < count; i++) a.p[i].ucx = rl_round(lds_x, rows, a.p[i].pl, fmt);
  if (mf) {
    if (rows <= 8) {
      if (fmt == FMT_Q8) launch_mp<FMT_Q8, 1>(a, rows, s);
      else if (fmt == FMT_Q4K) launch_mp<FMT_Q4K, 1>(a, rows, s);
      else launch_mp<FMT_Q4, 1>(a, rows, s);
    } else {
      if (fmt == FMT_Q8) launch_mp<FMT_Q8, 2>(a, rows, s);
      else if (fmt == FMT_Q4K) launch_mp<FMT_Q4K, 2>(a, rows, s);
      else launch_mp<FMT_Q4, 2>(a, rows, s);
    }
  } else {
    if (fmt == FMT_Q8) launch_rl_rows<FMT_Q8>(a, rows, fused, lds_x, s);
    else if (fmt == FMT_Q4K) launch_rl_rows<FMT_Q4K>(a, rows, fused, lds_x, s);
    else launch_rl_rows<FMT_Q4>(a, rows, fused, lds_x, s);
  }
  return hip_status(hipGetLastError(), mf ? "mp_set_kernel" : "rl_set_kernel");
}

bool grouped_glu_fits(int64_t k) {
  return (size_t)GROUPED_SMALL_ROWS * kbp_of(k) * x_block_bytes(FMT_Q8) <= (size_t)LDS_X_RL;
}

int launch_grouped_planned(const void* images, int64_t n_experts, int64_t n, int64_t k, const void* prep, int x_rows,
                           const int* header, const int* sorted, const int* items, const int32_t* x_index, int m,
                           int max_item_rows, float* y, hipStream_t s, const float* glu) {
  (void)n_experts;
  if (m == 0) return QG_OK;
  const int kbp = (int)kbp_of(k);
  const PartPlan pl = part_plan(kbp);
  const int rpt = WG / pl.P;
  const int tiles = (int)((n + rpt - 1) / rpt);
  const int64_t eb = (int64_t)image_total_bytes(QG_FMT_Q8_0, n, k);
  const size_t so = image_scale_offset(QG_FMT_Q8_0, n, k);
  const Prep pv = prep_view(prep, prep_layout_rows(x_rows, k));
  // LDS of a class: its largest row count staged (up to the RL cap), then the combine area
  auto lds_x_for = [&](int rows) {
    const size_t need = (size_t)rows * kbp * x_block_bytes(FMT_Q8);
    return (int)((need < (size_t)LDS_X_RL ? need : (size_t)LDS_X_RL) + 15) / 16 * 16;
  };
  // small items: at most m of them; items of more rows: at most m / (GROUPED_SMALL_ROWS + 1)
  const int lx_s = lds_x_for(GROUPED_SMALL_ROWS);
  const size_t lds_s = (size_t)lx_s + WAVES * WAVE * GROUPED_SMALL_ROWS * 4;
  const int mb = max_item_rows > GROUPED_SMALL_ROWS ? m / (GROUPED_SMALL_ROWS + 1) : 0;
  if (glu && (mb > 0 || !grouped_glu_fits(k)))
    return fail(QG_ELAUNCH, "SwiGLU rows need items of at most two rows and k=%lld staged whole", (long long)k);
  if (mb == 0) {
    // at most m items, so at most m * tiles units
    const bool few = (int64_t)m * tiles <= device_cus();
    auto kern = glu ? (few ? grouped_kernel<true, GROUPED_LA_FEW> : grouped_kernel<true, GROUPED_LA>)
                    : (few ? grouped_kernel<false, GROUPED_LA_FEW> : grouped_kernel<false, GROUPED_LA>);
    const unsigned gs = persistent_grid(kern, lds_s, (int64_t)m * tiles);
    hipLaunchKernelGGL(kern, dim3(gs), dim3(WG), lds_s, s, (const uint8_t*)images, eb, so, n, k, kbp, pl, pv, header,
                       sorted, items, x_index, y, lx_s, tiles, glu);
    return hip_status(hipGetLastError(), "grouped_kernel");
  }
  // items of more than two rows possible: one launch for both kinds of unit
  const int tb = (int)((n + grouped_mp_rows(pl) - 1) / grouped_mp_rows(pl));
  const size_t lds_b = (size_t)WAVES * WAVE * MP_NV_MAX * 4 + (size_t)WAVES * (kbp / pl.S) * TILE * 2;
  const size_t lds_a = lds_s > lds_b ? lds_s : lds_b;
  const unsigned ga = persistent_grid(grouped_all_kernel, lds_a, (int64_t)m * tiles + (int64_t)mb * tb);
  hipLaunchKernelGGL(grouped_all_kernel, dim3(ga), dim3(WG), lds_a, s, (const uint8_t*)images, eb, so, n, k, kbp, pl,
                     pv, header, sorted, items, x_index, y, lx_s, tiles, tb);
  if (int st = hip_status(hipGetLastError(), "grouped_all_kernel")) return st;
  return QG_OK;
}

int launch_moe_up(const void* images, int64_t n, int64_t k, const void* prep, const MoeUp& up_in, float* y,
                  hipStream_t s) {
  MoeUp up = up_in;
  const int slots = up.topk + up.shared, m = up.rows * slots;
  const int kbp = (int)kbp_of(k);
  const PartPlan pl = part_plan(kbp);
  const int tiles = (int)((n + WG / pl.P - 1) / (WG / pl.P));
  const int64_t eb = (int64_t)image_total_bytes(QG_FMT_Q8_0, n, k);
  const size_t so = image_scale_offset(QG_FMT_Q8_0, n, k);
  const Prep pv = prep_view(prep, prep_layout_rows(up.rows, k));
  const size_t need = (size_t)GROUPED_SMALL_ROWS * kbp * x_block_bytes(FMT_Q8);
  const int lx_s = (int)((need < (size_t)LDS_X_RL ? need : (size_t)LDS_X_RL) + 15) / 16 * 16;
  const size_t lds_s = (size_t)lx_s + WAVES * WAVE * GROUPED_SMALL_ROWS * 4;
  const size_t plan = plan_lds_bytes(m, up.E);
  if (up.rows <= GROUPED_SMALL_ROWS) {
    // every item is small: at most m of them, m * tiles units
    up.plan_off = (int)((lds_s + 15) / 16 * 16);
    const size_t lds = (size_t)up.plan_off + plan;
    const bool few = (int64_t)m * tiles <= device_cus();
    auto kern = few ? moe_up_small_kernel<GROUPED_LA_FEW> : moe_up_small_kernel<GROUPED_LA>;
    const unsigned g = persistent_grid(kern, lds, (int64_t)m * tiles);
    hipLaunchKernelGGL(kern, dim3(g), dim3(WG), lds, s, (const uint8_t*)images, eb, so, n, k, kbp, pl, pv, y, lx_s,
                       tiles, up);
    return hip_status(hipGetLastError(), "moe_up_small_kernel");
  }
  const int tb = (int)((n + grouped_mp_rows(pl) - 1) / grouped_mp_rows(pl));
  const size_t lds_b = (size_t)WAVES * WAVE * MP_NV_MAX * 4 + (size_t)WAVES * (kbp / pl.S) * TILE * 2;
  const size_t lds_a = lds_s > lds_b ? lds_s : lds_b;
  up.plan_off = (int)((lds_a + 15) / 16 * 16);
  const size_t lds = (size_t)up.plan_off + plan;
  const int mb = m / (GROUPED_SMALL_ROWS + 1);  // items of more than two rows: at most this many
  const unsigned g = persistent_grid(moe_up_all_kernel, lds, (int64_t)m * tiles + (int64_t)mb * tb);
  hipLaunchKernelGGL(moe_up_all_kernel, dim3(g), dim3(WG), lds, s, (const uint8_t*)images, eb, so, n, k, kbp, pl, pv,
                     y, lx_s, tiles, tb, up);
  return hip_status(hipGetLastError(), "moe_up_all_kernel");
}

int launch_grouped_plan(const int32_t* expert, const int32_t* x_index, int m, int64_t n_experts, int x_rows,
                        int* header, int* sorted, int* items, hipStream_t s, const float* x, int64_t k, void* xprep,
                        bool fp8) {
  // x null: the plan only (one workgroup); else the input rows' A1 (or, fp8,
  // their FP8 groups into the FP8 workspace) on workgroups 1..
  const int64_t quads = x ? (fp8 ? (int64_t)x_rows * (k / 128) * WAVE : (int64_t)x_rows * kbp_of(k) * 4) : 0;
  int8_t* xq = nullptr;
  float* xd = nullptr;
  int* xn = nullptr;
  uint8_t* fc = nullptr;
  float* fs = nullptr;
  if (x && fp8) {
    fc = (uint8_t*)xprep;
    fs = (float*)(fc + fp8_ws_scale_offset(x_rows, k));
  } else if (x) {
    const PrepLayout L = prep_layout_rows(x_rows, k);
    uint8_t* w = (uint8_t*)xprep;
    xq = (int8_t*)(w + L.codes);
    xd = (float*)(w + L.dx);
    xn = (int*)(w + L.nsx);
  }
  hipLaunchKernelGGL(grouped_plan_kernel, dim3(1 + (unsigned)((quads + 1023) / 1024)), dim3(1024), 0, s, expert,
                     x_index, m, n_experts, x_rows, header, sorted, items, x, k, xq, xd, xn, fc, fs);
  return hip_status(hipGetLastError(), "grouped_plan_kernel");
}

int launch_grouped(const void* images, int64_t n_experts, int64_t n, int64_t k, const float* x, int x_rows,
                   const int32_t* expert, const int32_t* x_index, int m, float* y, void* ws, hipStream_t s) {
  const GroupedLayout G = grouped_layout(x_rows, k, m);
  uint8_t* w = (uint8_t*)ws;
  int* header = (int*)(w + G.header);
  int* sorted = (int*)(w + G.sorted);
  int* items = (int*)(w + G.items);
  if (int st = launch_grouped_plan(expert, x_index, m, n_experts, x_rows, header, sorted, items, s, x, k, w + G.prep,
                                   false))
    return st;
  return launch_grouped_planned(images, n_experts, n, k, w + G.prep, x_rows, header, sorted, items, x_index, m,
                                QG_MAX_ROWS, y, s);
}

}  // namespace qg
