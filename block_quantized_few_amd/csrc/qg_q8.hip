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
//   * RL ("lanes own rows", 1..8 rows and the grouped path): a lane owns one
//     weight row and streams its blocks with 16-byte loads; the integer dot of
//     each block is exact inside the lane (v_dot4_i32_i8); activation blocks
//     are read from LDS by the whole lane group at once (broadcast).
//   * MF (9..16 rows): a wave owns 16 weight rows; one v_mfma_i32_16x16x32_i8
//     per block gives the exact block dots of 16 weight rows x 16 activation
//     rows, which the lanes then scale and accumulate in fp32.
// Both accumulate, per row and activation row, acc = fma(isum, dw * dx, acc)
// over the blocks of each part in the partition's order, then add lane parts
// by a fixed tree and wave parts left to right.
#include <hip/hip_runtime.h>
#include <string.h>

#include "qg_device.h"
#include "qg_internal.h"
#include "qg_launch.h"

namespace qg {

constexpr int WG = 512;
constexpr int WAVES = WG / WAVE;
constexpr int LDS_X_RL = 80 * 1024;   // staged rows, RL (leaves room for 2+ workgroups per CU)
constexpr int FUSE_MAX_ROWS = 2;      // rows quantized inside the GEMV launch

__host__ __device__ inline int x_block_bytes(int fmt) { return fmt == FMT_Q4 ? 40 : 36; }

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
      if (FMT == FMT_Q4) ln[r * nslot + e] = prep.nsx[src + b];
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
constexpr int XQ_FIRST = 2;  // work items per thread whose loads are issued first

struct XQuarter {
  float4 a, c;
};

// Work item e of R <= 2 rows: row r = e / (4 * nslot), without a division.
__device__ __forceinline__ int xq_row(int e, int nslot) { return e >= 4 * nslot ? 1 : 0; }

__device__ __forceinline__ XQuarter xq_load(const float* __restrict__ x, int64_t k, int kb, int nslot,
                                            const PartPlan& pl, int e, int total) {
  const int q = e & 3, blk = e >> 2;
  const int r = xq_row(e, nslot), slot = blk - r * nslot;
  const int b = slot_block(pl, 0, slot);
  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
  XQuarter v;
  v.a = z;
  v.c = z;
  if (e < total) {  // uniform over a wave: total is a multiple of 64
    // pad blocks read the row's first quarter and use zeros
    const bool ok = b < kb;
    const float4* src = reinterpret_cast<const float4*>(x + (ok ? (int64_t)r * k + (int64_t)b * QK + q * 8 : 0));
    const float4 a = src[0], c = src[1];
    v.a = ok ? a : z;
    v.c = ok ? c : z;
  }
  return v;
}

template <int FMT>
__device__ __forceinline__ void xq_store(const XQuarter& xv, uint8_t* lds, int R, int nslot, int e, int total) {
  if (e >= total) return;  // whole quads leave together: total and the stride are multiples of 4
  const int q = e & 3, blk = e >> 2;
  const int r = xq_row(e, nslot), slot = blk - r * nslot;
  const float v[8] = {xv.a.x, xv.a.y, xv.a.z, xv.a.w, xv.c.x, xv.c.y, xv.c.z, xv.c.w};
  unsigned lo, hi;
  float d;
  int sum;
  quantize_quarter(v, lo, hi, d, sum);
  *reinterpret_cast<uint2*>(lds + ((size_t)r * nslot + slot) * 32 + q * 8) = make_uint2(lo, hi);
  if (q == 0) {
    reinterpret_cast<float*>(lds + (size_t)R * nslot * 32)[r * nslot + slot] = d;
    if (FMT == FMT_Q4) reinterpret_cast<int*>(lds + (size_t)R * nslot * 36)[r * nslot + slot] = -8 * sum;
  }
}

// First part: load this thread's first XQ_FIRST work items.
__device__ __forceinline__ void stage_quantize_begin(XQuarter (&xv)[XQ_FIRST], const float* __restrict__ x,
                                                     int64_t k, int kb, int R, int kbp, const PartPlan& pl) {
  const int total = R * kbp * 4;
#pragma unroll
  for (int j = 0; j < XQ_FIRST; j++) xv[j] = xq_load(x, k, kb, kbp, pl, threadIdx.x + j * WG, total);
}

// Second part: quantize them into LDS, then the rest of the work items.
template <int FMT>
__device__ __forceinline__ void stage_quantize_end(const XQuarter (&xv)[XQ_FIRST], uint8_t* lds,
                                                   const float* __restrict__ x, int64_t k, int kb, int R, int kbp,
                                                   const PartPlan& pl) {
  const int total = R * kbp * 4;
#pragma unroll
  for (int j = 0; j < XQ_FIRST; j++) xq_store<FMT>(xv[j], lds, R, kbp, threadIdx.x + j * WG, total);
  for (int e = threadIdx.x + XQ_FIRST * WG; e < total; e += WG) {
    xq_store<FMT>(xq_load(x, k, kb, kbp, pl, e, total), lds, R, kbp, e, total);
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
};

// Block b of the lane's row.  The address is the tile's base (uniform) plus a
// 32-bit lane offset, so the loads take the scalar-base form.
template <int FMT>
__device__ __forceinline__ WBlock<FMT> load_block(const uint8_t* __restrict__ tcode, uint32_t woff,
                                                  const uint16_t* __restrict__ tscale, uint32_t soff, int b) {
  constexpr uint32_t CB = FMT == FMT_Q8 ? 512 : 256;
  WBlock<FMT> w;
  w.lo = ld16_stream(tcode + (woff + (uint32_t)b * CB));
  if (FMT == FMT_Q8) w.hi = ld16_stream(tcode + (woff + (uint32_t)b * CB + 256));
  w.sc = ld2_stream(tscale + (soff + (uint32_t)b * TILE));
  return w;
}

// acc[r] = fma(isum, dw * dx, acc[r]) for one block, its activation blocks at
// staged slot `slot`.
template <int FMT, int R>
__device__ __forceinline__ void compute_block(float (&acc)[R], const WBlock<FMT>& w, const uint8_t* lds, int nslot,
                                              int slot) {
  const float* ld = reinterpret_cast<const float*>(lds + (size_t)R * nslot * 32);
  const int* ln = reinterpret_cast<const int*>(lds + (size_t)R * nslot * 36);
  const float dw = h2f(w.sc);
#pragma unroll
  for (int r = 0; r < R; r++) {
    const uint8_t* xb = lds + ((size_t)r * nslot + slot) * 32;
    const uint4 xl = ld16(xb), xh = ld16(xb + 16);
    const float dxr = ld[r * nslot + slot];
    const int isum = FMT == FMT_Q8 ? dot_q8(w.lo, w.hi, xl, xh) : dot_q4(w.lo, xl, xh, ln[r * nslot + slot]);
    acc[r] = __builtin_fmaf((float)isum, dw * dxr, acc[r]);
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
template <int FMT, int R, bool FUSED>
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
  const uint32_t soff = (uint32_t)((rc >> 4) - t0) * (uint32_t)ta.kbp * 16u + (uint32_t)(rc & 15);

  float acc[R];
#pragma unroll
  for (int r = 0; r < R; r++) acc[r] = 0.0f;
  const int ucx = ta.ucx;
  const bool full = ucx == pl.BS;          // every block staged at once
  const int bpart = s * pl.H * pl.BS + h;  // this lane's block at u = 0
  const int sbase = s * pl.H + h;          // its slot at u = 0 of a round

  constexpr int LA = rl_lookahead(FUSED, R);
  XQuarter xv[XQ_FIRST];
  if (FUSED && stage) stage_quantize_begin(xv, ta.xf, ta.k, ta.kb, R, ta.kbp, pl);
  WBlock<FMT> w[LA];
#pragma unroll
  for (int j = 0; j < LA; j++) w[j] = load_block<FMT>(tcode, woff, tscale, soff, bpart + pl.H * j);  // BS >= 8
  __builtin_amdgcn_sched_barrier(0);
  int u0 = 0, nslot = ucx << pl.lgP;
  int next_round = (!full || stage) ? 0 : pl.BS;  // u at which activation rows are (re)staged
  for (int u = 0; u < pl.BS; u += LA) {
    if (u == next_round) {
      u0 = u;
      nslot = min(ucx, pl.BS - u) << pl.lgP;
      next_round = full ? pl.BS : u + ucx;
      __syncthreads();
      if (FUSED) stage_quantize_end<FMT>(xv, lds, ta.xf, ta.k, ta.kb, R, ta.kbp, pl);
      else stage_rl<FMT, R>(lds, ta.prep, ta.s_src, ta.kbp, pl, u0, nslot);
      __syncthreads();
    }
    const int slot = ((u - u0) << pl.lgP) + sbase;
#pragma unroll
    for (int j = 0; j < LA; j++) {
      if (u + j < pl.BS) {
        compute_block<FMT, R>(acc, w[j], lds, nslot, slot + (j << pl.lgP));
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

// ------------------------------------------------------------- MF tile ---

// NT 16-row image tiles per wave, so that a wave keeps several independent
// MFMA accumulations in flight and reuses each activation fragment NT times.
__host__ __device__ constexpr int mf_tiles_per_wave(int H) { return H >= 4 ? 1 : 2; }

// One step of an MF wave: HC lane parts of one u for NT image tiles (two or
// four MFMAs); the wave keeps two steps in flight.
template <int FMT, int HC, int NT>
struct MfStep {
  uint2 a[NT][HC];  // A fragments: 8 codes of row i (Q4_0: 16 nibbles)
  uint2 w[NT][HC];  // fp16 scales of rows 4q .. 4q+3
  long x[HC];       // B fragments: 8 codes of activation row i
  float dx[HC];
  int ns[HC];       // Q4_0 start value -8 * sum(q_x)
};

// Where an MF wave reads: per image tile a base shared by the wave plus a lane
// offset, so every load takes the scalar-base form and the addresses cost no
// vector registers.
template <int NT>
struct MfAddr {
  const uint8_t* code[NT];    // tile's code plane (wave-uniform)
  const uint16_t* scale[NT];  // tile's scales (wave-uniform)
  uint32_t aoff;              // lane's A-fragment byte offset in a cell
  uint32_t soff;              // lane's first scale (fp16 units) in a cell
  const int8_t* xc;           // prepared codes, fragment order (uniform)
  const float* xd;
  const int* xn;
  uint32_t xoff;  // lane's B-fragment byte offset in a block's fragments
  int R;
};

template <int FMT, int HC, int NT>
__device__ __forceinline__ void mf_load(MfStep<FMT, HC, NT>& st, const MfAddr<NT>& ad, int i, int b0) {
  constexpr int CB = FMT == FMT_Q8 ? 512 : 256;
#pragma unroll
  for (int hh = 0; hh < HC; hh++) {
    const size_t b = (size_t)(b0 + hh);
#pragma unroll
    for (int t = 0; t < NT; t++) {
      st.a[t][hh] = ld8_stream(ad.code[t] + b * CB + ad.aoff);
      st.w[t][hh] = ld8_stream(ad.scale[t] + b * TILE + ad.soff);
    }
    // lanes past the R rows read row R-1 again: their MFMA columns are never stored
    st.x[hh] = *reinterpret_cast<const long*>(ad.xc + b * 32 * ad.R + ad.xoff);
    st.dx[hh] = ad.xd[b * ad.R + i];
    st.ns[hh] = FMT == FMT_Q4 ? ad.xn[b * ad.R + i] : 0;
  }
}

template <int FMT, int HC, int NT>
__device__ __forceinline__ void mf_compute(float (&acc)[NT][HC][4], const MfStep<FMT, HC, NT>& st, int sh) {
#pragma unroll
  for (int hh = 0; hh < HC; hh++)
#pragma unroll
    for (int t = 0; t < NT; t++) {
      uint2 av = st.a[t][hh];
      if (FMT == FMT_Q4) {
        av.x = (av.x >> sh) & 0x0F0F0F0Fu;
        av.y = (av.y >> sh) & 0x0F0F0F0Fu;
      }
      long a;
      __builtin_memcpy(&a, &av, 8);
      const int ns = st.ns[hh];
      v4i c = {ns, ns, ns, ns};
      c = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, st.x[hh], c, 0, 0, 0);
      const uint2 wv = st.w[t][hh];
      const float dw[4] = {h2f((uint16_t)(wv.x & 0xffff)), h2f((uint16_t)(wv.x >> 16)),
                           h2f((uint16_t)(wv.y & 0xffff)), h2f((uint16_t)(wv.y >> 16))};
#pragma unroll
      for (int v = 0; v < 4; v++) acc[t][hh][v] = __builtin_fmaf((float)c[v], dw[v] * st.dx[hh], acc[t][hh][v]);
    }
}

// After the last step of a half: add its HC lane parts by the pairwise tree
// into `res` (second half: res = first + second, the tree's top node), and
// clear the accumulators.
template <int HC, int NT>
__device__ __forceinline__ void mf_fold(float (&acc)[NT][HC][4], float (&res)[NT][4], bool second) {
#pragma unroll
  for (int t = 0; t < NT; t++)
#pragma unroll
    for (int v = 0; v < 4; v++) {
      float a[HC];
#pragma unroll
      for (int h = 0; h < HC; h++) a[h] = acc[t][h][v];
#pragma unroll
      for (int st = 1; st < HC; st *= 2)
#pragma unroll
        for (int h = 0; h + st < HC; h += 2 * st) a[h] = a[h] + a[h + st];
      res[t][v] = second ? res[t][v] + a[0] : a[0];
#pragma unroll
      for (int h = 0; h < HC; h++) acc[t][h][v] = 0.0f;
    }
}

// The wave's part of the partition, as NH = H/HC halves of HC lane parts: for
// each half, u = 0 .. BS-1, one step (HC lane parts x NT tiles) per u.  Each lane part accumulates its blocks in u order; the halves are the two
// subtrees of the lane-part tree.  Two steps are in flight.
template <int FMT, int H, int NT>
__device__ __forceinline__ void mf_accumulate(float (&res)[NT][4], const MfAddr<NT>& ad, const PartPlan& pl, int s,
                                              int i, int q) {
  constexpr int HC = H >= 4 ? 4 : H;
  constexpr int NH = H / HC;  // 1, or 2 for H == 8
  const int ic = i < ad.R ? i : ad.R - 1;  // activation row this lane reads
  const int sh = (q >> 1) * 4;
  const int BS = pl.BS;
  const int bs0 = s * H * BS;
  const int nsteps = BS * NH;  // >= 8
  auto first_block = [&](int j) {
    const int half = (NH == 2 && j >= BS) ? 1 : 0;
    return bs0 + H * (j - half * BS) + half * HC;
  };
  float acc[NT][HC][4];
#pragma unroll
  for (int t = 0; t < NT; t++)
#pragma unroll
    for (int h = 0; h < HC; h++)
#pragma unroll
      for (int v = 0; v < 4; v++) acc[t][h][v] = 0.0f;
  MfStep<FMT, HC, NT> s0, s1;
  mf_load(s0, ad, ic, first_block(0));
  mf_load(s1, ad, ic, first_block(1));
  for (int j = 0; j < nsteps; j += 2) {
    mf_compute<FMT, HC, NT>(acc, s0, sh);
    if (j + 2 < nsteps) mf_load(s0, ad, ic, first_block(j + 2));
    if (j + 1 == BS || j + 1 == nsteps) mf_fold<HC, NT>(acc, res, j + 1 > BS);
    if (j + 1 < nsteps) {
      mf_compute<FMT, HC, NT>(acc, s1, sh);
      if (j + 3 < nsteps) mf_load(s1, ad, ic, first_block(j + 3));
      if (j + 2 == BS || j + 2 == nsteps) mf_fold<HC, NT>(acc, res, j + 2 > BS);
    }
  }
}

// One MF tile: 16-row image tiles, NT per wave, (4/S) waves' worth per tile;
// the R activation rows are the MFMA's 16 columns (the rest zero), read from
// the workspace in fragment order.
template <int FMT, int H>
__device__ void mf_tile(const TileArgs& ta, int R, float* red, int parity) {
  constexpr int CB = FMT == FMT_Q8 ? 512 : 256;
  constexpr int NT = mf_tiles_per_wave(H);
  const PartPlan& pl = ta.pl;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & (WAVE - 1);
  const int g = wave >> pl.lgS, s = wave & (pl.S - 1);
  const int i = lane & 15, q = lane >> 4;
  const int64_t ntiles = np_of(ta.n) / TILE;
  const int64_t wrow0 = ta.row0 + (int64_t)g * TILE * NT;  // first row of this wave's tiles
  MfAddr<NT> ad;
#pragma unroll
  for (int t = 0; t < NT; t++) {
    const int64_t it0 = (wrow0 >> 4) + t;
    const int64_t it = it0 < ntiles ? it0 : ntiles - 1;  // past the last tile: reread it, store nothing
    ad.code[t] = ta.code + ((size_t)it * ta.kbp) * CB;
    ad.scale[t] = ta.scale + ((size_t)it * ta.kbp) * TILE;
  }
  ad.aoff = FMT == FMT_Q8 ? (q >> 1) * 256 + i * 16 + (q & 1) * 8 : i * 16 + (q & 1) * 8;
  ad.soff = 4 * q;
  // rows prepared in fragment order: codes [kbp][4][R][8], dx and nsx [kbp][R]
  ad.xc = ta.prep.codes;
  ad.xd = ta.prep.dx;
  ad.xn = ta.prep.nsx;
  ad.xoff = (uint32_t)((q * R + (i < R ? i : R - 1)) * 8);
  ad.R = R;
  float res[NT][4];
  mf_accumulate<FMT, H, NT>(res, ad, pl, s, i, q);
  if (pl.S > 1) {
    float* rb = red + parity * (WAVES * WAVE * 4 * NT);
#pragma unroll
    for (int t = 0; t < NT; t++)
#pragma unroll
      for (int v = 0; v < 4; v++) rb[((wave * NT + t) * WAVE + lane) * 4 + v] = res[t][v];
    __syncthreads();
    if (s != 0) return;
#pragma unroll
    for (int t = 0; t < NT; t++)
#pragma unroll
      for (int v = 0; v < 4; v++) {
        float x = rb[(((g * pl.S) * NT + t) * WAVE + lane) * 4 + v];
        for (int s2 = 1; s2 < pl.S; s2++) x += rb[(((g * pl.S + s2) * NT + t) * WAVE + lane) * 4 + v];
        res[t][v] = x;
      }
  }
  if (i < R) {
#pragma unroll
    for (int t = 0; t < NT; t++)
#pragma unroll
      for (int v = 0; v < 4; v++) {
        const int64_t row = wrow0 + t * TILE + 4 * q + v;
        if (row < ta.n) ta.y[(int64_t)ta.s_dst[i] * ta.ldy + row] = res[t][v];
      }
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
  int ucx;  // RL staging round
};
struct SetArgs {
  ProjDev p[QG_MAX_SET];
  int count;
  int total_tiles;
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
template <int FMT, int R, bool FUSED>
__global__ __launch_bounds__(WG) __attribute__((amdgpu_waves_per_eu(4))) void rl_set_kernel(SetArgs a, int lds_x) {
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
    const bool full = rl_tile<FMT, R, FUSED>(ta, lds, red, parity, p != staged);
    staged = full ? p : -1;
    // the combine area alternates only between tiles that pass its barrier, so
    // a buffer is rewritten only after everyone has read it
    if (d.pl.S > 1) parity ^= 1;
  }
}

template <int FMT>
__global__ __launch_bounds__(WG) __attribute__((amdgpu_waves_per_eu(FMT == FMT_Q8 ? 4 : 3))) void mf_set_kernel(SetArgs a, int R) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int s_map[2 * QG_MAX_ROWS];
  identity_map(s_map);
  float* red = reinterpret_cast<float*>(lds);
  int parity = 0;
  for (int tile = blockIdx.x; tile < a.total_tiles; tile += gridDim.x) {
    int p = 0, t0 = tile;
    while (p + 1 < a.count && t0 >= a.p[p].tiles) t0 -= a.p[p++].tiles;
    const ProjDev& d = a.p[p];
    const TileArgs ta = tile_args(d, (int64_t)t0 * d.rows_per_tile, s_map, 0);
    const PartPlan& pl = d.pl;
    if (pl.H == 1) mf_tile<FMT, 1>(ta, R, red, parity);
    else if (pl.H == 2) mf_tile<FMT, 2>(ta, R, red, parity);
    else if (pl.H == 4) mf_tile<FMT, 4>(ta, R, red, parity);
    else mf_tile<FMT, 8>(ta, R, red, parity);
    if (pl.S > 1) parity ^= 1;
  }
}

// ------------------------------------------------------------- grouped ---

// One workgroup: the valid assignments ordered by (expert, index), then work
// items of at most 16 assignments of one expert.
__global__ __launch_bounds__(1024) void grouped_plan_kernel(const int32_t* __restrict__ expert,
                                                            const int32_t* __restrict__ x_index, int m,
                                                            int64_t n_experts, int x_rows, int* __restrict__ header,
                                                            int* __restrict__ sorted, int* __restrict__ items) {
  __shared__ int s_e[QG_MAX_ASSIGN];
  __shared__ int s_pos[QG_MAX_ASSIGN];  // sorted position -> assignment
  __shared__ int s_start[QG_MAX_ASSIGN];  // 1 where a work item starts
  __shared__ int s_bad, s_valid;
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
      items[3 * item] = s_e[s_pos[p]];
      items[3 * item + 1] = p;
      items[3 * item + 2] = cnt;
    }
  }
  if (tid == 0) {
    header[0] = nv ? s_start[nv - 1] : 0;
    header[1] = s_bad;
  }
}

template <int R>
__device__ __forceinline__ void grouped_rows(TileArgs ta, uint8_t* lds, float* red) {
  ta.ucx = rl_round(ta.lds_x, R, ta.pl, FMT_Q8);
  rl_tile<FMT_Q8, R, false>(ta, lds, red, 0, true);
}

__global__ __launch_bounds__(WG) void grouped_kernel(const uint8_t* __restrict__ images, int64_t expert_bytes,
                                                     size_t scale_off, int64_t n, int64_t k, int kbp, PartPlan pl,
                                                     Prep prep,
                                                     const int* __restrict__ header, const int* __restrict__ sorted,
                                                     const int* __restrict__ items,
                                                     const int32_t* __restrict__ x_index, float* y, int lds_x) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int s_map[2 * QG_MAX_ROWS];
  const int item = blockIdx.y;
  if (item >= header[0]) return;  // uniform over the workgroup, before any barrier
  const int e = items[3 * item], start = items[3 * item + 1], cnt = items[3 * item + 2];
  if (threadIdx.x < cnt) {
    const int a = sorted[start + threadIdx.x];
    s_map[threadIdx.x] = x_index[a];
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
  ta.row0 = (int64_t)blockIdx.x * (WG >> pl.lgP);
  ta.prep = prep;
  ta.xf = nullptr;
  ta.s_src = s_map;
  ta.y = y;
  ta.ldy = n;
  ta.s_dst = s_map + QG_MAX_ROWS;
  ta.lds_x = lds_x;
  ta.pl = pl;
  ta.ucx = 0;  // set per row count
  float* red = reinterpret_cast<float*>(lds + lds_x);
  switch (cnt) {
#define QG_CASE(RR) \
  case RR: grouped_rows<RR>(ta, lds, red); break;
    QG_CASE(1) QG_CASE(2) QG_CASE(3) QG_CASE(4) QG_CASE(5) QG_CASE(6) QG_CASE(7) QG_CASE(8)
    QG_CASE(9) QG_CASE(10) QG_CASE(11) QG_CASE(12) QG_CASE(13) QG_CASE(14) QG_CASE(15) QG_CASE(16)
#undef QG_CASE
    default: break;
  }
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
  if (lds > 64 * 1024) hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, WG, lds) != hipSuccess || per_cu < 1) per_cu = 1;
  const int64_t g = (int64_t)device_cus() * per_cu;
  return (unsigned)(tiles < g ? tiles : g);
}

bool fuses_quantization(int rows) { return rows >= 1 && rows <= FUSE_MAX_ROWS; }

template <int FMT, int R, bool FUSED>
static void launch_rl(const SetArgs& a, int lds_x, hipStream_t s) {
  auto kern = rl_set_kernel<FMT, R, FUSED>;
  const size_t lds = (size_t)lds_x + 2 * WAVES * WAVE * R * 4;
  hipLaunchKernelGGL(kern, dim3(persistent_grid(kern, lds, a.total_tiles)), dim3(WG), lds, s, a, lds_x);
}

template <int FMT>
static void launch_rl_rows(const SetArgs& a, int rows, bool fused, int lds_x, hipStream_t s) {
  if (fused) {
    if (rows == 1) launch_rl<FMT, 1, true>(a, lds_x, s);
    else launch_rl<FMT, 2, true>(a, lds_x, s);
    return;
  }
  switch (rows) {
    case 1: launch_rl<FMT, 1, false>(a, lds_x, s); break;
    case 2: launch_rl<FMT, 2, false>(a, lds_x, s); break;
    case 3: launch_rl<FMT, 3, false>(a, lds_x, s); break;
    case 4: launch_rl<FMT, 4, false>(a, lds_x, s); break;
    case 5: launch_rl<FMT, 5, false>(a, lds_x, s); break;
    case 6: launch_rl<FMT, 6, false>(a, lds_x, s); break;
    case 7: launch_rl<FMT, 7, false>(a, lds_x, s); break;
    default: launch_rl<FMT, 8, false>(a, lds_x, s); break;
  }
}

template <int FMT>
static void launch_mf(const SetArgs& a, int rows, hipStream_t s) {
  auto kern = mf_set_kernel<FMT>;
  const size_t lds = 2 * WAVES * WAVE * 4 * mf_tiles_per_wave(1) * 4;  // combine area: two parities
  hipLaunchKernelGGL(kern, dim3(persistent_grid(kern, lds, a.total_tiles)), dim3(WG), lds, s, a, rows);
}

int launch_qgemv_set(int fmt, const ProjArg* projs, int count, int rows, hipStream_t s) {
  SetArgs a;
  memset(&a, 0, sizeof a);
  a.count = count;
  const bool mf = prep_in_fragment_order(rows);
  // Tiles of projections with longer rows come first: their workgroups stage
  // the most activation blocks, so they get the earliest start.  The order
  // changes no result (each projection has its own output).
  int order[QG_MAX_SET];
  for (int i = 0; i < count; i++) order[i] = i;
  for (int i = 1; i < count; i++)
    for (int j = i; j > 0 && projs[order[j]].k > projs[order[j - 1]].k; j--) {
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
    d.prep = pa.ws ? prep_view(pa.ws, rows, pa.k) : Prep{nullptr, nullptr, nullptr};
    d.xf = pa.x;
    d.y = pa.y;
    d.n = pa.n;
    d.k = pa.k;
    d.kb = (int)kb_of(pa.k);
    d.kbp = (int)kbp_of(pa.k);
    const PartPlan pl = part_plan(d.kbp);
    d.pl = pl;
    d.rows_per_tile = mf ? (WAVES / pl.S) * TILE * mf_tiles_per_wave(pl.H) : WG / pl.P;
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
    if (fmt == FMT_Q8) launch_mf<FMT_Q8>(a, rows, s);
    else launch_mf<FMT_Q4>(a, rows, s);
  } else {
    if (fmt == FMT_Q8) launch_rl_rows<FMT_Q8>(a, rows, fused, lds_x, s);
    else launch_rl_rows<FMT_Q4>(a, rows, fused, lds_x, s);
  }
  return hip_status(hipGetLastError(), mf ? "mf_set_kernel" : "rl_set_kernel");
}

int launch_grouped(const void* images, int64_t n_experts, int64_t n, int64_t k, int x_rows, const int32_t* expert,
                   const int32_t* x_index, int m, float* y, void* ws, hipStream_t s) {
  const GroupedLayout G = grouped_layout(x_rows, k, m);
  uint8_t* w = (uint8_t*)ws;
  int* header = (int*)(w + G.header);
  int* sorted = (int*)(w + G.sorted);
  int* items = (int*)(w + G.items);
  hipLaunchKernelGGL(grouped_plan_kernel, dim3(1), dim3(1024), 0, s, expert, x_index, m, n_experts, x_rows, header,
                     sorted, items);
  if (int st = hip_status(hipGetLastError(), "grouped_plan_kernel")) return st;
  if (m == 0) return QG_OK;
  const int kbp = (int)kbp_of(k);
  const PartPlan pl = part_plan(kbp);
  const int rpt = WG / pl.P;
  const unsigned tiles = (unsigned)((n + rpt - 1) / rpt);
  const size_t need = (size_t)QG_MAX_ROWS * kbp * x_block_bytes(FMT_Q8);
  const int lds_x = (int)((need < (size_t)LDS_X_RL ? need : (size_t)LDS_X_RL) + 15) / 16 * 16;
  const size_t lds = (size_t)lds_x + WAVES * WAVE * QG_MAX_ROWS * 4;
  if (lds > 64 * 1024) hipFuncSetAttribute((const void*)grouped_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  const int64_t eb = (int64_t)image_total_bytes(QG_FMT_Q8_0, n, k);
  const size_t so = image_scale_offset(QG_FMT_Q8_0, n, k);
  hipLaunchKernelGGL(grouped_kernel, dim3(tiles, m), dim3(WG), lds, s, (const uint8_t*)images, eb, so, n, k, kbp, pl,
                     prep_view(w + G.prep, x_rows, k), header, sorted, items, x_index, y, lds_x);
  return hip_status(hipGetLastError(), "grouped_kernel");
}

}  // namespace qg
