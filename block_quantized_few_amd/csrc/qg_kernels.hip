// qg_kernels.hip -- gfx950 kernels of the few-row block-quantized GEMV and
// the C-ABI entry points that validate arguments and launch them.
//
// Work mapping of every GEMV kernel (q8 and f16 lanes).  A 256-thread
// workgroup is 4 waves of 64 lanes; a wave is 4 row slots of 16 lanes; each
// slot owns T weight rows.  Lane j of a slot takes blocks j, j+16, j+32, ... of
// its rows, so a slot streams 16 consecutive blocks per step with fully
// coalesced 16-byte loads, and each lane holds whole blocks, so a block's
// integer dot is exact inside one lane (no cross-lane integer sums).  The
// activation rows (all 1..16 of them) are staged once per workgroup in LDS and
// reused by every weight row of the tile: one weight pass serves every row.
// This is the row tiling of the dasLLAMA pages (a launch never reads past its
// tile, rows past eight share the weight pass; router-GEMV commit of the
// audio-towers page, commit 16880fe of the llama-leg page), done inside the
// kernel.  Each output row keeps its own accumulators in a fixed order
// (blocks in lane order, then a fixed 16-lane tree), so results do not depend
// on how many rows share the launch.
#include <hip/hip_runtime.h>
#include <string.h>

#include "qg_internal.h"
#include "qg_layout.h"

namespace qg {

constexpr int WAVE = 64;
constexpr int LPR = 16;             // lanes per weight row
constexpr int SLOTS = WAVE / LPR;   // row slots per wave
constexpr int WG = 256;             // threads per workgroup
constexpr int WAVES = WG / WAVE;
constexpr int LDS_BUDGET = 48 * 1024;  // activation staging per workgroup
constexpr int FMT_Q8 = 1, FMT_Q4 = 2;

// ------------------------------------------------------------ primitives ---

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Streaming load of weight bytes that are read exactly once: the non-temporal
// hint keeps them from displacing the activation rows in the caches.
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint16_t ld2_stream(const uint16_t* p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ float h2f(uint16_t h) {
  _Float16 v;
  __builtin_memcpy(&v, &h, 2);
  return (float)v;
}

// Exact int32 dot of one Q8_0 block (low/high halves) with one q8 block.
__device__ __forceinline__ int dot_q8(uint4 wl, uint4 wh, uint4 xl, uint4 xh) {
  int s = 0;
  s = __builtin_amdgcn_sdot4((int)wl.x, (int)xl.x, s, false);
  s = __builtin_amdgcn_sdot4((int)wl.y, (int)xl.y, s, false);
  s = __builtin_amdgcn_sdot4((int)wl.z, (int)xl.z, s, false);
  s = __builtin_amdgcn_sdot4((int)wl.w, (int)xl.w, s, false);
  s = __builtin_amdgcn_sdot4((int)wh.x, (int)xh.x, s, false);
  s = __builtin_amdgcn_sdot4((int)wh.y, (int)xh.y, s, false);
  s = __builtin_amdgcn_sdot4((int)wh.z, (int)xh.z, s, false);
  s = __builtin_amdgcn_sdot4((int)wh.w, (int)xh.w, s, false);
  return s;
}

// Exact int32 dot of one Q4_0 block (16 packed bytes) with one q8 block.  The
// raw codes c in [0,15] enter the dot as they are; the -8 offset is folded in
// through the start value nsx = -8 * sum(q_x).
__device__ __forceinline__ int dot_q4(uint4 p, uint4 xl, uint4 xh, int nsx) {
  const unsigned M = 0x0F0F0F0Fu;
  int s = nsx;
  s = __builtin_amdgcn_sdot4((int)(p.x & M), (int)xl.x, s, false);
  s = __builtin_amdgcn_sdot4((int)(p.y & M), (int)xl.y, s, false);
  s = __builtin_amdgcn_sdot4((int)(p.z & M), (int)xl.z, s, false);
  s = __builtin_amdgcn_sdot4((int)(p.w & M), (int)xl.w, s, false);
  s = __builtin_amdgcn_sdot4((int)((p.x >> 4) & M), (int)xh.x, s, false);
  s = __builtin_amdgcn_sdot4((int)((p.y >> 4) & M), (int)xh.y, s, false);
  s = __builtin_amdgcn_sdot4((int)((p.z >> 4) & M), (int)xh.z, s, false);
  s = __builtin_amdgcn_sdot4((int)((p.w >> 4) & M), (int)xh.w, s, false);
  return s;
}

// Sum over the 16 lanes of a row slot; every lane receives the same bits
// (pairs, quads, half-rows by mirror, rows by mirror).
__device__ __forceinline__ float sum16(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // half-row mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row mirror
  return v;
}

// -------------------------------------------------- activation quantizer ---

// q8 quantization of one 32-block: d = amax/127 by IEEE division, q =
// round-half-away(x/d) clamped to [-127, 127], all 0 when d == 0; codes packed
// four per word in element order.
__device__ __forceinline__ void quantize_block(const float* __restrict__ src, unsigned packed[8], float& d, int& sum) {
  float v[32];
  const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const float4 f = s4[i];
    v[4 * i] = f.x;
    v[4 * i + 1] = f.y;
    v[4 * i + 2] = f.z;
    v[4 * i + 3] = f.w;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(v[i]));
  d = amax / 127.0f;
  sum = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) packed[i] = 0;
  if (d != 0.0f) {
#pragma unroll
    for (int i = 0; i < 32; i++) {
      const int q = (int)fminf(fmaxf(roundf(v[i] / d), -127.0f), 127.0f);
      sum += q;
      packed[i >> 2] |= ((unsigned)(q & 0xff)) << (8 * (i & 3));
    }
  }
}

// Workspace layout store of one quantized block (grouped halves, -8*sum).
__device__ __forceinline__ void store_prepared(int8_t* codes, float* dx, int* nsx, int64_t r, int64_t b, int kbp,
                                               const unsigned packed[8], float d, int sum) {
  int8_t* dst = codes + (size_t)r * kbp * 32 + (size_t)(b / GROUP) * 512 + (size_t)(b % GROUP) * 16;
  *reinterpret_cast<uint4*>(dst) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  *reinterpret_cast<uint4*>(dst + 256) = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  dx[r * kbp + b] = d;
  nsx[r * kbp + b] = -8 * sum;
}

// One thread per (row, block).  LANE: workspace layout over kbp blocks (pad
// blocks zeroed); otherwise the plain layout [rows][k], with the code sum.
template <bool LANE>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const float* __restrict__ x, int rows, int64_t k,
                                                            int kb, int kbp, int8_t* __restrict__ codes,
                                                            float* __restrict__ dx, int* __restrict__ sums) {
  const int64_t nblk = LANE ? kbp : kb;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)rows * nblk) return;
  const int64_t r = t / nblk, b = t % nblk;
  unsigned packed[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float d = 0.0f;
  int sum = 0;
  if (b < kb) quantize_block(x + r * k + b * QK, packed, d, sum);
  if (LANE) {
    store_prepared(codes, dx, sums, r, b, kbp, packed, d, sum);
  } else {
    int8_t* dst = codes + r * k + b * QK;
    *reinterpret_cast<uint4*>(dst) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    *reinterpret_cast<uint4*>(dst + 16) = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    dx[r * kb + b] = d;
    sums[r * kb + b] = sum;
  }
}

// Several activation sets in one launch: blockIdx.y picks the set.
struct PrepSet {
  const float* x[QG_MAX_SET];
  int8_t* codes[QG_MAX_SET];
  float* dx[QG_MAX_SET];
  int* nsx[QG_MAX_SET];
  int64_t k[QG_MAX_SET];
  int count;
};

__global__ __launch_bounds__(256) void quantize_rows_set_kernel(PrepSet s, int rows) {
  const int p = blockIdx.y;
  const int64_t k = s.k[p];
  const int kb = (int)kb_of(k), kbp = (int)kbp_of(k);
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)rows * kbp) return;
  const int64_t r = t / kbp, b = t % kbp;
  unsigned packed[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float d = 0.0f;
  int sum = 0;
  if (b < kb) quantize_block(s.x[p] + r * k + b * QK, packed, d, sum);
  store_prepared(s.codes[p], s.dx[p], s.nsx[p], r, b, kbp, packed, d, sum);
}

// ------------------------------------------------------ weight quantizer ---

template <int FMT>
__global__ __launch_bounds__(256) void quantize_weights_kernel(const float* __restrict__ w, int64_t n, int64_t k,
                                                               int kb, int kbp, uint8_t* __restrict__ qs,
                                                               uint16_t* __restrict__ dsc) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n * kbp) return;
  const int64_t o = t / kbp, b = t % kbp;
  unsigned packed[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  uint16_t d16 = 0;
  if (b < kb) {
    float v[32];
    const float4* src = reinterpret_cast<const float4*>(w + o * k + b * QK);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      float4 f = src[i];
      v[4 * i] = f.x;
      v[4 * i + 1] = f.y;
      v[4 * i + 2] = f.z;
      v[4 * i + 3] = f.w;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(v[i]));
    const float qmax = FMT == FMT_Q8 ? 127.0f : 7.0f;
    _Float16 h = (_Float16)(amax / qmax);  // round to nearest even
    __builtin_memcpy(&d16, &h, 2);
    const float dq = (float)h;
    if (dq != 0.0f) {
      if (FMT == FMT_Q8) {
#pragma unroll
        for (int i = 0; i < 32; i++) {
          int q = (int)fminf(fmaxf(roundf(v[i] / dq), -127.0f), 127.0f);
          packed[i >> 2] |= ((unsigned)(q & 0xff)) << (8 * (i & 3));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; i++) {
          int lo = (int)fminf(fmaxf(roundf(v[i] / dq), -8.0f), 7.0f) + 8;
          int hi = (int)fminf(fmaxf(roundf(v[i + 16] / dq), -8.0f), 7.0f) + 8;
          packed[i >> 2] |= ((unsigned)(lo | (hi << 4))) << (8 * (i & 3));
        }
      }
    } else if (FMT == FMT_Q4) {
      for (int i = 0; i < 4; i++) packed[i] = 0x88888888u;  // code 8 stands for 0
    }
  }
  if (FMT == FMT_Q8) {
    uint8_t* dst = qs + q8_lo_offset(o, b, kbp);
    *reinterpret_cast<uint4*>(dst) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    *reinterpret_cast<uint4*>(dst + 256) = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  } else {
    *reinterpret_cast<uint4*>(qs + q4_offset(o, b, kbp)) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  }
  dsc[o * kbp + b] = d16;
}

// ----------------------------------------------------- q8-lane GEMV tile ---

// Prepared rows as the tile sees them.
struct Prep {
  const int8_t* codes;
  const float* dx;
  const int* nsx;
};

// Lanes that share one weight row, chosen from the row's block count alone so
// that a row's fp32 summation order never depends on the launch: each lane
// ends up holding about four blocks of every row it serves.
__host__ __device__ inline int lanes_per_row(int kbp) {
  if (kbp >= 256 && kbp % 64 == 0) return 64;
  if (kbp >= 128 && kbp % 32 == 0) return 32;
  return 16;
}

// LDS bytes of one staged block of one activation row (codes, scale, Q4 start).
__host__ __device__ inline int x_block_bytes(int fmt) { return fmt == FMT_Q4 ? 40 : 36; }

// Blocks per LDS chunk for R rows (multiple of 16, at most kbp).
__host__ __device__ inline int chunk_blocks(int R, int fmt, int kbp, int budget) {
  int cb = (budget / (R * x_block_bytes(fmt))) / GROUP * GROUP;
  if (cb < GROUP) cb = GROUP;
  return cb < kbp ? cb : kbp;
}

// Stage blocks [cb0, cb0 + cbn) of the R activation rows into LDS: codes
// [R][cbn*32], then scales [R][cbn], then (Q4) start values [R][cbn].
template <int FMT, int R>
__device__ __forceinline__ void stage_rows(uint8_t* lds, const Prep& prep, const int* s_src, int kbp, int cb0,
                                           int cbn) {
  int8_t* l_codes = reinterpret_cast<int8_t*>(lds);
  float* l_dx = reinterpret_cast<float*>(lds + (size_t)R * cbn * 32);
  int* l_nsx = reinterpret_cast<int*>(lds + (size_t)R * cbn * 36);
  const int tid = threadIdx.x;
  const int cu = cbn * 2;  // 16-byte units of codes per row
  for (int u = tid; u < R * cu; u += WG) {
    const int r = u / cu, c = u - r * cu;
    reinterpret_cast<uint4*>(l_codes)[u] =
        reinterpret_cast<const uint4*>(prep.codes + (size_t)s_src[r] * kbp * 32 + (size_t)cb0 * 32)[c];
  }
  const int su = cbn / 4;  // 16-byte units of scales per row
  for (int u = tid; u < R * su; u += WG) {
    const int r = u / su, c = u - r * su;
    reinterpret_cast<uint4*>(l_dx)[u] = reinterpret_cast<const uint4*>(prep.dx + (size_t)s_src[r] * kbp + cb0)[c];
    if (FMT == FMT_Q4)
      reinterpret_cast<uint4*>(l_nsx)[u] =
          reinterpret_cast<const uint4*>(prep.nsx + (size_t)s_src[r] * kbp + cb0)[c];
  }
}

// acc[t][r] += blocks [cb0, cb0 + cbn) of weight row t against activation row
// r (staged in LDS with a row stride of cbn blocks).  Lane j of the row's lpr
// lanes takes blocks j, j + lpr, ...; each block's integer dot is exact.
template <int FMT, int R, int T>
__device__ __forceinline__ void accumulate(float (&acc)[T][R], const uint8_t* const (&wrow)[T],
                                           const uint16_t* const (&drow)[T], const uint8_t* lds, int cb0, int cbn,
                                           int lpr, int j) {
  const int8_t* l_codes = reinterpret_cast<const int8_t*>(lds);
  const float* l_dx = reinterpret_cast<const float*>(lds + (size_t)R * cbn * 32);
  const int* l_nsx = reinterpret_cast<const int*>(lds + (size_t)R * cbn * 36);
  const int jo = (j % GROUP) * 16;
#pragma unroll 2
  for (int b = j; b < cbn; b += lpr) {
    const int gb = cb0 + b;
    uint4 wl[T], wh[T];
    float dw[T];
#pragma unroll
    for (int t = 0; t < T; t++) {
      if (FMT == FMT_Q8) {
        const uint8_t* p = wrow[t] + (size_t)(gb / GROUP) * 512 + jo;
        wl[t] = ld16_stream(p);
        wh[t] = ld16_stream(p + 256);
      } else {
        wl[t] = ld16_stream(wrow[t] + (size_t)gb * 16);
      }
      dw[t] = h2f(ld2_stream(drow[t] + gb));
    }
#pragma unroll
    for (int r = 0; r < R; r++) {
      const int8_t* xb = l_codes + (size_t)r * cbn * 32 + (b / GROUP) * 512 + jo;
      const uint4 xl = ld16(xb), xh = ld16(xb + 256);
      const float dxr = l_dx[r * cbn + b];
      const int ns = FMT == FMT_Q4 ? l_nsx[r * cbn + b] : 0;
#pragma unroll
      for (int t = 0; t < T; t++) {
        const int isum = FMT == FMT_Q8 ? dot_q8(wl[t], wh[t], xl, xh) : dot_q4(wl[t], xl, xh, ns);
        acc[t][r] = __builtin_fmaf((float)isum, dw[t] * dxr, acc[t][r]);
      }
    }
  }
}

// Sum over the lpr lanes of a row (fixed tree; every lane gets the same bits).
__device__ __forceinline__ float sum_lanes(float v, int lpr) {
  v = sum16(v);
  if (lpr >= 32) v += __shfl_xor(v, 16);
  if (lpr >= 64) v += __shfl_xor(v, 32);
  return v;
}

// One tile of one image: weight rows row0 + t*slots + s (t < T, slot s <
// WG/lpr) against R activation rows.  s_src[r] names the prepared row that
// feeds activation row r and s_dst[r] the output row it lands in (both LDS).
// `staged`: all kbp blocks of the rows are already in LDS; otherwise they are
// staged here in chunks that fit lds_bytes.
template <int FMT, int R, int T>
__device__ __forceinline__ void qgemv_tile(const uint8_t* __restrict__ qs, const uint16_t* __restrict__ dsc,
                                           int64_t N, int kbp, int64_t row0, const Prep& prep, const int* s_src,
                                           float* __restrict__ y, int64_t ldy, const int* s_dst, uint8_t* lds,
                                           int lds_bytes, bool staged) {
  constexpr int CODE_B = FMT == FMT_Q8 ? 32 : 16;
  const int lpr = lanes_per_row(kbp);
  const int slots = WG / lpr;
  const int slot = threadIdx.x / lpr, j = threadIdx.x % lpr;
  int64_t n[T];
  bool valid[T];
  const uint8_t* wrow[T];
  const uint16_t* drow[T];
#pragma unroll
  for (int t = 0; t < T; t++) {
    n[t] = row0 + (int64_t)(t * slots + slot);
    valid[t] = n[t] < N;
    const int64_t nc = valid[t] ? n[t] : N - 1;  // out-of-range slots read a real row, store nothing
    wrow[t] = qs + nc * kbp * CODE_B;
    drow[t] = dsc + nc * kbp;
  }
  float acc[T][R];
#pragma unroll
  for (int t = 0; t < T; t++)
#pragma unroll
    for (int r = 0; r < R; r++) acc[t][r] = 0.0f;
  if (staged) {
    accumulate<FMT, R, T>(acc, wrow, drow, lds, 0, kbp, lpr, j);
  } else {
    const int cbmax = chunk_blocks(R, FMT, kbp, lds_bytes);
    for (int cb0 = 0; cb0 < kbp; cb0 += cbmax) {
      const int cbn = min(cbmax, kbp - cb0);
      __syncthreads();  // earlier readers of LDS are done
      stage_rows<FMT, R>(lds, prep, s_src, kbp, cb0, cbn);
      __syncthreads();
      accumulate<FMT, R, T>(acc, wrow, drow, lds, cb0, cbn, lpr, j);
    }
  }
#pragma unroll
  for (int t = 0; t < T; t++)
#pragma unroll
    for (int r = 0; r < R; r++) {
      const float v = sum_lanes(acc[t][r], lpr);
      if (valid[t] && j == r) y[(int64_t)s_dst[r] * ldy + n[t]] = v;
    }
}

// Up to QG_MAX_SET projections (same rows) in one launch.  Tiles are numbered
// projection by projection; workgroup g takes tiles g, g + G, g + 2G, ... and
// keeps a projection's activation rows in LDS while its tiles last.
struct ProjDev {
  const uint8_t* qs;
  const uint16_t* dsc;
  Prep prep;
  float* y;
  int64_t n;
  int kbp;
  int tiles;
  int rows_per_tile;
};
struct SetArgs {
  ProjDev p[QG_MAX_SET];
  int count;
  int total_tiles;
};

template <int FMT, int R, int T>
__global__ __launch_bounds__(WG) void qgemv_set_kernel(SetArgs a, int lds_bytes) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int s_map[2 * QG_MAX_ROWS];
  if (threadIdx.x < QG_MAX_ROWS) {
    s_map[threadIdx.x] = threadIdx.x;
    s_map[QG_MAX_ROWS + threadIdx.x] = threadIdx.x;
  }
  __syncthreads();
  int staged = -1;
  for (int tile = blockIdx.x; tile < a.total_tiles; tile += gridDim.x) {
    int p = 0, t0 = tile;
    while (p + 1 < a.count && t0 >= a.p[p].tiles) t0 -= a.p[p++].tiles;
    const ProjDev& d = a.p[p];
    const bool fits = R * d.kbp * x_block_bytes(FMT) <= lds_bytes;
    if (fits && p != staged) {
      __syncthreads();
      stage_rows<FMT, R>(lds, d.prep, s_map, d.kbp, 0, d.kbp);
      __syncthreads();
      staged = p;
    } else if (!fits) {
      staged = -1;
    }
    qgemv_tile<FMT, R, T>(d.qs, d.dsc, d.n, d.kbp, (int64_t)t0 * d.rows_per_tile, d.prep, s_map, d.y, d.n,
                          s_map + QG_MAX_ROWS, lds, lds_bytes, fits);
  }
}

// ------------------------------------------------------------- grouped ---

// One workgroup: stable order of the valid assignments by expert (rank by
// (expert, index)), then work items of at most 16 assignments of one expert.
__global__ __launch_bounds__(1024) void grouped_plan_kernel(const int32_t* __restrict__ expert,
                                                            const int32_t* __restrict__ x_index, int m,
                                                            int64_t n_experts, int x_rows, int* __restrict__ header,
                                                            int* __restrict__ sorted, int* __restrict__ items) {
  __shared__ int s_e[QG_MAX_ASSIGN];
  __shared__ int s_sorted[QG_MAX_ASSIGN];
  __shared__ int s_bad, s_valid;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_bad = 0;
    s_valid = 0;
  }
  __syncthreads();
  for (int j = tid; j < m; j += blockDim.x) {
    const int e = expert[j], xi = x_index[j];
    const bool ok = e >= 0 && e < n_experts && xi >= 0 && xi < x_rows;
    s_e[j] = ok ? e : 0x7fffffff;
    if (!ok) atomicAdd(&s_bad, 1);
    else atomicAdd(&s_valid, 1);
  }
  __syncthreads();
  for (int j = tid; j < m; j += blockDim.x) {
    const int e = s_e[j];
    if (e == 0x7fffffff) continue;
    int rank = 0;
    for (int i = 0; i < m; i++) {
      const int f = s_e[i];
      rank += (f < e) || (f == e && i < j);
    }
    s_sorted[rank] = j;
    sorted[rank] = j;
  }
  __syncthreads();
  if (tid == 0) {
    const int nv = s_valid;
    int n_items = 0, run = 0, prev = -1;
    for (int p = 0; p < nv; p++) {
      const int e = s_e[s_sorted[p]];
      if (p == 0 || e != prev || run == QG_MAX_ROWS) {
        items[3 * n_items] = e;
        items[3 * n_items + 1] = p;
        items[3 * n_items + 2] = 0;
        n_items++;
        run = 0;
      }
      items[3 * (n_items - 1) + 2]++;
      run++;
      prev = e;
    }
    header[0] = n_items;
    header[1] = s_bad;
  }
}

template <int T>
__global__ __launch_bounds__(WG) void qgemv_grouped_kernel(const uint8_t* __restrict__ images, int64_t expert_bytes,
                                                           size_t scale_off, int64_t N, int kbp, Prep prep,
                                                           const int* __restrict__ header,
                                                           const int* __restrict__ sorted,
                                                           const int* __restrict__ items,
                                                           const int32_t* __restrict__ x_index, float* y,
                                                           int lds_bytes) {
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
  const uint16_t* dsc = reinterpret_cast<const uint16_t*>(img + scale_off);
  const int64_t row0 = (int64_t)blockIdx.x * ((WG / lanes_per_row(kbp)) * T);
  switch (cnt) {
#define QG_CASE(RR)                                                                                                \
  case RR:                                                                                                         \
    qgemv_tile<FMT_Q8, RR, T>(img, dsc, N, kbp, row0, prep, s_map, y, N, s_map + QG_MAX_ROWS, lds, lds_bytes,    \
                              false);                                                                             \
    break;
    QG_CASE(1) QG_CASE(2) QG_CASE(3) QG_CASE(4) QG_CASE(5) QG_CASE(6) QG_CASE(7) QG_CASE(8)
    QG_CASE(9) QG_CASE(10) QG_CASE(11) QG_CASE(12) QG_CASE(13) QG_CASE(14) QG_CASE(15) QG_CASE(16)
#undef QG_CASE
    default: break;
  }
}

// ------------------------------------------------------------ block dots ---

template <int FMT>
__global__ __launch_bounds__(256) void blockdots_kernel(const uint8_t* __restrict__ qs, int64_t N, int kbp, int kb,
                                                        const int8_t* __restrict__ qx, int rows, int64_t k,
                                                        int* __restrict__ isum) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)rows * N * kb) return;
  const int64_t b = t % kb, o = (t / kb) % N, r = t / (kb * N);
  const int8_t* xq = qx + r * k + b * QK;
  const uint4 xl = ld16(xq), xh = ld16(xq + 16);
  int s;
  if (FMT == FMT_Q8) {
    const uint8_t* p = qs + q8_lo_offset(o, b, kbp);
    s = dot_q8(ld16(p), ld16(p + 256), xl, xh);
  } else {
    int qsum = 0;
    const int8_t* xb = xq;
    for (int i = 0; i < 32; i++) qsum += xb[i];
    s = dot_q4(ld16(qs + q4_offset(o, b, kbp)), xl, xh, -8 * qsum);
  }
  isum[t] = s;
}

// ----------------------------------------------------------- f16 lane ---

// Same slot mapping; lane j reads 8 halfwords (16 bytes) at chunk j, j+16, ...
// and multiplies them with fp32 activations staged in LDS, one fma per weight
// and row (fp16 -> fp32 conversion is exact).
template <int R, int T>
__global__ __launch_bounds__(WG) void gemv_f16_kernel(const uint16_t* __restrict__ w, int64_t N, int64_t K,
                                                      const float* __restrict__ x, float* __restrict__ y, int ce) {
  extern __shared__ __align__(16) uint8_t lds[];
  float* l_x = reinterpret_cast<float*>(lds);
  const int tid = threadIdx.x;
  const int lane = tid & (WAVE - 1), wave = tid / WAVE;
  const int slot = lane / LPR, j = lane % LPR;
  const int64_t row0 = (int64_t)blockIdx.x * (WAVES * SLOTS * T);
  int64_t n[T];
  bool valid[T];
  const uint16_t* wrow[T];
#pragma unroll
  for (int t = 0; t < T; t++) {
    n[t] = row0 + (int64_t)((wave * T + t) * SLOTS + slot);
    valid[t] = n[t] < N;
    wrow[t] = w + (valid[t] ? n[t] : N - 1) * K;
  }
  float acc[T][R];
#pragma unroll
  for (int t = 0; t < T; t++)
#pragma unroll
    for (int r = 0; r < R; r++) acc[t][r] = 0.0f;

  for (int64_t c0 = 0; c0 < K; c0 += ce) {
    const int cen = (int)min((int64_t)ce, K - c0);  // multiple of 8
    if (c0) __syncthreads();
    const int cu = cen / 4;
    for (int u = tid; u < R * cu; u += WG) {
      const int r = u / cu, c = u - r * cu;
      reinterpret_cast<float4*>(l_x + (size_t)r * ce)[c] = reinterpret_cast<const float4*>(x + r * K + c0)[c];
    }
    __syncthreads();
#pragma unroll 2
    for (int c = j; c * 8 < cen; c += LPR) {
      uint4 wv[T];
#pragma unroll
      for (int t = 0; t < T; t++) wv[t] = ld16_stream(wrow[t] + c0 + c * 8);
#pragma unroll
      for (int r = 0; r < R; r++) {
        const float4 x0 = *reinterpret_cast<const float4*>(l_x + (size_t)r * ce + c * 8);
        const float4 x1 = *reinterpret_cast<const float4*>(l_x + (size_t)r * ce + c * 8 + 4);
        const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int t = 0; t < T; t++) {
          const unsigned wu[4] = {wv[t].x, wv[t].y, wv[t].z, wv[t].w};
          float a = acc[t][r];
#pragma unroll
          for (int e = 0; e < 4; e++) {
            a = __builtin_fmaf(h2f((uint16_t)(wu[e] & 0xffff)), xv[2 * e], a);
            a = __builtin_fmaf(h2f((uint16_t)(wu[e] >> 16)), xv[2 * e + 1], a);
          }
          acc[t][r] = a;
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < T; t++)
#pragma unroll
    for (int r = 0; r < R; r++) {
      const float v = sum16(acc[t][r]);
      if (valid[t] && j == r) y[(int64_t)r * N + n[t]] = v;
    }
}

// ------------------------------------------------------------- MoE glue ---

// One workgroup per row: softmax over the logits (double, max subtracted,
// fixed reduction tree) and the topk experts by logit, ties to the lower index.
__global__ __launch_bounds__(256) void moe_route_kernel(const float* __restrict__ logits, int E, int topk,
                                                        int shared_expert, int32_t* __restrict__ expert,
                                                        int32_t* __restrict__ x_index, float* __restrict__ weight) {
  __shared__ float s_l[1024];
  __shared__ unsigned char s_taken[1024];
  __shared__ double s_d[256];
  __shared__ float s_bv[256];
  __shared__ int s_bi[256];
  const int r = blockIdx.x, tid = threadIdx.x;
  const int slots = topk + (shared_expert >= 0 ? 1 : 0);
  for (int e = tid; e < E; e += 256) {
    s_l[e] = logits[(int64_t)r * E + e];
    s_taken[e] = 0;
  }
  __syncthreads();
  double mx = -INFINITY;
  for (int e = tid; e < E; e += 256) mx = fmax(mx, (double)s_l[e]);
  s_d[tid] = mx;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) s_d[tid] = fmax(s_d[tid], s_d[tid + s]);
    __syncthreads();
  }
  mx = s_d[0];
  __syncthreads();
  double sum = 0.0;
  for (int e = tid; e < E; e += 256) sum += exp((double)s_l[e] - mx);
  s_d[tid] = sum;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) s_d[tid] += s_d[tid + s];
    __syncthreads();
  }
  const double total = s_d[0];
  for (int k = 0; k < topk; k++) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int e = tid; e < E; e += 256)
      if (!s_taken[e] && (s_l[e] > bv || (s_l[e] == bv && e < bi))) {
        bv = s_l[e];
        bi = e;
      }
    s_bv[tid] = bv;
    s_bi[tid] = bi;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if (tid < s) {
        const float ov = s_bv[tid + s];
        const int oi = s_bi[tid + s];
        if (ov > s_bv[tid] || (ov == s_bv[tid] && oi < s_bi[tid])) {
          s_bv[tid] = ov;
          s_bi[tid] = oi;
        }
      }
      __syncthreads();
    }
    if (tid == 0) {
      const int e = s_bi[0];
      s_taken[e] = 1;
      expert[(int64_t)r * slots + k] = e;
      x_index[(int64_t)r * slots + k] = r;
      weight[(int64_t)r * slots + k] = (float)(exp((double)s_l[e] - mx) / total);
    }
    __syncthreads();
  }
  if (tid == 0 && shared_expert >= 0) {
    expert[(int64_t)r * slots + topk] = shared_expert;
    x_index[(int64_t)r * slots + topk] = r;
    weight[(int64_t)r * slots + topk] = 1.0f;
  }
}

__global__ __launch_bounds__(256) void swiglu_kernel(const float* __restrict__ gu, int m, int64_t ffn,
                                                     float* __restrict__ h) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)m * ffn) return;
  const int64_t j = t / ffn, i = t % ffn;
  const float g = gu[j * 2 * ffn + i], u = gu[j * 2 * ffn + ffn + i];
  h[t] = g / (1.0f + expf(-g)) * u;
}

// Each thread writes 4 contiguous outputs from 16-byte loads; every sum runs
// over the slots in order.
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ o,
                                                          const float* __restrict__ weight, int slots,
                                                          int64_t hidden, float* __restrict__ y) {
  const int r = blockIdx.y;
  const int64_t i4 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i4 * 4 >= hidden) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < slots; s++) {
    const float wgt = weight[(int64_t)r * slots + s];
    const float4 v = reinterpret_cast<const float4*>(o + ((int64_t)r * slots + s) * hidden)[i4];
    acc.x = __builtin_fmaf(wgt, v.x, acc.x);
    acc.y = __builtin_fmaf(wgt, v.y, acc.y);
    acc.z = __builtin_fmaf(wgt, v.z, acc.z);
    acc.w = __builtin_fmaf(wgt, v.w, acc.w);
  }
  reinterpret_cast<float4*>(y + (int64_t)r * hidden)[i4] = acc;
}

// --------------------------------------------------------- host helpers ---

static int launched(const char* what) { return hip_status(hipGetLastError(), what); }

static unsigned grid1(int64_t threads, int per) { return (unsigned)((threads + per - 1) / per); }

// Weight rows per lane group: T = 2 when that still yields enough tiles.
static int pick_t(int64_t total_rows) { return (total_rows + 31) / 32 >= 1024 ? 2 : 1; }

constexpr int LDS_MAX = 80 * 1024;  // staged activation rows: at least two workgroups per CU

static int device_cus() {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    hipGetDevice(&dev);
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  }
  return cus;
}

// Workgroups to launch: no more than the device holds at once (the kernel
// loops over the remaining tiles) and no more than there are tiles.
template <typename K>
static unsigned persistent_grid(K kernel, size_t lds, int64_t tiles) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, WG, lds) != hipSuccess || per_cu < 1) per_cu = 1;
  const int64_t g = (int64_t)device_cus() * per_cu;
  return (unsigned)(tiles < g ? tiles : g);
}

template <int FMT, int R, int T>
static void launch_set_rt(const SetArgs& a, size_t lds, hipStream_t s) {
  auto kern = qgemv_set_kernel<FMT, R, T>;
  if (lds > 64 * 1024) hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  const unsigned grid = persistent_grid(kern, lds, a.total_tiles);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(WG), lds, s, a, (int)lds);
}

template <int FMT, int T>
static void launch_set_t(const SetArgs& a, int rows, size_t lds, hipStream_t s) {
  switch (rows) {
#define QG_R(RR) \
  case RR: launch_set_rt<FMT, RR, T>(a, lds, s); break;
    QG_R(1) QG_R(2) QG_R(3) QG_R(4) QG_R(5) QG_R(6) QG_R(7) QG_R(8)
    QG_R(9) QG_R(10) QG_R(11) QG_R(12) QG_R(13) QG_R(14) QG_R(15) QG_R(16)
#undef QG_R
  }
}

static int launch_set(int fmt, SetArgs& a, int rows, hipStream_t s) {
  int64_t total_rows = 0;
  for (int i = 0; i < a.count; i++) total_rows += a.p[i].n;
  const int T = pick_t(total_rows);
  int64_t tiles = 0;
  size_t lds = 0;
  for (int i = 0; i < a.count; i++) {
    ProjDev& d = a.p[i];
    d.rows_per_tile = (WG / lanes_per_row(d.kbp)) * T;
    d.tiles = (int)((d.n + d.rows_per_tile - 1) / d.rows_per_tile);
    tiles += d.tiles;
    const size_t x = (size_t)rows * d.kbp * x_block_bytes(fmt);
    lds = x > lds ? x : lds;
  }
  if (lds > (size_t)LDS_MAX) lds = LDS_MAX;  // larger rows are staged in chunks
  a.total_tiles = (int)tiles;
  if (fmt == FMT_Q8) {
    if (T == 2) launch_set_t<FMT_Q8, 2>(a, rows, lds, s);
    else launch_set_t<FMT_Q8, 1>(a, rows, lds, s);
  } else {
    if (T == 2) launch_set_t<FMT_Q4, 2>(a, rows, lds, s);
    else launch_set_t<FMT_Q4, 1>(a, rows, lds, s);
  }
  return launched("qgemv_set_kernel");
}

static ProjDev proj_dev(int fmt, const void* image, int64_t n, int64_t k, const void* ws, int rows, float* y) {
  ProjDev d;
  const uint8_t* img = (const uint8_t*)image;
  d.qs = img;
  d.dsc = (const uint16_t*)(img + image_scale_offset(fmt, n, k));
  const PrepLayout L = prep_layout(rows, k);
  const uint8_t* w = (const uint8_t*)ws;
  d.prep.codes = (const int8_t*)(w + L.codes);
  d.prep.dx = (const float*)(w + L.dx);
  d.prep.nsx = (const int*)(w + L.nsx);
  d.y = y;
  d.n = n;
  d.kbp = (int)kbp_of(k);
  d.tiles = 0;
  return d;
}

// Common argument checks of the q8 lane.
static int check_q8_args(int fmt, const void* image, int64_t n, int64_t k, int rows, const float* y) {
  if (fmt != QG_FMT_Q8_0 && fmt != QG_FMT_Q4_0) return fail(QG_EINVAL, "fmt=%d is not Q8_0 (1) or Q4_0 (2)", fmt);
  if (rows < 0 || rows > QG_MAX_ROWS) return fail(QG_EROWS, "rows=%d outside 0..%d", rows, QG_MAX_ROWS);
  if (n < 1 || n > (1LL << 31) - 1) return fail(QG_ESHAPE, "n=%lld outside 1..2^31-1", (long long)n);
  if (k < QK || k % QK || k > (1LL << 24))
    return fail(QG_ESHAPE, "k=%lld is not a positive multiple of 32 up to 2^24", (long long)k);
  if (!image) return fail(QG_EINVAL, "w_image is null");
  if (!y) return fail(QG_EINVAL, "y is null");
  if (!aligned(image, 256)) return fail(QG_EALIGN, "w_image %p is not 256-byte aligned", image);
  if (!aligned(y, 4)) return fail(QG_EALIGN, "y %p is not 4-byte aligned", (const void*)y);
  return QG_OK;
}

static int check_ws(const void* ws, size_t have, int rows, int64_t k) {
  if (!ws) return fail(QG_EINVAL, "ws is null");
  if (!aligned(ws, 256)) return fail(QG_EALIGN, "ws %p is not 256-byte aligned", ws);
  const size_t need = prep_layout(rows, k).total;
  if (have < need) return fail(QG_EWORKSPACE, "ws_bytes=%zu < %zu needed for rows=%d k=%lld", have, need, rows,
                               (long long)k);
  return QG_OK;
}

static int check_x(const float* x, int rows, int64_t k) {
  if (!x) return fail(QG_EINVAL, "x is null");
  if (!aligned(x, 16)) return fail(QG_EALIGN, "x %p is not 16-byte aligned", (const void*)x);
  if (rows < 1 || rows > QG_MAX_PREP_ROWS) return fail(QG_EROWS, "rows=%d outside 1..%d", rows, QG_MAX_PREP_ROWS);
  if (k < QK || k % QK || k > (1LL << 24))
    return fail(QG_ESHAPE, "k=%lld is not a positive multiple of 32 up to 2^24", (long long)k);
  return QG_OK;
}

static int prepare(const float* x, int rows, int64_t k, void* ws, hipStream_t s) {
  const PrepLayout L = prep_layout(rows, k);
  uint8_t* w = (uint8_t*)ws;
  const int kbp = (int)kbp_of(k);
  hipLaunchKernelGGL(quantize_rows_kernel<true>, dim3(grid1((int64_t)rows * kbp, 256)), dim3(256), 0, s, x, rows, k,
                     (int)kb_of(k), kbp, (int8_t*)(w + L.codes), (float*)(w + L.dx), (int*)(w + L.nsx));
  return launched("quantize_rows_kernel");
}

static int gemv_one(int fmt, const void* image, int64_t n, int64_t k, const void* ws, int rows, float* y,
                    hipStream_t s) {
  SetArgs a;
  memset(&a, 0, sizeof a);
  a.count = 1;
  a.p[0] = proj_dev(fmt, image, n, k, ws, rows, y);
  return launch_set(fmt, a, rows, s);
}

template <int R, int T>
static void launch_f16_rt(const uint16_t* w, int64_t n, int64_t k, const float* x, float* y, hipStream_t s) {
  int ce = (LDS_BUDGET / (R * 4)) / 128 * 128;
  if (ce < 128) ce = 128;
  const int64_t kr = (k + 127) / 128 * 128;
  if (ce > kr) ce = (int)kr;
  const unsigned grid = (unsigned)((n + 16 * T - 1) / (16 * T));
  hipLaunchKernelGGL((gemv_f16_kernel<R, T>), dim3(grid), dim3(WG), (size_t)R * ce * 4, s, w, n, k, x, y, ce);
}

template <int T>
static void launch_f16_t(const uint16_t* w, int64_t n, int64_t k, const float* x, int rows, float* y,
                         hipStream_t s) {
  switch (rows) {
#define QG_R(RR) \
  case RR: launch_f16_rt<RR, T>(w, n, k, x, y, s); break;
    QG_R(1) QG_R(2) QG_R(3) QG_R(4) QG_R(5) QG_R(6) QG_R(7) QG_R(8)
    QG_R(9) QG_R(10) QG_R(11) QG_R(12) QG_R(13) QG_R(14) QG_R(15) QG_R(16)
#undef QG_R
  }
}

}  // namespace qg

using namespace qg;

extern "C" {

int qg_quantize_weights(int fmt, const float* w, int64_t n, int64_t k, void* image, qg_stream stream) {
  if (fmt != QG_FMT_Q8_0 && fmt != QG_FMT_Q4_0) return fail(QG_EINVAL, "fmt=%d is not Q8_0 (1) or Q4_0 (2)", fmt);
  if (!w || !image) return fail(QG_EINVAL, "null buffer");
  if (n < 1 || k < QK || k % QK) return fail(QG_ESHAPE, "n=%lld k=%lld", (long long)n, (long long)k);
  if (!aligned(w, 16)) return fail(QG_EALIGN, "w %p is not 16-byte aligned", (const void*)w);
  if (!aligned(image, 256)) return fail(QG_EALIGN, "image %p is not 256-byte aligned", image);
  if (int st = check_device()) return st;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* img = (uint8_t*)image;
  uint16_t* dsc = (uint16_t*)(img + image_scale_offset(fmt, n, k));
  const int kb = (int)kb_of(k), kbp = (int)kbp_of(k);
  const unsigned g = grid1(n * kbp, 256);
  if (fmt == QG_FMT_Q8_0)
    hipLaunchKernelGGL(quantize_weights_kernel<FMT_Q8>, dim3(g), dim3(256), 0, s, w, n, k, kb, kbp, img, dsc);
  else
    hipLaunchKernelGGL(quantize_weights_kernel<FMT_Q4>, dim3(g), dim3(256), 0, s, w, n, k, kb, kbp, img, dsc);
  if (int st = launched("quantize_weights_kernel")) return st;
  return ok();
}

int qg_prepare_rows(const float* x, int rows, int64_t k, void* ws, size_t ws_bytes, qg_stream stream) {
  if (int st = check_x(x, rows, k)) return st;
  if (int st = check_ws(ws, ws_bytes, rows, k)) return st;
  if (int st = check_device()) return st;
  if (int st = prepare(x, rows, k, ws, (hipStream_t)stream)) return st;
  return ok();
}

int qg_prepare_rows_set(const qg_act* acts, int count, int rows, qg_stream stream) {
  if (!acts || count < 1 || count > QG_MAX_SET) return fail(QG_EINVAL, "count=%d outside 1..%d", count, QG_MAX_SET);
  PrepSet ps;
  memset(&ps, 0, sizeof ps);
  ps.count = count;
  int maxkbp = 0;
  for (int i = 0; i < count; i++) {
    if (int st = check_x(acts[i].x, rows, acts[i].k)) return fail(st, "acts[%d]: x/rows/k invalid", i);
    if (int st = check_ws(acts[i].ws, acts[i].ws_bytes, rows, acts[i].k)) return fail(st, "acts[%d]: bad ws", i);
    const PrepLayout L = prep_layout(rows, acts[i].k);
    uint8_t* w = (uint8_t*)acts[i].ws;
    ps.x[i] = acts[i].x;
    ps.k[i] = acts[i].k;
    ps.codes[i] = (int8_t*)(w + L.codes);
    ps.dx[i] = (float*)(w + L.dx);
    ps.nsx[i] = (int*)(w + L.nsx);
    maxkbp = (int)kbp_of(acts[i].k) > maxkbp ? (int)kbp_of(acts[i].k) : maxkbp;
  }
  if (int st = check_device()) return st;
  hipLaunchKernelGGL(quantize_rows_set_kernel, dim3(grid1((int64_t)rows * maxkbp, 256), count), dim3(256), 0,
                     (hipStream_t)stream, ps, rows);
  if (int st = launched("quantize_rows_set_kernel")) return st;
  return ok();
}

int qgemv_prepared(int fmt, const void* w_image, int64_t n, int64_t k, const void* ws, int rows, float* y,
                   qg_stream stream) {
  if (int st = check_q8_args(fmt, w_image, n, k, rows, y)) return st;
  if (rows == 0) return ok();
  if (!ws) return fail(QG_EINVAL, "ws is null");
  if (!aligned(ws, 256)) return fail(QG_EALIGN, "ws %p is not 256-byte aligned", ws);
  if (int st = check_device()) return st;
  if (int st = gemv_one(fmt, w_image, n, k, ws, rows, y, (hipStream_t)stream)) return st;
  return ok();
}

static int qgemv_fmt(int fmt, const void* w_image, int64_t n, int64_t k, const float* x, int rows, float* y,
                     void* ws, size_t ws_bytes, qg_stream stream) {
  if (int st = check_q8_args(fmt, w_image, n, k, rows, y)) return st;
  if (rows == 0) return ok();
  if (int st = check_x(x, rows, k)) return st;
  if (int st = check_ws(ws, ws_bytes, rows, k)) return st;
  if (int st = check_device()) return st;
  hipStream_t s = (hipStream_t)stream;
  if (int st = prepare(x, rows, k, ws, s)) return st;
  if (int st = gemv_one(fmt, w_image, n, k, ws, rows, y, s)) return st;
  return ok();
}

int qgemv_q8_0(const void* w_image, int64_t n, int64_t k, const float* x, int rows, float* y, void* ws,
               size_t ws_bytes, qg_stream stream) {
  return qgemv_fmt(QG_FMT_Q8_0, w_image, n, k, x, rows, y, ws, ws_bytes, stream);
}

int qgemv_q4_0(const void* w_image, int64_t n, int64_t k, const float* x, int rows, float* y, void* ws,
               size_t ws_bytes, qg_stream stream) {
  return qgemv_fmt(QG_FMT_Q4_0, w_image, n, k, x, rows, y, ws, ws_bytes, stream);
}

int qgemv_set(int fmt, const qg_proj* projs, int count, int rows, qg_stream stream) {
  if (!projs || count < 1 || count > QG_MAX_SET) return fail(QG_EINVAL, "count=%d outside 1..%d", count, QG_MAX_SET);
  for (int i = 0; i < count; i++) {
    if (int st = check_q8_args(fmt, projs[i].w_image, projs[i].n, projs[i].k, rows, projs[i].y))
      return fail(st, "projs[%d]: invalid (%s)", i, qg_status_string(st));
    if (!projs[i].ws || !aligned(projs[i].ws, 256)) return fail(QG_EALIGN, "projs[%d].ws null or misaligned", i);
  }
  if (rows == 0) return ok();
  if (int st = check_device()) return st;
  SetArgs a;
  memset(&a, 0, sizeof a);
  a.count = count;
  for (int i = 0; i < count; i++)
    a.p[i] = proj_dev(fmt, projs[i].w_image, projs[i].n, projs[i].k, projs[i].ws, rows, projs[i].y);
  if (int st = launch_set(fmt, a, rows, (hipStream_t)stream)) return st;
  return ok();
}

int gemv_f16(const uint16_t* w, int64_t n, int64_t k, const float* x, int rows, float* y, qg_stream stream) {
  if (rows < 0 || rows > QG_MAX_ROWS) return fail(QG_EROWS, "rows=%d outside 0..%d", rows, QG_MAX_ROWS);
  if (n < 1 || n > (1LL << 31) - 1) return fail(QG_ESHAPE, "n=%lld outside 1..2^31-1", (long long)n);
  if (k < 8 || k % 8 || k > (1LL << 24))
    return fail(QG_ESHAPE, "k=%lld is not a positive multiple of 8 up to 2^24", (long long)k);
  if (!w || !y || (!x && rows)) return fail(QG_EINVAL, "null buffer");
  if (!aligned(w, 16)) return fail(QG_EALIGN, "w %p is not 16-byte aligned", (const void*)w);
  if (rows && !aligned(x, 16)) return fail(QG_EALIGN, "x %p is not 16-byte aligned", (const void*)x);
  if (!aligned(y, 4)) return fail(QG_EALIGN, "y %p is not 4-byte aligned", (const void*)y);
  if (rows == 0) return ok();
  if (int st = check_device()) return st;
  hipStream_t s = (hipStream_t)stream;
  if (pick_t(n) == 2) launch_f16_t<2>(w, n, k, x, rows, y, s);
  else launch_f16_t<1>(w, n, k, x, rows, y, s);
  if (int st = launched("gemv_f16_kernel")) return st;
  return ok();
}

int qgemv_q8_0_grouped(const void* w_images, int64_t n_experts, int64_t n, int64_t k, const float* x, int x_rows,
                       const int32_t* expert, const int32_t* x_index, int m, float* y, void* ws, size_t ws_bytes,
                       qg_stream stream) {
  if (n_experts < 1 || n_experts > (1 << 30)) return fail(QG_ESHAPE, "n_experts=%lld", (long long)n_experts);
  if (m < 0 || m > QG_MAX_ASSIGN) return fail(QG_ESHAPE, "m=%d outside 0..%d", m, QG_MAX_ASSIGN);
  // y (and the assignment arrays) may be null when m == 0
  if (int st = check_q8_args(QG_FMT_Q8_0, w_images, n, k, 1, m ? y : (const float*)w_images)) return st;
  if (int st = check_x(x, x_rows, k)) return st;
  if (m && (!expert || !x_index)) return fail(QG_EINVAL, "expert or x_index is null");
  if (!ws) return fail(QG_EINVAL, "ws is null");
  if (!aligned(ws, 256)) return fail(QG_EALIGN, "ws %p is not 256-byte aligned", ws);
  const GroupedLayout G = grouped_layout(x_rows, k, m);
  if (ws_bytes < G.total) return fail(QG_EWORKSPACE, "ws_bytes=%zu < %zu needed", ws_bytes, G.total);
  if (int st = check_device()) return st;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* w = (uint8_t*)ws;
  int* header = (int*)(w + G.header);
  int* sorted = (int*)(w + G.sorted);
  int* items = (int*)(w + G.items);
  if (int st = prepare(x, x_rows, k, w + G.prep, s)) return st;
  hipLaunchKernelGGL(grouped_plan_kernel, dim3(1), dim3(1024), 0, s, expert, x_index, m, n_experts, x_rows, header,
                     sorted, items);
  if (int st = launched("grouped_plan_kernel")) return st;
  if (m == 0) return ok();
  const PrepLayout L = prep_layout(x_rows, k);
  Prep prep;
  prep.codes = (const int8_t*)(w + G.prep + L.codes);
  prep.dx = (const float*)(w + G.prep + L.dx);
  prep.nsx = (const int*)(w + G.prep + L.nsx);
  const int kbp = (int)kbp_of(k);
  const int T = pick_t(n * 8);
  const int rpt = (WG / lanes_per_row(kbp)) * T;
  const unsigned tiles = (unsigned)((n + rpt - 1) / rpt);
  size_t lds = (size_t)QG_MAX_ROWS * kbp * x_block_bytes(FMT_Q8);
  if (lds > (size_t)LDS_MAX) lds = LDS_MAX;
  const int64_t eb = (int64_t)image_total_bytes(QG_FMT_Q8_0, n, k);
  const size_t so = image_scale_offset(QG_FMT_Q8_0, n, k);
  if (T == 2) {
    if (lds > 64 * 1024)
      hipFuncSetAttribute((const void*)qgemv_grouped_kernel<2>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(qgemv_grouped_kernel<2>, dim3(tiles, m), dim3(WG), lds, s, (const uint8_t*)w_images, eb, so, n,
                       kbp, prep, header, sorted, items, x_index, y, (int)lds);
  } else {
    if (lds > 64 * 1024)
      hipFuncSetAttribute((const void*)qgemv_grouped_kernel<1>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(qgemv_grouped_kernel<1>, dim3(tiles, m), dim3(WG), lds, s, (const uint8_t*)w_images, eb, so, n,
                       kbp, prep, header, sorted, items, x_index, y, (int)lds);
  }
  if (int st = launched("qgemv_grouped_kernel")) return st;
  return ok();
}

int qg_grouped_status(const void* ws, int32_t* bad, qg_stream stream) {
  if (!ws || !bad) return fail(QG_EINVAL, "null argument");
  if (int st = check_device()) return st;
  if (int st = hip_status(hipStreamSynchronize((hipStream_t)stream), "hipStreamSynchronize")) return st;
  int32_t h[2];
  if (int st = hip_status(hipMemcpy(h, ws, sizeof h, hipMemcpyDeviceToHost), "hipMemcpy")) return st;
  *bad = h[1];
  return ok();
}

int qg_moe_route(const float* logits, int rows, int n_experts, int topk, int shared_expert, int32_t* expert,
                 int32_t* x_index, float* weight, qg_stream stream) {
  if (!logits || !expert || !x_index || !weight) return fail(QG_EINVAL, "null buffer");
  if (rows < 0 || rows > 65535) return fail(QG_EROWS, "rows=%d outside 0..65535", rows);
  if (n_experts < 1 || n_experts > 1024) return fail(QG_ESHAPE, "n_experts=%d outside 1..1024", n_experts);
  if (topk < 1 || topk > 32 || topk > n_experts) return fail(QG_ESHAPE, "topk=%d outside 1..min(32, n_experts)", topk);
  if (rows == 0) return ok();
  if (int st = check_device()) return st;
  hipLaunchKernelGGL(moe_route_kernel, dim3(rows), dim3(256), 0, (hipStream_t)stream, logits, n_experts, topk,
                     shared_expert, expert, x_index, weight);
  if (int st = launched("moe_route_kernel")) return st;
  return ok();
}

int qg_swiglu(const float* gu, int m, int64_t ffn, float* h, qg_stream stream) {
  if (!gu || !h) return fail(QG_EINVAL, "null buffer");
  if (m < 0 || ffn < 1) return fail(QG_ESHAPE, "m=%d ffn=%lld", m, (long long)ffn);
  if (m == 0) return ok();
  if (int st = check_device()) return st;
  hipLaunchKernelGGL(swiglu_kernel, dim3(grid1((int64_t)m * ffn, 256)), dim3(256), 0, (hipStream_t)stream, gu, m, ffn,
                     h);
  if (int st = launched("swiglu_kernel")) return st;
  return ok();
}

int qg_moe_combine(const float* o, const float* weight, int rows, int slots, int64_t hidden, float* y,
                   qg_stream stream) {
  if (!o || !weight || !y) return fail(QG_EINVAL, "null buffer");
  if (rows < 0 || rows > 65535 || slots < 1 || hidden < 4 || hidden % 4)
    return fail(QG_ESHAPE, "rows=%d slots=%d hidden=%lld (hidden must be a multiple of 4)", rows, slots,
                (long long)hidden);
  if (!aligned(o, 16) || !aligned(y, 16)) return fail(QG_EALIGN, "o and y must be 16-byte aligned");
  if (rows == 0) return ok();
  if (int st = check_device()) return st;
  hipLaunchKernelGGL(moe_combine_kernel, dim3(grid1(hidden / 4, 256), rows), dim3(256), 0, (hipStream_t)stream, o,
                     weight, slots, hidden, y);
  if (int st = launched("moe_combine_kernel")) return st;
  return ok();
}

int qg_quantize_rows_q8(const float* x, int rows, int64_t k, int8_t* qx, float* dx, int32_t* sx, qg_stream stream) {
  if (int st = check_x(x, rows, k)) return st;
  if (!qx || !dx || !sx) return fail(QG_EINVAL, "null output");
  if (!aligned(qx, 16)) return fail(QG_EALIGN, "qx %p is not 16-byte aligned", (const void*)qx);
  if (int st = check_device()) return st;
  const int kb = (int)kb_of(k);
  hipLaunchKernelGGL(quantize_rows_kernel<false>, dim3(grid1((int64_t)rows * kb, 256)), dim3(256), 0,
                     (hipStream_t)stream, x, rows, k, kb, (int)kbp_of(k), qx, dx, sx);
  if (int st = launched("quantize_rows_kernel")) return st;
  return ok();
}

int qgemv_blockdots(int fmt, const void* w_image, int64_t n, int64_t k, const int8_t* qx, int rows, int32_t* isum,
                    qg_stream stream) {
  if (int st = check_q8_args(fmt, w_image, n, k, rows, (const float*)isum)) return st;
  if (!qx) return fail(QG_EINVAL, "qx is null");
  if (!aligned(qx, 16)) return fail(QG_EALIGN, "qx %p is not 16-byte aligned", (const void*)qx);
  if (rows == 0) return ok();
  if (int st = check_device()) return st;
  const int kb = (int)kb_of(k), kbp = (int)kbp_of(k);
  const unsigned g = grid1((int64_t)rows * n * kb, 256);
  if (fmt == QG_FMT_Q8_0)
    hipLaunchKernelGGL(blockdots_kernel<FMT_Q8>, dim3(g), dim3(256), 0, (hipStream_t)stream, (const uint8_t*)w_image,
                       n, kbp, kb, qx, rows, k, isum);
  else
    hipLaunchKernelGGL(blockdots_kernel<FMT_Q4>, dim3(g), dim3(256), 0, (hipStream_t)stream, (const uint8_t*)w_image,
                       n, kbp, kb, qx, rows, k, isum);
  if (int st = launched("blockdots_kernel")) return st;
  return ok();
}

}  // extern "C"
