// qg_route.h -- routing of a routed MoE decode step (softmax over the router
// logits, the top-k experts) and its plan (the assignments ordered by expert
// into work items of the grouped GEMV), as device code any workgroup can run.
#pragma once
#include <hip/hip_runtime.h>

#include <climits>

#include "qg_device.h"

namespace qg {

constexpr int ROUTE_MAX_E = 1024;
constexpr int ROUTE_PER_LANE = ROUTE_MAX_E / WAVE;

// Wave-wide reductions without LDS: DPP within each row of 16 lanes (pairs,
// quads, half-row mirror, row mirror: every lane of the row ends with the
// row's value), then the four rows' values read from lanes 0, 16, 32, 48 and
// combined as (r0 . r1) . (r2 . r3).  Every lane gets the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, dpp_i<0xB1>(v));
  v = min(v, dpp_i<0x4E>(v));
  v = min(v, dpp_i<0x141>(v));
  v = min(v, dpp_i<0x140>(v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

__device__ __forceinline__ int wave_max_i(int v) {
  v = max(v, dpp_i<0xB1>(v));
  v = max(v, dpp_i<0x4E>(v));
  v = max(v, dpp_i<0x141>(v));
  v = max(v, dpp_i<0x140>(v));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Inclusive sum over the lanes: within each row of 16 by shifts of 1, 2, 4
// and 8 lanes (lanes shifted in from before the row read 0), then each row
// adds the totals of the rows before it.
__device__ __forceinline__ unsigned wave_scan_u(unsigned v) {
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);
  v += (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);
  const unsigned r0 = (unsigned)__builtin_amdgcn_readlane((int)v, 15);
  const unsigned r1 = (unsigned)__builtin_amdgcn_readlane((int)v, 31);
  const unsigned r2 = (unsigned)__builtin_amdgcn_readlane((int)v, 47);
  const int row = (threadIdx.x & (WAVE - 1)) >> 4;
  return v + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// A logit as a signed integer of the same order (-0 taken as +0, so equal
// logits have equal keys; a NaN never gets here), and back.
__device__ __forceinline__ int logit_key(float v) {
  const int b = __float_as_int(v + 0.0f);
  return b ^ ((b >> 31) & 0x7fffffff);
}
__device__ __forceinline__ float key_logit(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7fffffff)); }

// (ka, ia) ahead of (kb, ib): the larger key, ties to the lower index.
__device__ __forceinline__ void order2(int& ka, int& ia, int& kb, int& ib) {
  const bool swap = (kb > ka) | ((kb == ka) & (ib < ia));
  const int tk = ka, ti = ia;
  ka = swap ? kb : ka;
  ia = swap ? ib : ia;
  kb = swap ? tk : kb;
  ib = swap ? ti : ib;
}

// Routing of one row by one wave: softmax over the E logits in fp32 (max
// subtracted; each lane sums its experts in index order, then the fixed
// wave_sum tree), and the topk experts by logit, ties to the lower index, in
// descending order: lane k < topk gets pick k.  NPER: logits per lane
// (E <= 64 * NPER); route_load issues the row's loads, route_pick the rest.
//
// Selection on integer keys of the logits (logit_key): each lane orders its
// own entries once (expert lane + 64 i; a NaN logit ranks as -inf with its own
// index, so a row of NaN picks experts 0, 1, ...; past E: -inf with an index
// above every expert's, never picked as topk <= E), so its best remaining
// entry is always its first.  A pick is the wave's largest first key; the
// lanes holding it are found by ballot, and of several (equal logits) the
// lowest expert index wins.  The winner's lane then moves its next entry up.
template <int NPER>
__device__ __forceinline__ void route_load(const float* __restrict__ lrow, int E, float (&l)[NPER]) {
  const int lane = threadIdx.x & (WAVE - 1);
#pragma unroll
  for (int i = 0; i < NPER; i++) {
    const int e = lane + WAVE * i;
    l[i] = e < E ? lrow[e] : -INFINITY;
  }
}

template <int NPER>
__device__ __forceinline__ void route_pick(const float (&l)[NPER], int E, int topk, int& ex, float& wt) {
  const int lane = threadIdx.x & (WAVE - 1);
  int sk[NPER], si[NPER];
  int kmax = INT_MIN;
#pragma unroll
  for (int i = 0; i < NPER; i++) {
    const int e = lane + WAVE * i;
    sk[i] = logit_key((e < E) & (l[i] == l[i]) ? l[i] : -INFINITY);
    si[i] = e < E ? e : 0x7fffffff;
    kmax = max(kmax, sk[i]);
  }
  const float mx = key_logit(wave_max_i(kmax));  // the largest logit (NaN aside)
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < NPER; i++) {
    const float t = expf(l[i] - mx);
    sum += lane + WAVE * i < E ? t : 0.0f;
  }
  sum = wave_sum(sum);
#pragma unroll
  for (int i = 1; i < NPER; i++)
#pragma unroll
    for (int j = i; j > 0; j--) order2(sk[j - 1], si[j - 1], sk[j], si[j]);
  int mk = 0, mi = 0;  // this lane's pick (lane k: the k-th)
  for (int k = 0; k < topk; k++) {
    const int bk = wave_max_i(sk[0]);
    const unsigned long long at = __ballot(sk[0] == bk);
    int bi;
    if (__popcll(at) == 1) bi = __builtin_amdgcn_readlane(si[0], (int)__builtin_ctzll(at));
    else bi = wave_min_i(sk[0] == bk ? si[0] : 0x7fffffff);
    const bool win = si[0] == bi;  // the winner's lane: its next entry first
#pragma unroll
    for (int i = 0; i + 1 < NPER; i++) {
      sk[i] = win ? sk[i + 1] : sk[i];
      si[i] = win ? si[i + 1] : si[i];
    }
    sk[NPER - 1] = win ? INT_MIN : sk[NPER - 1];
    si[NPER - 1] = win ? 0x7fffffff : si[NPER - 1];
    mk = lane == k ? bk : mk;
    mi = lane == k ? bi : mi;
  }
  ex = mi;
  wt = expf(key_logit(mk) - mx) / sum;
}

template <int NPER>
__device__ __forceinline__ void route_row_n(const float* __restrict__ lrow, int E, int topk, int& ex, float& wt) {
  float l[NPER];
  route_load<NPER>(lrow, E, l);
  route_pick<NPER>(l, E, topk, ex, wt);
}

// lane k < topk: pick k of row lrow
__device__ __forceinline__ void route_row(const float* __restrict__ lrow, int E, int topk, int& ex, float& wt) {
  if (E <= 4 * WAVE) route_row_n<4>(lrow, E, topk, ex, wt);
  else if (E <= 8 * WAVE) route_row_n<8>(lrow, E, topk, ex, wt);
  else route_row_n<ROUTE_PER_LANE>(lrow, E, topk, ex, wt);
}

// ------------------------------------------------------------------ plan ---
//
// The plan of a step of `rows` rows and `slots` = topk (+1 with a shared
// expert) assignments a row: assignment j = r * slots + s is row r's s-th
// pick (the shared expert, index E, last, weight 1).  Work items: one per
// touched expert (an expert meets a row at most once, so with rows <= 16 an
// expert's assignments are one item), those of at most GROUPED_SMALL_ROWS
// rows first, each class by expert index; an item's assignments sit in
// `sorted` from its first position, by row.  Every step is a scan or a
// per-element write, so any workgroup that runs it gets the same plan.
struct PlanLds {
  int* e;          // [m] expert of assignment j
  float* w;        // [m] its weight
  unsigned* mask;  // [E + 1] bit r: row r picked the expert
  unsigned* off;   // [E + 1] before expert e: assignments | touched experts << 10 | small items << 21
  int* items;      // [3 m] (expert, first sorted position, rows)
  int* sorted;     // [m]
  int* xi;         // [m] activation row of assignment j
  int* misc;       // [2] item count, small-item count
};

// Bytes of a plan's LDS (16-byte multiple): e, w, items (3), sorted, xi: 7 m
// words; mask, off: 2 (E + 1); misc 2 (the carve below, in order).
__host__ __device__ constexpr size_t plan_lds_bytes(int m, int E) {
  return ((size_t)(7 * m + 2 * (E + 1) + 2) * 4 + 15) / 16 * 16;
}

__device__ inline PlanLds plan_carve(uint8_t* p, int m, int E) {
  PlanLds P;
  int* b = reinterpret_cast<int*>(p);
  P.e = b;
  P.w = reinterpret_cast<float*>(b + m);
  P.mask = reinterpret_cast<unsigned*>(b + 2 * m);
  P.off = P.mask + (E + 1);
  P.items = reinterpret_cast<int*>(P.off + (E + 1));
  P.sorted = P.items + 3 * m;
  P.xi = P.sorted + m;
  P.misc = P.xi + m;
  return P;
}

// Packed counts of an expert's mask: assignments | touched << 10 | small item << 21.
__device__ __forceinline__ unsigned plan_val(unsigned mk) {
  const unsigned c = __popc(mk);
  return c | (mk ? 1u << 10 : 0u) | (mk && c <= (unsigned)GROUPED_SMALL_ROWS ? 1u << 21 : 0u);
}

// The plan into P (every thread of the NTH-thread workgroup calls it; a row
// a wave: rows <= NTH / 64 <= 16; rows * slots <= QG_MOE_MAX_M,
// E <= ROUTE_MAX_E).  Ends with a barrier.
template <int NTH, int NPER>
__device__ void moe_plan_n(const float* __restrict__ logits, int rows, int E, int topk, bool shared,
                           const PlanLds& P) {
  const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
  const int slots = topk + (shared ? 1 : 0), m = rows * slots, ne = E + 1;
  const bool routes = wave < rows;  // wave r routes row r
  float l[NPER];
  if (routes) route_load<NPER>(logits + (int64_t)wave * E, E, l);
  if (rows == 1) {
    // one row: its slots' experts are distinct, so every item is one
    // assignment (small), at its expert's rank among the slots, found by
    // wave 0 from its own lanes
    if (wave == 0) {
      int ex;
      float wt;
      route_pick<NPER>(l, E, topk, ex, wt);
      const bool sh = lane == topk;
      const int e = lane < topk ? ex : sh ? E : INT_MAX;
      int rank = 0;
      for (int i = 0; i < slots; i++) rank += __builtin_amdgcn_readlane(e, i) < e;
      if (lane < slots) {
        P.e[lane] = e;
        P.w[lane] = sh ? 1.0f : wt;
        P.xi[lane] = 0;
        P.sorted[rank] = lane;
        P.items[3 * rank] = e;
        P.items[3 * rank + 1] = rank;
        P.items[3 * rank + 2] = 1;
      }
      if (lane == 0) {
        P.misc[0] = slots;
        P.misc[1] = slots;
      }
    }
    __syncthreads();
    return;
  }
  for (int e = tid; e < ne; e += NTH) P.mask[e] = 0u;
  __syncthreads();
  if (routes) {
    int ex;
    float wt;
    route_pick<NPER>(l, E, topk, ex, wt);
    if (lane < slots) {  // lane topk: the shared expert
      const bool sh = lane == topk;
      const int e = sh ? E : ex;
      P.e[wave * slots + lane] = e;
      P.w[wave * slots + lane] = sh ? 1.0f : wt;
      atomicOr(&P.mask[e], 1u << wave);
    }
  }
  __syncthreads();
  // exclusive scan over experts of their packed counts, by one wave: lane t
  // takes experts t*c .. t*c + c - 1 (c <= NPER + 1), its masks read at once
  if (wave == 0) {
    constexpr int C = NPER + 1;
    const int c = (ne + WAVE - 1) / WAVE, e0 = lane * c;
    unsigned v[C];
    unsigned loc = 0;
#pragma unroll
    for (int i = 0; i < C; i++) {
      const unsigned mk = P.mask[min(e0 + i, ne - 1)];
      v[i] = (i < c) & (e0 + i < ne) ? plan_val(mk) : 0u;
      loc += v[i];
    }
    const unsigned inc = wave_scan_u(loc);
    unsigned run = inc - loc;
#pragma unroll
    for (int i = 0; i < C; i++)
      if ((i < c) & (e0 + i < ne)) {
        P.off[e0 + i] = run;
        run += v[i];
      }
    if (lane == WAVE - 1) {
      P.misc[0] = (int)((inc >> 10) & 2047u);
      P.misc[1] = (int)(inc >> 21);
    }
  }
  __syncthreads();
  const int nsmall = P.misc[1];
  for (int j = tid; j < m; j += NTH) {
    const int e = P.e[j], r = j / slots;
    const unsigned mk = P.mask[e], o = P.off[e], below = mk & ((1u << r) - 1u);
    const int start = (int)(o & 1023u);
    P.sorted[start + __popc(below)] = j;
    P.xi[j] = r;
    if (below) continue;  // the expert's first row makes its item
    const int cnt = __popc(mk), touched = (int)((o >> 10) & 2047u), small_before = (int)(o >> 21);
    const int dst = cnt <= GROUPED_SMALL_ROWS ? small_before : nsmall + (touched - small_before);
    P.items[3 * dst] = e;
    P.items[3 * dst + 1] = start;
    P.items[3 * dst + 2] = cnt;
  }
  __syncthreads();
}

template <int NTH>
__device__ inline void moe_plan_block(const float* __restrict__ logits, int rows, int E, int topk, bool shared,
                                      const PlanLds& P) {
  if (E <= 4 * WAVE) moe_plan_n<NTH, 4>(logits, rows, E, topk, shared, P);
  else if (E <= 8 * WAVE) moe_plan_n<NTH, 8>(logits, rows, E, topk, shared, P);
  else moe_plan_n<NTH, ROUTE_PER_LANE>(logits, rows, E, topk, shared, P);
}

// The plan's global copies: the step's expert / weight / x_index outputs
// (expert E is the shared one), and the grouped GEMV's header, sorted, items.
// With ditems: the items again, each of c > GROUPED_SMALL_ROWS rows cut into
// ceil(c / 2) items of two rows (the last of c - 2 (ceil(c / 2) - 1)), in item
// order, and their header (count, 0, count: every one small) at dheader, for
// a down launch that quantizes the SwiGLU in its staging.
template <int NTH>
__device__ inline void plan_store(const PlanLds& P, int m, int32_t* __restrict__ expert, float* __restrict__ weight,
                                  int32_t* __restrict__ x_index, int* __restrict__ header, int* __restrict__ sorted,
                                  int* __restrict__ items, int* __restrict__ dheader = nullptr,
                                  int* __restrict__ ditems = nullptr) {
  const int tid = threadIdx.x, nt = NTH, ni = P.misc[0];
  for (int j = tid; j < m; j += nt) {
    expert[j] = P.e[j];
    weight[j] = P.w[j];
    x_index[j] = P.xi[j];
    sorted[j] = P.sorted[j];
  }
  for (int i = tid; i < 3 * ni; i += nt) items[i] = P.items[i];
  if (tid == 0) {
    header[0] = ni;
    header[1] = 0;
    header[2] = P.misc[1];
  }
  if (ditems && tid < WAVE) {  // one wave, 64 items a pass, places by a scan of the pieces
    const int lane = tid;
    int base = 0;
    for (int c0 = 0; c0 < ni; c0 += WAVE) {
      const int i = c0 + lane;
      const int cnt = i < ni ? P.items[3 * i + 2] : 0;
      const unsigned pieces = (unsigned)(cnt + 1) >> 1;
      const unsigned inc = wave_scan_u(pieces);
      if (i < ni) {
        const int e = P.items[3 * i], start = P.items[3 * i + 1];
        int* d = ditems + 3 * (base + (int)(inc - pieces));
        for (int p = 0; p < (int)pieces; p++) {
          d[3 * p] = e;
          d[3 * p + 1] = start + 2 * p;
          d[3 * p + 2] = min(2, cnt - 2 * p);
        }
      }
      base += __builtin_amdgcn_readlane((int)inc, WAVE - 1);
    }
    if (lane == 0) {
      dheader[0] = base;
      dheader[1] = 0;
      dheader[2] = base;
    }
  }
}

}  // namespace qg
