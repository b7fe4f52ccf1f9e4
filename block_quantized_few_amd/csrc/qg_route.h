// qg_route.h -- routing of a routed MoE decode step (softmax over the router
// logits, the top-k experts) and its plan (the assignments ordered by expert
// into work items of the grouped GEMV), as device code any workgroup can run.
#pragma once
#include <hip/hip_runtime.h>

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

// (va, ia) ahead of (vb, ib): the larger logit, ties to the lower index.
__device__ __forceinline__ void order2(float& va, int& ia, float& vb, int& ib) {
  const bool swap = (vb > va) | ((vb == va) & (ib < ia));
  const float tv = va;
  const int ti = ia;
  va = swap ? vb : va;
  ia = swap ? ib : ia;
  vb = swap ? tv : vb;
  ib = swap ? ti : ib;
}

// Routing of one row by one wave: softmax over the E logits in fp32 (max
// subtracted; each lane sums its experts in index order, then the fixed
// wave_sum tree), and the topk experts by logit, ties to the lower index, in
// descending order, written to ex[] / wt[] (lane k writes pick k).  NPER:
// logits per lane (E <= 64 * NPER).
//
// Selection: each lane orders its own entries once (expert lane + 64 i; past
// E, or a NaN logit, never picked: -inf with an index above every expert's),
// so its best remaining entry is always its first.  A pick is the wave's
// largest first entry; the lanes holding that value are found by ballot, and
// of several (equal logits) the lowest expert index wins.  The winner's lane
// then moves its next entry up.
template <int NPER>
__device__ void route_row_n(const float* __restrict__ lrow, int E, int topk, int* ex, float* wt) {
  const int lane = threadIdx.x & (WAVE - 1);
  float l[NPER];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NPER; i++) {
    const int e = lane + WAVE * i;
    l[i] = e < E ? lrow[e] : -INFINITY;
    mx = fmaxf(mx, l[i]);
  }
  mx = wave_max(mx);
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < NPER; i++) {
    const float t = expf(l[i] - mx);
    sum += lane + WAVE * i < E ? t : 0.0f;
  }
  sum = wave_sum(sum);
  float sv[NPER];
  int si[NPER];
#pragma unroll
  for (int i = 0; i < NPER; i++) {
    const int e = lane + WAVE * i;
    const bool ok = (e < E) & (l[i] == l[i]);
    sv[i] = ok ? l[i] : -INFINITY;
    si[i] = ok ? e : 0x7fffffff;
  }
#pragma unroll
  for (int i = 1; i < NPER; i++)
#pragma unroll
    for (int j = i; j > 0; j--) order2(sv[j - 1], si[j - 1], sv[j], si[j]);
  float mv = 0.0f;  // this lane's pick (lane k: the k-th)
  int mi = 0;
  for (int k = 0; k < topk; k++) {
    const float bv = wave_max(sv[0]);
    const unsigned long long at = __ballot(sv[0] == bv);
    int bi;
    if (__popcll(at) == 1) bi = __builtin_amdgcn_readlane(si[0], (int)__builtin_ctzll(at));
    else bi = wave_min_i(sv[0] == bv ? si[0] : 0x7fffffff);
    if (si[0] == bi) {  // the winner's lane: its next entry first
#pragma unroll
      for (int i = 0; i + 1 < NPER; i++) {
        sv[i] = sv[i + 1];
        si[i] = si[i + 1];
      }
      sv[NPER - 1] = -INFINITY;
      si[NPER - 1] = 0x7fffffff;
    }
    mv = lane == k ? bv : mv;  // lane k keeps pick k
    mi = lane == k ? bi : mi;
  }
  if (lane < topk) {
    ex[lane] = mi;
    wt[lane] = expf(mv - mx) / sum;
  }
}

__device__ __forceinline__ void route_row(const float* __restrict__ lrow, int E, int topk, int* ex, float* wt) {
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
  unsigned* wsum;  // [16] per-wave sums of the scan
  int* items;      // [3 m] (expert, first sorted position, rows)
  int* sorted;     // [m]
  int* xi;         // [m] activation row of assignment j
  int* misc;       // [2] item count, small-item count
};

// Bytes of a plan's LDS (16-byte multiple): e, w, items (3), sorted, xi: 7 m
// words; mask, off: 2 (E + 1); wsum 16; misc 2 (the carve below, in order).
__host__ __device__ constexpr size_t plan_lds_bytes(int m, int E) {
  return ((size_t)(7 * m + 2 * (E + 1) + 16 + 2) * 4 + 15) / 16 * 16;
}

__device__ inline PlanLds plan_carve(uint8_t* p, int m, int E) {
  PlanLds P;
  int* b = reinterpret_cast<int*>(p);
  P.e = b;
  P.w = reinterpret_cast<float*>(b + m);
  P.mask = reinterpret_cast<unsigned*>(b + 2 * m);
  P.off = P.mask + (E + 1);
  P.wsum = P.off + (E + 1);
  P.items = reinterpret_cast<int*>(P.wsum + 16);
  P.sorted = P.items + 3 * m;
  P.xi = P.sorted + m;
  P.misc = P.xi + m;
  return P;
}

// The plan into P (every thread of the workgroup calls it; at most 16 waves;
// rows <= 16, rows * slots <= QG_MOE_MAX_M, E <= ROUTE_MAX_E).  Ends with a
// barrier.
__device__ inline void moe_plan_block(const float* __restrict__ logits, int rows, int E, int topk, bool shared,
                                      const PlanLds& P) {
  const int tid = threadIdx.x, nt = blockDim.x, wave = tid / WAVE, lane = tid % WAVE;
  const int slots = topk + (shared ? 1 : 0), m = rows * slots, ne = E + 1;
  for (int r = wave; r < rows; r += nt / WAVE) {
    route_row(logits + (int64_t)r * E, E, topk, P.e + r * slots, P.w + r * slots);
    if (lane == 0 && shared) {
      P.e[r * slots + topk] = E;
      P.w[r * slots + topk] = 1.0f;
    }
  }
  for (int e = tid; e < ne; e += nt) P.mask[e] = 0u;
  __syncthreads();
  for (int j = tid; j < m; j += nt) atomicOr(&P.mask[P.e[j]], 1u << (j / slots));
  __syncthreads();
  // exclusive scan over experts of their (assignments, touched, small item)
  // counts: thread t takes experts t*c .. t*c + c - 1
  auto val = [](unsigned mk) {
    const unsigned c = __popc(mk);
    return c | (mk ? 1u << 10 : 0u) | (mk && c <= (unsigned)GROUPED_SMALL_ROWS ? 1u << 21 : 0u);
  };
  const int c = (ne + nt - 1) / nt, e0 = tid * c;
  unsigned loc = 0;
  for (int i = 0; i < c; i++)
    if (e0 + i < ne) loc += val(P.mask[e0 + i]);
  unsigned inc = loc;  // inclusive within the wave
  for (int o = 1; o < WAVE; o <<= 1) {
    const unsigned v = __shfl_up(inc, o);
    inc += lane >= o ? v : 0u;
  }
  if (lane == WAVE - 1) P.wsum[wave] = inc;
  __syncthreads();
  unsigned run = 0, total = 0;
  for (int w = 0; w < nt / WAVE; w++) {
    run += w < wave ? P.wsum[w] : 0u;
    total += P.wsum[w];
  }
  run += inc - loc;
  for (int i = 0; i < c; i++)
    if (e0 + i < ne) {
      P.off[e0 + i] = run;
      run += val(P.mask[e0 + i]);
    }
  __syncthreads();
  const int nitems = (int)((total >> 10) & 2047u), nsmall = (int)(total >> 21);
  for (int j = tid; j < m; j += nt) {
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
  if (tid == 0) {
    P.misc[0] = nitems;
    P.misc[1] = nsmall;
  }
  __syncthreads();
}

// The plan's global copies: the step's expert / weight / x_index outputs
// (expert E is the shared one), and the grouped GEMV's header, sorted, items.
__device__ inline void plan_store(const PlanLds& P, int m, int32_t* __restrict__ expert, float* __restrict__ weight,
                                  int32_t* __restrict__ x_index, int* __restrict__ header, int* __restrict__ sorted,
                                  int* __restrict__ items) {
  const int tid = threadIdx.x, nt = blockDim.x, ni = P.misc[0];
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
}

}  // namespace qg
