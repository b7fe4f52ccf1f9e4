// qg_moe.hip -- glue of a routed MoE decode step around the grouped GEMV:
// softmax top-k routing, SwiGLU, and the weighted combine.
#include <hip/hip_runtime.h>

#include "qg_device.h"
#include "qg_internal.h"
#include "qg_launch.h"

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

// (value, index) with the larger value, ties to the lower index (selects,
// no branches).
__device__ __forceinline__ void pick(float& v, int& i, float ov, int oi) {
  const bool better = (ov > v) | ((ov == v) & (oi < i));
  v = better ? ov : v;
  i = better ? oi : i;
}
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
  pick(v, i, dpp_f<CTRL>(v), dpp_i<CTRL>(i));
}
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_step<0xB1>(v, i);
  argmax_step<0x4E>(v, i);
  argmax_step<0x141>(v, i);
  argmax_step<0x140>(v, i);
  float v0 = lane_f(v, 0), v2 = lane_f(v, 32);
  int i0 = __builtin_amdgcn_readlane(i, 0), i2 = __builtin_amdgcn_readlane(i, 32);
  pick(v0, i0, lane_f(v, 16), __builtin_amdgcn_readlane(i, 16));
  pick(v2, i2, lane_f(v, 48), __builtin_amdgcn_readlane(i, 48));
  pick(v0, i0, v2, i2);
  v = v0;
  i = i0;
}

// Routing of one row by one wave: softmax over the E logits in fp32 (max
// subtracted; each lane sums its experts in index order, then the fixed
// wave_sum tree), and the topk experts by logit, ties to the lower index, in
// descending order, written to ex[] / wt[] (lane k writes pick k).  NPER:
// logits per lane (E <= 64 * NPER).
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
  float mv = 0.0f;  // this lane's pick (lane k: the k-th)
  int mi = 0;
  unsigned avail = 0;  // bit i: entry i is a real expert not picked yet
#pragma unroll
  for (int i = 0; i < NPER; i++) avail |= (lane + WAVE * i < E ? 1u : 0u) << i;
  for (int k = 0; k < topk; k++) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NPER; i++) {
      const int e = lane + WAVE * i;
      const bool ok = (avail >> i) & 1u;
      const bool better = ok & ((l[i] > bv) | ((l[i] == bv) & (e < bi)));
      bv = better ? l[i] : bv;
      bi = better ? e : bi;
    }
    wave_argmax(bv, bi);
    avail &= ~((bi % WAVE == lane ? 1u : 0u) << (bi / WAVE));
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

// One wave per row.
__global__ __launch_bounds__(64) void moe_route_kernel(const float* __restrict__ logits, int E, int topk,
                                                       int shared_expert, int32_t* __restrict__ expert,
                                                       int32_t* __restrict__ x_index, float* __restrict__ weight) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const int slots = topk + (shared_expert >= 0 ? 1 : 0);
  __shared__ int s_ex[32];
  __shared__ float s_wt[32];
  route_row(logits + (int64_t)r * E, E, topk, s_ex, s_wt);
  if (lane < slots) {
    const bool sh = lane == topk;
    expert[(int64_t)r * slots + lane] = sh ? shared_expert : s_ex[lane];
    x_index[(int64_t)r * slots + lane] = r;
    weight[(int64_t)r * slots + lane] = sh ? 1.0f : s_wt[lane];
  }
}

// The plan of a routed MoE step, one workgroup: route every row (a wave per
// row), then order the assignments by (expert, index) into work items of at
// most 16 rows of one expert (the grouped GEMV's plan; the down projection
// reuses it).  Workgroups 1.. quantize the input rows into row order (A1)
// meanwhile.
__global__ __launch_bounds__(1024) void moe_plan_kernel(const float* __restrict__ logits, int rows, int E, int topk,
                                                        int shared_expert, int32_t* __restrict__ expert,
                                                        float* __restrict__ weight, int32_t* __restrict__ x_index,
                                                        int* __restrict__ header,
                                                        int* __restrict__ sorted, int* __restrict__ items,
                                                        const float* __restrict__ x, int64_t k, int8_t* __restrict__ xq,
                                                        float* __restrict__ xd, int* __restrict__ xn,
                                                        uint8_t* __restrict__ fcodes, float* __restrict__ fscales) {
  __shared__ int s_e[QG_MOE_MAX_M];
  __shared__ int s_pos[QG_MOE_MAX_M];
  __shared__ float s_w[QG_MOE_MAX_M];
  __shared__ int s_ie[QG_MOE_MAX_M], s_is[QG_MOE_MAX_M], s_ic[QG_MOE_MAX_M];  // work items
  __shared__ unsigned s_mask[ROUTE_MAX_E + 1];  // bit r: row r picked expert e
  __shared__ int s_off[ROUTE_MAX_E + 1];        // (assignments, touched experts) before expert e, packed
  __shared__ int s_wsum[1024 / WAVE];
  __shared__ int s_cnt[2];
  const int tid = threadIdx.x, nt = blockDim.x, wave = tid / WAVE, lane = tid % WAVE;
  if (blockIdx.x > 0) {
    if (fcodes) plan_prepare_fp8(x, rows, k, fcodes, fscales);
    else plan_prepare_q8(x, rows, k, xq, xd, xn);
    return;
  }
  // workgroup 0: routing and the plan
  const int slots = topk + (shared_expert >= 0 ? 1 : 0);
  const int m = rows * slots;
  for (int r = wave; r < rows; r += nt / WAVE) {
    route_row(logits + (int64_t)r * E, E, topk, s_e + r * slots, s_w + r * slots);
    if (lane == 0 && shared_expert >= 0) {
      s_e[r * slots + topk] = shared_expert;
      s_w[r * slots + topk] = 1.0f;
    }
  }
  // Counting sort by expert.  An expert meets a row at most once (distinct
  // top-k picks; the shared expert is index E), so with rows <= 16 every
  // touched expert is one work item, and an assignment's place among its
  // expert's is the number of earlier rows in the expert's row mask.
  const int ne = E + 1;  // experts 0..E-1 and the shared expert E
  for (int e = tid; e < ne; e += nt) s_mask[e] = 0u;
  __syncthreads();
  for (int j = tid; j < m; j += nt) atomicOr(&s_mask[s_e[j]], 1u << (j / slots));
  __syncthreads();
  // exclusive scan over experts of (count | touched << 16), two experts per thread
  const int e0 = 2 * tid, e1 = e0 + 1;
  const unsigned m0 = e0 < ne ? s_mask[e0] : 0u, m1 = e1 < ne ? s_mask[e1] : 0u;
  const int v0 = __popc(m0) | (m0 ? 1 << 16 : 0), v1 = __popc(m1) | (m1 ? 1 << 16 : 0);
  int inc = v0 + v1;  // inclusive scan within the wave
  for (int off = 1; off < WAVE; off <<= 1) {
    const int o = __shfl_up(inc, off);
    inc += lane >= off ? o : 0;
  }
  if (lane == WAVE - 1) s_wsum[wave] = inc;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; w++) base += s_wsum[w];
  const int ex0 = base + inc - (v0 + v1);  // before expert e0
  if (e0 < ne) s_off[e0] = ex0;
  if (e1 < ne) s_off[e1] = ex0 + v0;
  __syncthreads();
  int nitems = 0;
  for (int w = 0; w < nt / WAVE; w++) nitems += s_wsum[w];
  nitems >>= 16;
  for (int j = tid; j < m; j += nt) {
    const int e = s_e[j], r = j / slots;
    const unsigned mk = s_mask[e];
    const int rank = (s_off[e] & 0xffff) + __popc(mk & ((1u << r) - 1u));
    expert[j] = e;
    weight[j] = s_w[j];
    x_index[j] = r;
    sorted[rank] = j;
    if (mk & ((1u << r) - 1u)) continue;  // the expert's first row makes its item
    const int item = s_off[e] >> 16;
    s_ie[item] = e;
    s_is[item] = s_off[e] & 0xffff;
    s_ic[item] = __popc(mk);
  }
  if (tid == 0) header[1] = 0;
  __syncthreads();
  store_items_small_first(s_ie, s_is, s_ic, nitems, s_pos, s_cnt, items, header);
}

// SwiGLU of m assignments, h = silu(g) * u in fp32, quantized at once into
// row order (m rows of ffn) for the down projection: four lanes per 32-block.
__global__ __launch_bounds__(256) void swiglu_q8_kernel(const float* __restrict__ gu, int m, int64_t ffn, int kbp,
                                                        int8_t* __restrict__ hq, float* __restrict__ hd,
                                                        int* __restrict__ hn) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = t >> 2;
  const int q = (int)(t & 3);
  const bool active = blk < (int64_t)m * kbp;  // whole quads are active or not
  const int64_t j = active ? blk / kbp : 0, b = active ? blk % kbp : 0;
  float v[8];
  if (active && b < ffn / QK) {
    const float* g = gu + j * 2 * ffn + b * QK + q * 8;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float gv = g[i], uv = g[ffn + i];
      v[i] = gv / (1.0f + expf(-gv)) * uv;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = 0.0f;
  }
  unsigned lo, hi;
  float d;
  int sum;
  quantize_quarter(v, lo, hi, d, sum);
  if (!active) return;
  *reinterpret_cast<uint2*>(hq + (j * kbp + b) * 32 + q * 8) = make_uint2(lo, hi);
  if (q == 0) {
    hd[j * kbp + b] = d;
    hn[j * kbp + b] = -8 * sum;
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

// A thread owns four neighbouring outputs of a row and reads them as one
// float4 per slot; it adds the slots strictly in slot order, so the result
// does not depend on how the loads are grouped (the drama page, series
// commits: its combine kernel was widened without changing any sum's order).
__global__ __launch_bounds__(256) void moe_combine_kernel(const float* __restrict__ o,
                                                          const float* __restrict__ weight, int slots,
                                                          int64_t hidden, float* __restrict__ y) {
  const int r = blockIdx.y;
  const int64_t i4 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i4 * 4 >= hidden) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // slots in order; each group of eight slots' loads issued together (a slot
  // past the end re-reads the last one and is not used)
  constexpr int B = 8;
  for (int s0 = 0; s0 < slots; s0 += B) {
    float wgt[B];
    float4 v[B];
#pragma unroll
    for (int j = 0; j < B; j++) {
      const int s = s0 + j < slots ? s0 + j : slots - 1;
      wgt[j] = weight[(int64_t)r * slots + s];
      v[j] = reinterpret_cast<const float4*>(o + ((int64_t)r * slots + s) * hidden)[i4];
    }
#pragma unroll
    for (int j = 0; j < B; j++) {
      if (s0 + j < slots) {
        acc.x = __builtin_fmaf(wgt[j], v[j].x, acc.x);
        acc.y = __builtin_fmaf(wgt[j], v[j].y, acc.y);
        acc.z = __builtin_fmaf(wgt[j], v[j].z, acc.z);
        acc.w = __builtin_fmaf(wgt[j], v[j].w, acc.w);
      }
    }
  }
  reinterpret_cast<float4*>(y + (int64_t)r * hidden)[i4] = acc;
}

static unsigned grid1(int64_t threads, int per) { return (unsigned)((threads + per - 1) / per); }

int launch_moe_route(const float* logits, int rows, int n_experts, int topk, int shared_expert, int32_t* expert,
                     int32_t* x_index, float* weight, hipStream_t s) {
  hipLaunchKernelGGL(moe_route_kernel, dim3(rows), dim3(64), 0, s, logits, n_experts, topk, shared_expert, expert,
                     x_index, weight);
  return hip_status(hipGetLastError(), "moe_route_kernel");
}

int launch_moe_plan(const float* logits, int rows, int n_experts, int topk, int shared_expert, int32_t* expert,
                    float* weight, int32_t* x_index, int* header, int* sorted, int* items, const float* x, int64_t k,
                    void* xprep, bool fp8, hipStream_t s) {
  // x null: routing and the plan only (one workgroup); else the input rows'
  // A1 (or, fp8, their FP8 groups into the FP8 workspace) on workgroups 1..
  const int64_t quads = x ? (fp8 ? (int64_t)rows * (k / 128) * WAVE : (int64_t)rows * kbp_of(k) * 4) : 0;
  int8_t* xq = nullptr;
  float* xd = nullptr;
  int* xn = nullptr;
  uint8_t* fc = nullptr;
  float* fs = nullptr;
  if (x && fp8) {
    fc = (uint8_t*)xprep;
    fs = (float*)(fc + fp8_ws_scale_offset(rows, k));
  } else if (x) {
    const PrepLayout L = prep_layout_rows(rows, k);
    uint8_t* w = (uint8_t*)xprep;
    xq = (int8_t*)(w + L.codes);
    xd = (float*)(w + L.dx);
    xn = (int*)(w + L.nsx);
  }
  hipLaunchKernelGGL(moe_plan_kernel, dim3(1 + (unsigned)((quads + 1023) / 1024)), dim3(1024), 0, s, logits, rows,
                     n_experts, topk, shared_expert, expert, weight, x_index, header, sorted, items, x, k, xq, xd, xn,
                     fc, fs);
  return hip_status(hipGetLastError(), "moe_plan_kernel");
}

int launch_swiglu_q8(const float* gu, int m, int64_t ffn, void* hprep, hipStream_t s) {
  const PrepLayout L = prep_layout_rows(m, ffn);
  uint8_t* w = (uint8_t*)hprep;
  const int kbp = (int)kbp_of(ffn);
  hipLaunchKernelGGL(swiglu_q8_kernel, dim3(grid1((int64_t)m * kbp * 4, 256)), dim3(256), 0, s, gu, m, ffn, kbp,
                     (int8_t*)(w + L.codes), (float*)(w + L.dx), (int*)(w + L.nsx));
  return hip_status(hipGetLastError(), "swiglu_q8_kernel");
}

int launch_swiglu(const float* gu, int m, int64_t ffn, float* h, hipStream_t s) {
  hipLaunchKernelGGL(swiglu_kernel, dim3(grid1((int64_t)m * ffn, 256)), dim3(256), 0, s, gu, m, ffn, h);
  return hip_status(hipGetLastError(), "swiglu_kernel");
}

int launch_moe_combine(const float* o, const float* weight, int rows, int slots, int64_t hidden, float* y,
                       hipStream_t s) {
  hipLaunchKernelGGL(moe_combine_kernel, dim3(grid1(hidden / 4, 256), rows), dim3(256), 0, s, o, weight, slots, hidden,
                     y);
  return hip_status(hipGetLastError(), "moe_combine_kernel");
}

}  // namespace qg
