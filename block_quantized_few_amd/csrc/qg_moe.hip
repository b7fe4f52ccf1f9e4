// qg_moe.hip -- glue of a routed MoE decode step around the grouped GEMV:
// softmax top-k routing, SwiGLU, and the weighted combine.
#include <hip/hip_runtime.h>

#include "qg_device.h"
#include "qg_internal.h"
#include "qg_launch.h"
#include "qg_route.h"

namespace qg {

// One wave per row.
__global__ __launch_bounds__(64) void moe_route_kernel(const float* __restrict__ logits, int E, int topk,
                                                       int shared_expert, int32_t* __restrict__ expert,
                                                       int32_t* __restrict__ x_index, float* __restrict__ weight) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const int slots = topk + (shared_expert >= 0 ? 1 : 0);
  int ex;
  float wt;
  route_row(logits + (int64_t)r * E, E, topk, ex, wt);  // lane k < topk: pick k
  if (lane < slots) {
    const bool sh = lane == topk;
    expert[(int64_t)r * slots + lane] = sh ? shared_expert : ex;
    x_index[(int64_t)r * slots + lane] = r;
    weight[(int64_t)r * slots + lane] = sh ? 1.0f : wt;
  }
}

static_assert(QG_MAX_ROWS <= 1024 / WAVE, "the plan launch routes a row a wave");

// The plan of a routed MoE step, one workgroup (moe_plan_block): route every
// row, order the assignments by expert into work items (the grouped GEMV's
// plan; the down projection reuses it).  Workgroups 1.. quantize the input
// rows into row order (A1) meanwhile.
__global__ __launch_bounds__(1024) void moe_plan_kernel(const float* __restrict__ logits, int rows, int E, int topk,
                                                        int shared_expert, int32_t* __restrict__ expert,
                                                        float* __restrict__ weight, int32_t* __restrict__ x_index,
                                                        int* __restrict__ header,
                                                        int* __restrict__ sorted, int* __restrict__ items,
                                                        const float* __restrict__ x, int64_t k, int8_t* __restrict__ xq,
                                                        float* __restrict__ xd, int* __restrict__ xn,
                                                        uint8_t* __restrict__ fcodes, float* __restrict__ fscales) {
  __shared__ __align__(16) uint8_t s_plan[plan_lds_bytes(QG_MOE_MAX_M, ROUTE_MAX_E)];
  if (blockIdx.x > 0) {
    if (fcodes) plan_prepare_fp8(x, rows, k, fcodes, fscales, blockIdx.x - 1);
    else plan_prepare_q8(x, rows, k, xq, xd, xn, blockIdx.x - 1);
    return;
  }
  const int slots = topk + (shared_expert >= 0 ? 1 : 0), m = rows * slots;
  const PlanLds P = plan_carve(s_plan, m, E);
  moe_plan_block<1024>(logits, rows, E, topk, shared_expert >= 0, P);
  plan_store<1024>(P, m, expert, weight, x_index, header, sorted, items);
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
constexpr int COMBINE_WG = 128;
constexpr int COMBINE_BATCH = 16;  // slots whose loads are issued together

__global__ __launch_bounds__(COMBINE_WG) void moe_combine_kernel(const float* __restrict__ o,
                                                                 const float* __restrict__ weight, int slots,
                                                                 int64_t hidden, float* __restrict__ y) {
  const int r = blockIdx.y;
  const int64_t i4 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i4 * 4 >= hidden) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // slots in order; each batch's loads issued together (a slot past the end
  // re-reads the last one and is not used)
  constexpr int B = COMBINE_BATCH;
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
  hipLaunchKernelGGL(moe_combine_kernel, dim3(grid1(hidden / 4, COMBINE_WG), rows), dim3(COMBINE_WG), 0, s, o, weight,
                     slots, hidden, y);
  return hip_status(hipGetLastError(), "moe_combine_kernel");
}

}  // namespace qg
