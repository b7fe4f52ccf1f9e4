// qg_moe.hip -- glue of a routed MoE decode step around the grouped GEMV:
// softmax top-k routing, SwiGLU, and the weighted combine.
#include <hip/hip_runtime.h>

#include "qg_device.h"
#include "qg_internal.h"
#include "qg_launch.h"

namespace qg {

constexpr int ROUTE_MAX_E = 1024;
constexpr int ROUTE_PER_LANE = ROUTE_MAX_E / WAVE;

// One wave per row.  Softmax over all experts in double (max subtracted; each
// lane sums its experts in order, then a fixed butterfly), and the topk
// experts by logit, ties to the lower index, in descending order.
__global__ __launch_bounds__(64) void moe_route_kernel(const float* __restrict__ logits, int E, int topk,
                                                       int shared_expert, int32_t* __restrict__ expert,
                                                       int32_t* __restrict__ x_index, float* __restrict__ weight) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const int slots = topk + (shared_expert >= 0 ? 1 : 0);
  float l[ROUTE_PER_LANE];
  double mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < ROUTE_PER_LANE; i++) {
    const int e = lane + WAVE * i;
    l[i] = e < E ? logits[(int64_t)r * E + e] : -INFINITY;
    mx = fmax(mx, (double)l[i]);
  }
  for (int off = 32; off > 0; off >>= 1) mx = fmax(mx, __shfl_xor(mx, off));
  double sum = 0.0;
#pragma unroll
  for (int i = 0; i < ROUTE_PER_LANE; i++)
    if (lane + WAVE * i < E) sum += exp((double)l[i] - mx);
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  unsigned taken = 0;
  for (int k = 0; k < topk; k++) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < ROUTE_PER_LANE; i++) {
      const int e = lane + WAVE * i;
      if (e < E && !(taken >> i & 1u) && (l[i] > bv || (l[i] == bv && e < bi))) {
        bv = l[i];
        bi = e;
      }
    }
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (bi % WAVE == lane) taken |= 1u << (bi / WAVE);
    if (lane == 0) {
      expert[(int64_t)r * slots + k] = bi;
      x_index[(int64_t)r * slots + k] = r;
      weight[(int64_t)r * slots + k] = (float)(exp((double)bv - mx) / sum);
    }
  }
  if (lane == 0 && shared_expert >= 0) {
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
// over the slots in order (the combine of the TensorFold drama page keeps each
// sum's order the same way).
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

static unsigned grid1(int64_t threads, int per) { return (unsigned)((threads + per - 1) / per); }

int launch_moe_route(const float* logits, int rows, int n_experts, int topk, int shared_expert, int32_t* expert,
                     int32_t* x_index, float* weight, hipStream_t s) {
  hipLaunchKernelGGL(moe_route_kernel, dim3(rows), dim3(64), 0, s, logits, n_experts, topk, shared_expert, expert,
                     x_index, weight);
  return hip_status(hipGetLastError(), "moe_route_kernel");
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
