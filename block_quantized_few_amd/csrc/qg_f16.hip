// qg_f16.hip -- the f16 lane: halfword weights, fp32 activations, fp32
// accumulation (the reference lane of the dasLLAMA audio-towers page,
// feature commit).
#include <hip/hip_runtime.h>

#include "qg_device.h"
#include "qg_internal.h"
#include "qg_launch.h"

namespace qg {

constexpr int F16_WG = 256;
constexpr int F16_LPR = 16;                     // lanes per weight row
constexpr int F16_SLOTS = F16_WG / F16_LPR;     // rows per workgroup step
constexpr int F16_LDS = 48 * 1024;              // staged fp32 activation chunk

// Sum over the 16 lanes of a row (pairs, quads, half-rows by mirror, rows by
// mirror); every lane receives the same bits.
__device__ __forceinline__ float sum16(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
  return v;
}

// Lane j of a row's 16 lanes reads 8 halfwords (16 bytes) at j, j+16, ... and
// multiplies them with fp32 activations staged in LDS: one fma per weight and
// row (fp16 -> fp32 conversion is exact), rows kept in fp32.
template <int R, int T>
__global__ __launch_bounds__(F16_WG) void gemv_f16_kernel(const uint16_t* __restrict__ w, int64_t N, int64_t K,
                                                          const float* __restrict__ x, float* __restrict__ y, int ce) {
  extern __shared__ __align__(16) uint8_t lds[];
  float* l_x = reinterpret_cast<float*>(lds);
  const int tid = threadIdx.x;
  const int slot = tid / F16_LPR, j = tid % F16_LPR;
  const int64_t row0 = (int64_t)blockIdx.x * (F16_SLOTS * T);
  int64_t n[T];
  bool valid[T];
  const uint16_t* wrow[T];
#pragma unroll
  for (int t = 0; t < T; t++) {
    n[t] = row0 + (int64_t)(t * F16_SLOTS + slot);
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
    for (int u = tid; u < R * cu; u += F16_WG) {
      const int r = u / cu, c = u - r * cu;
      reinterpret_cast<float4*>(l_x + (size_t)r * ce)[c] = reinterpret_cast<const float4*>(x + r * K + c0)[c];
    }
    __syncthreads();
#pragma unroll 2
    for (int c = j; c * 8 < cen; c += F16_LPR) {
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

template <int R, int T>
static void launch_f16_rt(const uint16_t* w, int64_t n, int64_t k, const float* x, float* y, hipStream_t s) {
  int ce = (F16_LDS / (R * 4)) / 128 * 128;
  if (ce < 128) ce = 128;
  const int64_t kr = (k + 127) / 128 * 128;
  if (ce > kr) ce = (int)kr;
  const unsigned grid = (unsigned)((n + F16_SLOTS * T - 1) / (F16_SLOTS * T));
  hipLaunchKernelGGL((gemv_f16_kernel<R, T>), dim3(grid), dim3(F16_WG), (size_t)R * ce * 4, s, w, n, k, x, y, ce);
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

int launch_gemv_f16(const uint16_t* w, int64_t n, int64_t k, const float* x, int rows, float* y, hipStream_t s) {
  if ((n + 31) / 32 >= 1024) launch_f16_t<2>(w, n, k, x, rows, y, s);
  else launch_f16_t<1>(w, n, k, x, rows, y, s);
  return hip_status(hipGetLastError(), "gemv_f16_kernel");
}

}  // namespace qg
