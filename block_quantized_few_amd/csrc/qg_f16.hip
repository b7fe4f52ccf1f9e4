// qg_f16.hip -- the f16 lane: halfword weights, fp32 activations, fp32
// accumulation (the reference lane of the dasLLAMA audio-towers page,
// feature commit), on v_mfma_f32_16x16x32_f16.
//
// Weight image.  The row-major [n][k] halfword matrix is repacked once into
// 16-row tiles of 32-column steps: tile t, step s is one 1 KB block in which
// lane l = i + 16q of a wave finds its 16 bytes at 16*l, the halfwords
// w[16t + i][32s + 8q .. 32s + 8q + 7] -- exactly the A operand the MFMA
// wants from that lane.  A tile's steps follow each other, tiles follow each
// other; rows past n and columns past k are zero.  One wave load of a step is
// then 1 KB of consecutive bytes (row-major weights give 16 rows x 64 bytes
// per load, which the memory system serves markedly slower).
//
// Arithmetic.  A lane (i, q) feeds the MFMA its 8 weights and the same 8 k
// of activation row i; the activation goes in as two halfword terms,
// hi = f16(x * 2^-e) and lo = f16(x * 2^-e - hi), so x * 2^-e = hi + lo to
// about 2^-22 relative, and both terms meet the exact halfword weights in
// fp32.  The power of two 2^-e puts the largest |x| of the wave's k range of
// that row in [2^14, 2^15) (the halfword range); the wave's fp32 sum is scaled
// back by 2^e (exact).  The S waves of a workgroup take S contiguous k ranges,
// added left to right at the end.  A row's result depends on its own
// activations, K and N only, never on the other rows of the call.
#include <hip/hip_runtime.h>

#include "qg_device.h"
#include "qg_internal.h"
#include "qg_launch.h"

namespace qg {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int FM_STEP_HALVES = 512;  // halfwords of one (tile, step) block
constexpr int FM_NT_BIG = 8;         // tiles per step of the kernel on large N
constexpr int FM_LA_BIG = 2;         // and its steps in flight
constexpr int64_t FM_ROT = 7;        // start-step stride between neighbouring tiles

// ------------------------------------------------------------------ pack ---
// One thread per 16-byte chunk of the image.
__global__ void f16_pack_kernel(const uint16_t* __restrict__ w, int64_t N, int64_t K, int64_t ks,
                                uint4* __restrict__ img, int64_t chunks) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= chunks) return;
  const int lane = (int)(c & 63);
  const int64_t blk = c >> 6, t = blk / ks, s = blk - t * ks;
  const int64_t row = 16 * t + (lane & 15), k0 = 32 * s + 8 * (lane >> 4);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row < N && k0 < K) v = *reinterpret_cast<const uint4*>(w + row * K + k0);  // K % 8 == 0
  img[c] = v;
}

int launch_f16_pack(const uint16_t* w, int64_t n, int64_t k, void* image, hipStream_t s) {
  const int64_t ks = f16_steps(k), chunks = f16_tiles(n) * ks * 64;
  const int64_t g = (chunks + 255) / 256;
  hipLaunchKernelGGL(f16_pack_kernel, dim3((unsigned)g), dim3(256), 0, s, w, n, k, ks,
                     reinterpret_cast<uint4*>(image), chunks);
  return hip_status(hipGetLastError(), "f16_pack_kernel");
}

// ------------------------------------------------------------------ GEMV ---
template <int NT>
struct FmStep {
  uint4 a[NT];  // weights of NT 16-row tiles
  float4 x[2];  // 8 activations
};

template <int NT>
__device__ __forceinline__ void fm_load(FmStep<NT>& st, const uint16_t* const (&wt)[NT], const float* xrow,
                                        int64_t kend, int64_t s) {
  const int64_t k0 = s * 32;
  const bool in = k0 < kend;  // kend = K - 8q; K % 8 == 0: the lane's 8 activations are all in or all out
#pragma unroll
  for (int t = 0; t < NT; t++) st.a[t] = ld16_stream(wt[t] + s * FM_STEP_HALVES);  // zero-padded image
  st.x[0] = in ? *reinterpret_cast<const float4*>(xrow + k0) : make_float4(0.f, 0.f, 0.f, 0.f);
  st.x[1] = in ? *reinterpret_cast<const float4*>(xrow + k0 + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
}

template <int NT>
__device__ __forceinline__ void fm_compute(v4f (&c)[NT], const FmStep<NT>& st, float scale) {
  const float v[8] = {st.x[0].x, st.x[0].y, st.x[0].z, st.x[0].w, st.x[1].x, st.x[1].y, st.x[1].z, st.x[1].w};
  v8h hi, lo;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const float sv = v[j] * scale;
    const _Float16 h = (_Float16)sv;
    hi[j] = h;
    lo[j] = (_Float16)(sv - (float)h);
  }
#pragma unroll
  for (int t = 0; t < NT; t++) {
    v8h a;
    __builtin_memcpy(&a, &st.a[t], 16);
    c[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, hi, c[t], 0, 0, 0);
    c[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, lo, c[t], 0, 0, 0);
  }
}

// NT 16-row tiles per workgroup step (a tile group), S waves (k ranges), LA
// steps in flight; the workgroup takes groups first, first + stride, ...
template <int NT, int S, int LA>
__device__ __forceinline__ void gemv_f16_groups(const uint16_t* __restrict__ img, int64_t N, int64_t K,
                                                const float* __restrict__ x, int R, float* __restrict__ y,
                                                int64_t groups, int64_t first, int64_t stride) {
  __shared__ float red[S * NT * 4 * WAVE];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & (WAVE - 1);
  const int i = lane & 15, q = lane >> 4;
  const int64_t ks = (K + 31) / 32, tiles = (N + 15) / 16;
  const int64_t s0 = ks * wave / S, s1 = ks * (wave + 1) / S;  // this wave's k steps
  const int xr = i < R ? i : R - 1;                             // activation row of this lane's column
  const float* xrow = x + (int64_t)xr * K + 8 * q;
  const int64_t kend = K - 8 * q;  // the lane reads k0 + 8q .. k0 + 8q + 7 while k0 < kend
  const int64_t nst = s1 - s0;
  const uint16_t* wt[NT];
  int64_t lc = s0;  // next step to load
  FmStep<NT> f[LA];
  // Points the wave at tile group grp and puts its first LA steps in flight.
  // The wave walks its k range from a group-dependent starting step, wrapping
  // round: groups in flight together then read different k offsets.
  auto start = [&](int64_t grp) {
#pragma unroll
    for (int t = 0; t < NT; t++) {
      const int64_t tt = grp * NT + t;
      wt[t] = img + (tt < tiles ? tt : tiles - 1) * ks * FM_STEP_HALVES + 8 * lane;  // past the end: reread
    }
    lc = s0 + (nst ? (grp * FM_ROT) % nst : 0);
#pragma unroll
    for (int j = 0; j < LA; j++)
      if (j < nst) {
        fm_load<NT>(f[j], wt, xrow, kend, lc);
        lc = lc + 1 == s1 ? s0 : lc + 1;
      }
  };
  if (first < groups) start(first);

  // the scale of this column over the wave's k range (from the steps in flight
  // when they cover it, else from a pass of its own)
  auto amax8 = [](float4 a, float4 b) {
    return fmaxf(fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))),
                 fmaxf(fmaxf(fabsf(b.x), fabsf(b.y)), fmaxf(fabsf(b.z), fabsf(b.w))));
  };
  float amax = 0.0f;
  if (nst <= LA && first < groups) {
#pragma unroll
    for (int j = 0; j < LA; j++)
      if (j < nst) amax = fmaxf(amax, amax8(f[j].x[0], f[j].x[1]));  // zeros past k
  } else {
    for (int64_t st = s0; st < s1; st++) {
      const int64_t k0 = st * 32;
      if (k0 < kend)
        amax = fmaxf(amax, amax8(*reinterpret_cast<const float4*>(xrow + k0),
                                 *reinterpret_cast<const float4*>(xrow + k0 + 4)));
    }
  }
  amax = fmaxf(amax, __shfl_xor(amax, 16));
  amax = fmaxf(amax, __shfl_xor(amax, 32));
  int ex = 0;
  if (amax > 0.0f) frexpf(amax, &ex);  // amax in [2^(ex-1), 2^ex)
  const int se = min(max(15 - ex, -126), 126);
  const float scale = ldexpf(1.0f, se);

  for (int64_t grp = first; grp < groups; grp += stride) {
    v4f c[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) c[t] = (v4f){0.f, 0.f, 0.f, 0.f};
    for (int64_t st = 0; st < nst; st += LA) {
#pragma unroll
      for (int j = 0; j < LA; j++) {
        if (st + j < nst) {
          fm_compute<NT>(c, f[j], scale);
          if (st + j + LA < nst) {
            fm_load<NT>(f[j], wt, xrow, kend, lc);
            lc = lc + 1 == s1 ? s0 : lc + 1;
          }
        }
      }
    }
    // every step is consumed: the next group's first loads fly during the reduction
    if (grp + stride < groups) start(grp + stride);
    // k ranges left to right (each scaled back first)
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; t++)
#pragma unroll
      for (int v = 0; v < 4; v++) red[((wave * NT + t) * 4 + v) * WAVE + lane] = ldexpf(c[t][v], -se);
    __syncthreads();
    if (wave == 0 && i < R) {
#pragma unroll
      for (int t = 0; t < NT; t++)
#pragma unroll
        for (int v = 0; v < 4; v++) {
          float acc = red[(t * 4 + v) * WAVE + lane];
          for (int s2 = 1; s2 < S; s2++) acc += red[((s2 * NT + t) * 4 + v) * WAVE + lane];
          const int64_t row = (grp * NT + t) * 16 + 4 * q + v;
          if (row < N) y[(int64_t)i * N + row] = acc;
        }
    }
  }
}

// Persistent over tile groups.
template <int NT, int S, int LA>
__global__ __launch_bounds__(S * WAVE) void gemv_f16_kernel(const uint16_t* __restrict__ img, int64_t N, int64_t K,
                                                            const float* __restrict__ x, int R,
                                                            float* __restrict__ y, int64_t groups) {
  gemv_f16_groups<NT, S, LA>(img, N, K, x, R, y, groups, blockIdx.x, gridDim.x);
}

template <int NT, int S, int LA>
static void launch_f16(const uint16_t* img, int64_t n, int64_t k, const float* x, int rows, float* y, hipStream_t s) {
  auto kern = gemv_f16_kernel<NT, S, LA>;
  const int64_t groups = (f16_tiles(n) + NT - 1) / NT;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, S * WAVE, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  const int64_t g = (int64_t)device_cus() * per_cu;
  hipLaunchKernelGGL(kern, dim3((unsigned)(groups < g ? groups : g)), dim3(S * WAVE), 0, s, img, n, k, x, rows, y,
                     groups);
}

int launch_gemv_f16(const void* image, int64_t n, int64_t k, const float* x, int rows, float* y, hipStream_t s) {
  const uint16_t* img = static_cast<const uint16_t*>(image);
  const int64_t t16 = f16_tiles(n);
  // few tiles: more waves per tile (shorter k ranges) to keep loads in flight
  if (t16 >= 4096) launch_f16<FM_NT_BIG, 4, FM_LA_BIG>(img, n, k, x, rows, y, s);
  else if (t16 >= 256) launch_f16<1, 4, 4>(img, n, k, x, rows, y, s);
  else launch_f16<1, 16, 4>(img, n, k, x, rows, y, s);
  return hip_status(hipGetLastError(), "gemv_f16_kernel");
}

// The router of a routed MoE step: workgroups 0 .. gemv_wgs - 1 run the f16
// GEMV of the router image (n < 4096 rows: the 16-wave form launch_gemv_f16
// takes for that size, so the logits have its bits); the others quantize the
// input rows (A1, row order) for the expert GEMVs.
__global__ __launch_bounds__(16 * WAVE) void moe_router_kernel(const uint16_t* __restrict__ img, int64_t N, int64_t K,
                                                               const float* __restrict__ x, int R,
                                                               float* __restrict__ y, int64_t groups, int gemv_wgs,
                                                               int8_t* __restrict__ xq, float* __restrict__ xd,
                                                               int* __restrict__ xn, uint8_t* __restrict__ fcodes,
                                                               float* __restrict__ fscales) {
  if ((int)blockIdx.x < gemv_wgs) {
    gemv_f16_groups<1, 16, 4>(img, N, K, x, R, y, groups, blockIdx.x, gemv_wgs);
    return;
  }
  if (fcodes) plan_prepare_fp8(x, R, K, fcodes, fscales, (int)blockIdx.x - gemv_wgs);
  else plan_prepare_q8(x, R, K, xq, xd, xn, (int)blockIdx.x - gemv_wgs);
}

int launch_moe_router(const void* image, int64_t n, int64_t k, const float* x, int rows, float* y, void* xprep,
                      hipStream_t s, bool fp8) {
  const int64_t groups = f16_tiles(n);
  if (groups >= 256) return fail(QG_ELAUNCH, "router of %lld experts: at most 4095", (long long)n);
  uint8_t* w = static_cast<uint8_t*>(xprep);
  int8_t* xq = nullptr;
  float* xd = nullptr;
  int* xn = nullptr;
  uint8_t* fc = nullptr;
  float* fs = nullptr;
  // threads of the A1 workgroups: four a 32-block, or (FP8) a wave a 1 x 128 group
  int64_t quads;
  if (fp8) {
    fc = w;
    fs = reinterpret_cast<float*>(w + fp8_ws_scale_offset(rows, k));
    quads = (int64_t)rows * (k / 128) * WAVE;
  } else {
    const PrepLayout L = prep_layout_rows(rows, k);
    xq = reinterpret_cast<int8_t*>(w + L.codes);
    xd = reinterpret_cast<float*>(w + L.dx);
    xn = reinterpret_cast<int*>(w + L.nsx);
    quads = (int64_t)rows * kbp_of(k) * 4;
  }
  const unsigned a1 = (unsigned)((quads + 1023) / 1024);
  hipLaunchKernelGGL(moe_router_kernel, dim3((unsigned)groups + a1), dim3(16 * WAVE), 0, s,
                     static_cast<const uint16_t*>(image), n, k, x, rows, y, groups, (int)groups, xq, xd, xn, fc, fs);
  return hip_status(hipGetLastError(), "moe_router_kernel");
}

}  // namespace qg
