// qg_fp8.hip -- the FP8 lane: block-FP8 weights and dynamic 1 x 128 FP8
// activation groups (the drama page's backbone section: its MoE experts are
// block-FP8 and its activations are quantized per 1 x 128 group as they are
// produced), on gfx950's v_mfma_scale_f32_16x16x128_f8f6f4.
//
// Formats.  Elements are OCP E4M3 (bias 7, three mantissa bits, largest
// finite 448, round to nearest even, saturating).  A weight block is 128 rows x
// 128 columns with one fp32 scale amax / 448; an activation group is 128
// consecutive columns of one row with its own fp32 scale.  One 16x16x128 MFMA
// covers exactly one group: its fp32 result for (weight row, activation row)
// is the group's dot of the codes, which the kernel multiplies by the two
// scales and adds, group after group.
//
// Weight image.  16-row tiles of 128-column groups: tile t, group g is one
// 2 KB block holding, for lane l = i + 16q of a wave, the codes of row 16t + i,
// columns 128g + 32q .. 128g + 32q + 31 (the MFMA's A operand; its B operand
// pairs byte e of lane (j, q) with byte e of lane (i, q)): the first 16 of them
// at 16*l, the other 16 at 1024 + 16*l, so that each of the wave's two 16-byte
// loads reads 1 KB of consecutive bytes.  Groups of a tile follow each other,
// tiles follow each other, rows past n are zero.  Then (256-byte aligned) the
// fp32 block scales [ceil(n/128)][k/128], row major.
#include <hip/hip_runtime.h>

#include "qg_device.h"
#include "qg_internal.h"
#include "qg_launch.h"
#include "qg_route.h"

namespace qg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int F8_GROUP = 128;
constexpr int F8_STEP_BYTES = 2048;  // one (tile, group) block
constexpr int F8_HALF_U4 = 64;       // second 16 bytes of a lane: 1 KB on, in uint4
constexpr int F8_E8M0_ONE = 127;     // MFMA operand scale 2^0
constexpr int64_t F8_ROT = 7;        // start-group stride between neighbouring tile groups

// ------------------------------------------------------- weight image ---
// One workgroup per (128-row block, group): thread t takes row t / 2, half t % 2
// of the group (64 columns).
__global__ __launch_bounds__(256) void fp8_quantize_weights_kernel(const float* __restrict__ w, int64_t n, int64_t k,
                                                                   int64_t kg, int64_t np16,
                                                                   uint8_t* __restrict__ img,
                                                                   float* __restrict__ scales) {
  __shared__ float s_max[256 / WAVE];
  const int64_t bi = blockIdx.x, g = blockIdx.y;
  const int tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
  const int64_t o = bi * F8_GROUP + (tid >> 1);
  const int h = tid & 1;
  float v[64];
  float am = 0.0f;
  const float* src = w + o * k + g * F8_GROUP + 64 * h;
#pragma unroll
  for (int j = 0; j < 16; j++) {
    const float4 a = o < n ? reinterpret_cast<const float4*>(src)[j] : make_float4(0.f, 0.f, 0.f, 0.f);
    v[4 * j] = a.x, v[4 * j + 1] = a.y, v[4 * j + 2] = a.z, v[4 * j + 3] = a.w;
    am = fmaxf(am, fmaxf(fmaxf(fabsf(a.x), fabsf(a.y)), fmaxf(fabsf(a.z), fabsf(a.w))));
  }
  for (int off = 32; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
  if (lane == 0) s_max[wave] = am;
  __syncthreads();
  am = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const float s = am / 448.0f;
  if (tid == 0) scales[bi * kg + g] = s;
  if (o >= np16) return;  // past the image's last tile
  const int64_t t = o >> 4, i = o & 15;
  uint8_t* dst = img + (t * kg + g) * F8_STEP_BYTES;
#pragma unroll
  for (int qq = 0; qq < 2; qq++) {  // lanes i + 16q, q = 2h + qq: 32 columns each
    uint32_t wd[8];
#pragma unroll
    for (int d = 0; d < 8; d++) {
      uint32_t word = 0;
#pragma unroll
      for (int b = 0; b < 4; b++) {
        const float x = v[qq * 32 + d * 4 + b];
        word |= (s != 0.0f ? e4m3_code(x / s) : 0u) << (8 * b);
      }
      wd[d] = word;
    }
    uint4* p = reinterpret_cast<uint4*>(dst + (i + 16 * (2 * h + qq)) * 16);
    p[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    p[F8_HALF_U4] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
  }
}

int launch_fp8_quantize_weights(const float* w, int64_t n, int64_t k, void* image, hipStream_t s) {
  const int64_t kg = k / F8_GROUP, nb = (n + F8_GROUP - 1) / F8_GROUP;
  uint8_t* img = static_cast<uint8_t*>(image);
  float* scales = reinterpret_cast<float*>(img + fp8_scale_offset(n, k));
  hipLaunchKernelGGL(fp8_quantize_weights_kernel, dim3((unsigned)nb, (unsigned)kg), dim3(256), 0, s, w, n, k, kg,
                     f16_tiles(n) * 16, img, scales);
  return hip_status(hipGetLastError(), "fp8_quantize_weights_kernel");
}

// ---------------------------------------------------- activation groups ---
// One wave per (row, group): two columns per lane.  Codes [rows][k] then fp32
// scales [rows][k/128] (the FP8 workspace).
__global__ __launch_bounds__(256) void fp8_prepare_kernel(const float* __restrict__ x, int rows, int64_t k, int64_t kg,
                                                          uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int64_t wi = (int64_t)blockIdx.x * (256 / WAVE) + (threadIdx.x / WAVE);
  const int lane = threadIdx.x % WAVE;
  if (wi >= (int64_t)rows * kg) return;  // whole waves
  const int64_t r = wi / kg, g = wi - r * kg;
  const float2 v = reinterpret_cast<const float2*>(x + r * k + g * F8_GROUP)[lane];
  fp8_group_store(v, lane, codes + r * k + g * F8_GROUP, scales + wi);
}

// SwiGLU of m gate/up rows (gate values [0, ffn), up values [ffn, 2 ffn)),
// h = silu(g) * u in the arithmetic of swiglu_kernel, into FP8 groups as
// fp8_prepare_kernel writes them (the FP8 workspace of m rows of ffn).
__global__ __launch_bounds__(256) void swiglu_fp8_kernel(const float* __restrict__ gu, int m, int64_t ffn, int64_t kg,
                                                         uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int64_t wi = (int64_t)blockIdx.x * (256 / WAVE) + (threadIdx.x / WAVE);
  const int lane = threadIdx.x % WAVE;
  if (wi >= (int64_t)m * kg) return;  // whole waves
  const int64_t j = wi / kg, g = wi - j * kg;
  const float* row = gu + j * 2 * ffn + g * F8_GROUP + 2 * lane;
  const float2 gv = *reinterpret_cast<const float2*>(row), uv = *reinterpret_cast<const float2*>(row + ffn);
  const float2 h = make_float2(gv.x / (1.0f + expf(-gv.x)) * uv.x, gv.y / (1.0f + expf(-gv.y)) * uv.y);
  fp8_group_store(h, lane, codes + j * ffn + g * F8_GROUP, scales + wi);
}

int launch_swiglu_fp8(const float* gu, int m, int64_t ffn, void* hws, hipStream_t s) {
  const int64_t kg = ffn / F8_GROUP, waves = (int64_t)m * kg;
  uint8_t* w = static_cast<uint8_t*>(hws);
  hipLaunchKernelGGL(swiglu_fp8_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, gu, m, ffn, kg, w,
                     reinterpret_cast<float*>(w + fp8_ws_scale_offset(m, ffn)));
  return hip_status(hipGetLastError(), "swiglu_fp8_kernel");
}

int launch_fp8_prepare(const float* x, int rows, int64_t k, void* ws, hipStream_t s) {
  const int64_t kg = k / F8_GROUP;
  uint8_t* w = static_cast<uint8_t*>(ws);
  const int64_t waves = (int64_t)rows * kg;
  hipLaunchKernelGGL(fp8_prepare_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, x, rows, k, kg, w,
                     reinterpret_cast<float*>(w + fp8_ws_scale_offset(rows, k)));
  return hip_status(hipGetLastError(), "fp8_prepare_kernel");
}

// ----------------------------------------------------------------- GEMV ---
template <int NT>
struct F8Step {
  uint4 a[NT][2];  // 32 weight codes per tile
  uint4 b[2];      // 32 activation codes
  float sx;        // the activation group's scale
  float sw[NT];    // the weight blocks' scales
};

template <int NT>
__device__ __forceinline__ void f8_load(F8Step<NT>& st, const uint8_t* const (&wt)[NT], const float* const (&wsr)[NT],
                                        const uint8_t* xc, const float* xs, int64_t g) {
#pragma unroll
  for (int t = 0; t < NT; t++) {
    const uint4* p = reinterpret_cast<const uint4*>(wt[t] + g * F8_STEP_BYTES);
    st.a[t][0] = ld16_stream(p);
    st.a[t][1] = ld16_stream(p + F8_HALF_U4);
    st.sw[t] = wsr[t][g];
  }
  const uint4* xb = reinterpret_cast<const uint4*>(xc + g * F8_GROUP);
  st.b[0] = xb[0];
  st.b[1] = xb[1];
  st.sx = xs[g];
}

template <int NT>
__device__ __forceinline__ void f8_compute(v4f (&acc)[NT], const F8Step<NT>& st) {
  v8i b;
  __builtin_memcpy(&b, &st.b, 32);
#pragma unroll
  for (int t = 0; t < NT; t++) {
    v8i a;
    __builtin_memcpy(&a, &st.a[t], 32);
    const v4f c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0,
                                                                    F8_E8M0_ONE, 0, F8_E8M0_ONE);
    const float m = st.sw[t] * st.sx;
#pragma unroll
    for (int v = 0; v < 4; v++) acc[t][v] = __builtin_fmaf(c[v], m, acc[t][v]);
  }
}

// NT 16-row tiles per workgroup step, S waves over contiguous group ranges
// (added left to right at the end), LA groups in flight; persistent over tile
// groups.  A row's result depends on its own activations, K, N and S only: a
// wave starts its range at a group set by the tile's index / 4, the same for
// NT = 1, 2 and 4, whatever the rows.
template <int NT, int S, int LA>
__global__ __launch_bounds__(S * WAVE) void gemv_fp8_kernel(const uint8_t* __restrict__ img,
                                                            const float* __restrict__ wsc, int64_t N, int64_t K,
                                                            const uint8_t* __restrict__ xcodes,
                                                            const float* __restrict__ xscales, int R,
                                                            float* __restrict__ y, int64_t tgroups) {
  __shared__ float red[S * NT * 4 * WAVE];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & (WAVE - 1);
  const int i = lane & 15, q = lane >> 4;
  const int64_t kg = K / F8_GROUP, tiles = (N + 15) / 16;
  const int64_t g0 = kg * wave / S, g1 = kg * (wave + 1) / S;  // this wave's groups
  const int64_t ng = g1 - g0;
  const int xr = i < R ? i : R - 1;  // activation row of this lane's column
  const uint8_t* xc = xcodes + (int64_t)xr * K + 32 * q;
  const float* xs = xscales + (int64_t)xr * kg;
  const uint8_t* wt[NT];
  const float* wsr[NT];
  int64_t lc = g0;  // next group to load
  F8Step<NT> f[LA];
  // Points the wave at tile group grp and puts its first LA groups in flight.
  // The wave walks its groups from a tile-dependent start, wrapping round, so
  // that tile groups in flight together read different offsets.
  auto start = [&](int64_t grp) {
#pragma unroll
    for (int t = 0; t < NT; t++) {
      int64_t tt = grp * NT + t;
      tt = tt < tiles ? tt : tiles - 1;  // past the end: reread, store nothing
      wt[t] = img + tt * kg * F8_STEP_BYTES + 16 * lane;
      wsr[t] = wsc + (tt >> 3) * kg;  // 8 tiles per 128-row block
    }
    lc = g0 + (ng ? ((grp * NT >> 2) * F8_ROT) % ng : 0);
    // (no bounds branch, which would make the step loop wait for every load in
    // flight: a wave with fewer than LA groups loads groups of its range again,
    // or the last group when it has none, and never uses the extra copies)
#pragma unroll
    for (int j = 0; j < LA; j++) {
      f8_load<NT>(f[j], wt, wsr, xc, xs, lc < kg ? lc : kg - 1);
      if (ng) lc = lc + 1 == g1 ? g0 : lc + 1;
    }
  };
  if (blockIdx.x < tgroups) start(blockIdx.x);
  for (int64_t grp = blockIdx.x; grp < tgroups; grp += gridDim.x) {
    v4f acc[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] = (v4f){0.f, 0.f, 0.f, 0.f};
    int64_t st = 0;
    // rounds whose every group has a next group to load: no branch around the loads
    for (; st + 2 * LA <= ng; st += LA) {
#pragma unroll
      for (int j = 0; j < LA; j++) {
        f8_compute<NT>(acc, f[j]);
        f8_load<NT>(f[j], wt, wsr, xc, xs, lc);
        lc = lc + 1 == g1 ? g0 : lc + 1;
        __builtin_amdgcn_sched_barrier(0);  // each group's loads ahead of the next group's product
      }
    }
    for (; st < ng; st += LA) {
#pragma unroll
      for (int j = 0; j < LA; j++) {
        if (st + j < ng) {
          f8_compute<NT>(acc, f[j]);
          if (st + j + LA < ng) {
            f8_load<NT>(f[j], wt, wsr, xc, xs, lc);
            lc = lc + 1 == g1 ? g0 : lc + 1;
          }
        }
      }
    }
    // every group is consumed: the next tile group's first loads fly during the reduction
    if (grp + gridDim.x < tgroups) start(grp + gridDim.x);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; t++)
#pragma unroll
      for (int v = 0; v < 4; v++) red[((wave * NT + t) * 4 + v) * WAVE + lane] = acc[t][v];
    __syncthreads();
    if (wave == 0 && i < R) {
#pragma unroll
      for (int t = 0; t < NT; t++)
#pragma unroll
        for (int v = 0; v < 4; v++) {
          float a = red[(t * 4 + v) * WAVE + lane];
          for (int s2 = 1; s2 < S; s2++) a += red[((s2 * NT + t) * 4 + v) * WAVE + lane];
          const int64_t row = (grp * NT + t) * 16 + 4 * q + v;
          if (row < N) y[(int64_t)i * N + row] = a;
        }
    }
  }
}

template <int NT, int S, int LA>
static void launch_fp8_t(const uint8_t* img, const float* wsc, int64_t n, int64_t k, const uint8_t* xc,
                         const float* xs, int rows, float* y, hipStream_t s) {
  auto kern = gemv_fp8_kernel<NT, S, LA>;
  const int64_t groups = (f16_tiles(n) + NT - 1) / NT;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, S * WAVE, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  const int64_t g = (int64_t)device_cus() * per_cu;
  hipLaunchKernelGGL(kern, dim3((unsigned)(groups < g ? groups : g)), dim3(S * WAVE), 0, s, img, wsc, n, k, xc, xs,
                     rows, y, groups);
}

// Wave ranges of k (S) for an n x k FP8 GEMV: 2 on large n, 4 on mid-size, 8
// on small, never more than k has 128-column groups.  The dense and grouped
// launches take S from here, so a row's sums depend on n and k only.
static int fp8_waves(int64_t t16, int64_t kg) {
  int S = t16 >= 4096 ? 2 : t16 >= 256 ? 4 : 8;
  while (S > 1 && S > kg) S >>= 1;
  return S;
}

int launch_gemv_fp8(const void* image, int64_t n, int64_t k, const void* ws, int rows, float* y, hipStream_t s) {
  const uint8_t* img = static_cast<const uint8_t*>(image);
  const float* wsc = reinterpret_cast<const float*>(img + fp8_scale_offset(n, k));
  const uint8_t* xc = static_cast<const uint8_t*>(ws);
  const float* xs = reinterpret_cast<const float*>(xc + fp8_ws_scale_offset(rows, k));
  const int64_t t16 = f16_tiles(n);
  // For each n and k the same S (so the same sums) at every row count; above
  // 8 rows wider tiles share each activation load where there are tiles enough.
  switch (fp8_waves(t16, k / F8_GROUP)) {
    case 8: launch_fp8_t<1, 8, 4>(img, wsc, n, k, xc, xs, rows, y, s); break;
    case 4:
      if (t16 >= 512 && rows > 8) launch_fp8_t<2, 4, 2>(img, wsc, n, k, xc, xs, rows, y, s);
      else launch_fp8_t<1, 4, 4>(img, wsc, n, k, xc, xs, rows, y, s);
      break;
    case 2:
      if (t16 >= 4096 && rows > 8) launch_fp8_t<4, 2, 2>(img, wsc, n, k, xc, xs, rows, y, s);
      else if (t16 >= 4096) launch_fp8_t<2, 2, 2>(img, wsc, n, k, xc, xs, rows, y, s);
      else launch_fp8_t<1, 2, 4>(img, wsc, n, k, xc, xs, rows, y, s);
      break;
    default: launch_fp8_t<2, 1, 2>(img, wsc, n, k, xc, xs, rows, y, s); break;
  }
  return hip_status(hipGetLastError(), "gemv_fp8_kernel");
}

// ------------------------------------------------------------ grouped ---
// Routed experts: persistent over the (item, tile group) units of the grouped
// plan (items of at most 16 assignments of one expert).  A unit is a tile
// group of gemv_fp8_kernel over the item's expert image, its activation
// columns the item's rows gathered from the prepared rows through the row
// map, its outputs written to the assignments' rows.  The group order and
// the wave split are those of gemv_fp8_kernel for the same n (S set by the
// tile count alike), so each assignment's output has the bits of the
// one-row dense call on its row.
// LDS of a grouped FP8 launch that takes the SwiGLU in its staging: the FP8
// groups of up to 16 rows of k (codes, then fp32 scales).
static inline size_t fp8_glu_lds_bytes(int64_t k) { return (size_t)QG_MAX_ROWS * ((size_t)k + (size_t)(k / F8_GROUP) * 4); }
bool fp8_glu_fits(int64_t k) { return fp8_glu_lds_bytes(k) <= 40 * 1024; }

// The (item, tile group) units of a grouped FP8 launch, nitems items of the
// plan (sorted, items, x_index: global memory, or the workgroup's LDS).
// Every thread calls it.  GLU: a unit's activation rows are the SwiGLU of
// the item's gate/up rows of glu ([m][2K]: gate values, then up values),
// put in FP8 groups in the workgroup's LDS (hst: codes [16][K], then scales
// [16][K/128]) with the arithmetic of swiglu_fp8_kernel, so the SwiGLU
// launch goes; xcodes / xscales are not read.
template <int NT, int S, int LA, bool GLU = false>
__device__ __forceinline__ void grouped_fp8_units(const uint8_t* __restrict__ images, int64_t expert_bytes,
                                                  int64_t scale_off, int64_t N, int64_t K,
                                                  const uint8_t* __restrict__ xcodes,
                                                  const float* __restrict__ xscales, int nitems,
                                                  const int* __restrict__ sorted, const int* __restrict__ items,
                                                  const int32_t* __restrict__ x_index, float* __restrict__ y,
                                                  int64_t tgroups, float* red, int* s_map,
                                                  const float* __restrict__ glu = nullptr, uint8_t* hst = nullptr) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & (WAVE - 1);
  const int i = lane & 15, q = lane >> 4;
  const int64_t kg = K / F8_GROUP, tiles = (N + 15) / 16;
  const int64_t g0 = kg * wave / S, g1 = kg * (wave + 1) / S;  // this wave's groups
  const int64_t ng = g1 - g0;
  const int64_t units = (int64_t)nitems * tgroups;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {  // uniform over the workgroup
    const int item = (int)(u / tgroups);
    const int64_t grp = u - (int64_t)item * tgroups;
    const int e = items[3 * item], start = items[3 * item + 1], cnt = items[3 * item + 2];
    __syncthreads();  // the previous unit is done with s_map and red
    if ((int)threadIdx.x < cnt) {
      const int a = sorted[start + threadIdx.x];
      s_map[threadIdx.x] = x_index ? x_index[a] : a;
      s_map[QG_MAX_ROWS + threadIdx.x] = a;
    }
    __syncthreads();
    const uint8_t* img = images + (int64_t)e * expert_bytes;
    const float* wsc = reinterpret_cast<const float*>(img + scale_off);
    const uint8_t* xc;
    const float* xs;
    if constexpr (GLU) {
      // a wave per (row, group) of the item's rows
      float* hsc = reinterpret_cast<float*>(hst + QG_MAX_ROWS * K);
      const int kgi = (int)kg;
      for (int w = wave; w < cnt * kgi; w += S) {
        const int r = w / kgi, gi = w - r * kgi;
        const float* row = glu + (int64_t)s_map[r] * 2 * K + gi * F8_GROUP + 2 * lane;
        const float2 gv = *reinterpret_cast<const float2*>(row), uv = *reinterpret_cast<const float2*>(row + K);
        const float2 h = make_float2(gv.x / (1.0f + expf(-gv.x)) * uv.x, gv.y / (1.0f + expf(-gv.y)) * uv.y);
        fp8_group_store(h, lane, hst + (int64_t)r * K + gi * F8_GROUP, hsc + r * kgi + gi);
      }
      __syncthreads();
      const int xr = i < cnt ? i : cnt - 1;  // columns past the item's rows read a real row, store nothing
      xc = hst + (int64_t)xr * K + 32 * q;
      xs = hsc + (int64_t)xr * kg;
    } else {
      const int xr = s_map[i < cnt ? i : cnt - 1];  // columns past the item's rows read a real row, store nothing
      xc = xcodes + (int64_t)xr * K + 32 * q;
      xs = xscales + (int64_t)xr * kg;
    }
    const uint8_t* wt[NT];
    const float* wsr[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) {
      int64_t tt = grp * NT + t;
      tt = tt < tiles ? tt : tiles - 1;  // past the end: reread, store nothing
      wt[t] = img + tt * kg * F8_STEP_BYTES + 16 * lane;
      wsr[t] = wsc + (tt >> 3) * kg;
    }
    int64_t lc = g0 + (ng ? ((grp * NT >> 2) * F8_ROT) % ng : 0);
    F8Step<NT> f[LA];
#pragma unroll
    for (int j = 0; j < LA; j++)
      if (j < ng) {
        f8_load<NT>(f[j], wt, wsr, xc, xs, lc);
        lc = lc + 1 == g1 ? g0 : lc + 1;
      }
    v4f acc[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) acc[t] = (v4f){0.f, 0.f, 0.f, 0.f};
    for (int64_t st = 0; st < ng; st += LA) {
#pragma unroll
      for (int j = 0; j < LA; j++) {
        if (st + j < ng) {
          f8_compute<NT>(acc, f[j]);
          if (st + j + LA < ng) {
            f8_load<NT>(f[j], wt, wsr, xc, xs, lc);
            lc = lc + 1 == g1 ? g0 : lc + 1;
          }
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NT; t++)
#pragma unroll
      for (int v = 0; v < 4; v++) red[((wave * NT + t) * 4 + v) * WAVE + lane] = acc[t][v];
    __syncthreads();
    if (wave == 0 && i < cnt) {
      const int64_t orow = s_map[QG_MAX_ROWS + i];
#pragma unroll
      for (int t = 0; t < NT; t++)
#pragma unroll
        for (int v = 0; v < 4; v++) {
          float a = red[(t * 4 + v) * WAVE + lane];
          for (int s2 = 1; s2 < S; s2++) a += red[((s2 * NT + t) * 4 + v) * WAVE + lane];
          const int64_t row = (grp * NT + t) * 16 + 4 * q + v;
          if (row < N) y[orow * N + row] = a;
        }
    }
  }
}

template <int NT, int S, int LA, bool GLU>
__global__ __launch_bounds__(S * WAVE) void grouped_fp8_kernel(
    const uint8_t* __restrict__ images, int64_t expert_bytes, int64_t scale_off, int64_t N, int64_t K,
    const uint8_t* __restrict__ xcodes, const float* __restrict__ xscales, const int* __restrict__ header,
    const int* __restrict__ sorted, const int* __restrict__ items, const int32_t* __restrict__ x_index,
    float* __restrict__ y, int64_t tgroups, const float* __restrict__ glu) {
  __shared__ float red[S * NT * 4 * WAVE];
  __shared__ int s_map[2 * QG_MAX_ROWS];  // activation row, then output row, of each column
  extern __shared__ __align__(16) uint8_t hst[];  // GLU: the SwiGLU rows' FP8 groups
  grouped_fp8_units<NT, S, LA, GLU>(images, expert_bytes, scale_off, N, K, xcodes, xscales, header[0], sorted,
                                    items, x_index, y, tgroups, red, s_map, glu, hst);
}

// The FP8 MoE step's gate/up launch up to S rows (a row a wave): every
// workgroup computes the step's plan from the router logits (moe_plan_block,
// the same plan in each) into its LDS, workgroup 0 stores it for the down
// launch, and the units run as in grouped_fp8_kernel on the plan in LDS.
template <int NT, int S, int LA>
__global__ __launch_bounds__(S * WAVE) void moe_up_fp8_kernel(const uint8_t* __restrict__ images,
                                                               int64_t expert_bytes, int64_t scale_off, int64_t N,
                                                               int64_t K, const uint8_t* __restrict__ xcodes,
                                                               const float* __restrict__ xscales,
                                                               float* __restrict__ y, int64_t tgroups, MoeUp up) {
  __shared__ float red[S * NT * 4 * WAVE];
  __shared__ int s_map[2 * QG_MAX_ROWS];
  extern __shared__ __align__(16) uint8_t lds[];  // the plan
  const int m = up.rows * (up.topk + up.shared);
  const PlanLds P = plan_carve(lds, m, up.E);
  moe_plan_block<S * WAVE>(up.logits, up.rows, up.E, up.topk, up.shared != 0, P);
  if (blockIdx.x == 0)
    plan_store<S * WAVE>(P, m, up.expert, up.weight, up.x_index, up.header, up.sorted, up.items);
  grouped_fp8_units<NT, S, LA>(images, expert_bytes, scale_off, N, K, xcodes, xscales, P.misc[0], P.sorted,
                               P.items, P.xi, y, tgroups, red, s_map);
}

template <int NT, int S, int LA>
static void launch_grouped_fp8_t(const uint8_t* images, int64_t eb, int64_t so, int64_t n, int64_t k,
                                 const uint8_t* xc, const float* xs, const int* header, const int* sorted,
                                 const int* items, const int32_t* x_index, int m, float* y, hipStream_t s,
                                 const float* glu) {
  auto kern = glu ? grouped_fp8_kernel<NT, S, LA, true> : grouped_fp8_kernel<NT, S, LA, false>;
  const size_t lds = glu ? fp8_glu_lds_bytes(k) : 0;
  const int64_t tgroups = (f16_tiles(n) + NT - 1) / NT;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, S * WAVE, lds) != hipSuccess || per_cu < 1)
    per_cu = 1;
  const int64_t g = (int64_t)device_cus() * per_cu, units = (int64_t)m * tgroups;  // at most m items
  hipLaunchKernelGGL(kern, dim3((unsigned)(units < g ? units : g)), dim3(S * WAVE), lds, s, images, eb, so, n, k, xc,
                     xs, header, sorted, items, x_index, y, tgroups, glu);
}

int launch_grouped_fp8(const void* images, int64_t n, int64_t k, const void* ws, int x_rows, const int* header,
                       const int* sorted, const int* items, const int32_t* x_index, int m, float* y, hipStream_t s,
                       const float* glu) {
  if (m == 0) return QG_OK;
  if (glu && !fp8_glu_fits(k)) return fail(QG_ELAUNCH, "SwiGLU rows staged in LDS: k=%lld too long", (long long)k);
  const uint8_t* img = static_cast<const uint8_t*>(images);
  const int64_t eb = (int64_t)fp8_image_bytes(n, k), so = (int64_t)fp8_scale_offset(n, k);
  const uint8_t* xc = static_cast<const uint8_t*>(ws);
  const float* xs = reinterpret_cast<const float*>(xc + fp8_ws_scale_offset(x_rows, k));
  // S as launch_gemv_fp8 sets it for this n and k (the bits of the dense call);
  // two tiles per unit on small experts, whose units are otherwise too short
  // for their fixed costs (1024 x 2048 experts at 16 rows: 63.0 -> 51.8 us)
  const int64_t t16 = f16_tiles(n);
  switch (fp8_waves(t16, k / F8_GROUP)) {
    case 8: launch_grouped_fp8_t<2, 8, 2>(img, eb, so, n, k, xc, xs, header, sorted, items, x_index, m, y, s, glu); break;
    case 4:
      if (t16 >= 256) launch_grouped_fp8_t<1, 4, 4>(img, eb, so, n, k, xc, xs, header, sorted, items, x_index, m, y, s, glu);
      else launch_grouped_fp8_t<2, 4, 2>(img, eb, so, n, k, xc, xs, header, sorted, items, x_index, m, y, s, glu);
      break;
    case 2: launch_grouped_fp8_t<2, 2, 2>(img, eb, so, n, k, xc, xs, header, sorted, items, x_index, m, y, s, glu); break;
    default: launch_grouped_fp8_t<2, 1, 2>(img, eb, so, n, k, xc, xs, header, sorted, items, x_index, m, y, s, glu); break;
  }
  return hip_status(hipGetLastError(), "grouped_fp8_kernel");
}

template <int NT, int S, int LA>
static void launch_moe_up_fp8_t(const uint8_t* images, int64_t eb, int64_t so, int64_t n, int64_t k,
                                const uint8_t* xc, const float* xs, const MoeUp& up, float* y, hipStream_t s) {
  auto kern = moe_up_fp8_kernel<NT, S, LA>;
  const int64_t tgroups = (f16_tiles(n) + NT - 1) / NT;
  const int m = up.rows * (up.topk + up.shared);
  const size_t lds = plan_lds_bytes(m, up.E);
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, S * WAVE, lds) != hipSuccess || per_cu < 1)
    per_cu = 1;
  const int64_t g = (int64_t)device_cus() * per_cu, units = (int64_t)m * tgroups;  // at most m items
  hipLaunchKernelGGL(kern, dim3((unsigned)(units < g ? units : g)), dim3(S * WAVE), lds, s, images, eb, so, n, k, xc,
                     xs, y, tgroups, up);
}

bool moe_up_fp8_fits(int64_t n, int64_t k, int rows) {
  return rows >= 1 && rows <= fp8_waves(f16_tiles(n), k / F8_GROUP);
}

int launch_moe_up_fp8(const void* images, int64_t n, int64_t k, const void* xprep, const MoeUp& up, float* y,
                      hipStream_t s) {
  if (!moe_up_fp8_fits(n, k, up.rows))
    return fail(QG_ELAUNCH, "the FP8 gate/up launch plans at most a row a wave: rows=%d", up.rows);
  const uint8_t* img = static_cast<const uint8_t*>(images);
  const int64_t eb = (int64_t)fp8_image_bytes(n, k), so = (int64_t)fp8_scale_offset(n, k);
  const uint8_t* xc = static_cast<const uint8_t*>(xprep);
  const float* xs = reinterpret_cast<const float*>(xc + fp8_ws_scale_offset(up.rows, k));
  // the tiling of launch_grouped_fp8 (the same bits)
  const int64_t t16 = f16_tiles(n);
  switch (fp8_waves(t16, k / F8_GROUP)) {
    case 8: launch_moe_up_fp8_t<2, 8, 2>(img, eb, so, n, k, xc, xs, up, y, s); break;
    case 4:
      if (t16 >= 256) launch_moe_up_fp8_t<1, 4, 4>(img, eb, so, n, k, xc, xs, up, y, s);
      else launch_moe_up_fp8_t<2, 4, 2>(img, eb, so, n, k, xc, xs, up, y, s);
      break;
    case 2: launch_moe_up_fp8_t<2, 2, 2>(img, eb, so, n, k, xc, xs, up, y, s); break;
    default: launch_moe_up_fp8_t<2, 1, 2>(img, eb, so, n, k, xc, xs, up, y, s); break;
  }
  return hip_status(hipGetLastError(), "moe_up_fp8_kernel");
}

}  // namespace qg
