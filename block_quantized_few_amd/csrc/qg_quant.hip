// qg_quant.hip -- activation quantizer (A1), offline weight quantizer, and
// the block-dot test hook (A3).
#include <hip/hip_runtime.h>
#include <string.h>

#include "qg_device.h"
#include "qg_internal.h"
#include "qg_launch.h"

namespace qg {

Prep prep_view(const void* ws, const PrepLayout& L) {
  const uint8_t* w = (const uint8_t*)ws;
  return Prep{(const int8_t*)(w + L.codes), (const float*)(w + L.dx), (const int*)(w + L.nsx)};
}

// Loads the eight fp32 elements of quarter q of block b of row r (zeros past
// the row's kb real blocks).
__device__ __forceinline__ void load_quarter(const float* __restrict__ x, int64_t k, int64_t r, int64_t b, int kb,
                                             int q, bool active, float (&v)[8]) {
  if (active && b < kb) {
    const float4* src = reinterpret_cast<const float4*>(x + r * k + b * QK + q * 8);
    const float4 a = src[0], c = src[1];
    v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = c.x, v[5] = c.y, v[6] = c.z, v[7] = c.w;
  } else {
#pragma unroll
    for (int e = 0; e < 8; e++) v[e] = 0.0f;
  }
}

// Where quarter q of block b of row r lands in a workspace (the orders of
// qg_layout.h).  In pair order each quarter also clears the matching quarter
// of its zero partner lane, so every chunk is fully written.
struct PrepDst {
  int8_t* codes;
  float* dx;
  int* nsx;
  int rows;    // rows to quantize (pair order: padded to a multiple of 8)
  int kbp;
  int groups;  // 0: row order; else pair order with this many row groups
  __device__ __forceinline__ void put(int64_t r, int64_t b, int q, unsigned lo, unsigned hi, float d, int sum) const {
    if (groups) {
      const int par = (int)(b & 1), i = (int)(r & 7) + 8 * par, half = q >> 1;
      const int64_t chunk = (b >> 1) * groups + (r >> 3);
      const int64_t lane = (half + 2 * par) * 16 + i, zlane = (half + 2 * (1 - par)) * 16 + i;
      *reinterpret_cast<uint2*>(codes + (chunk * 64 + lane) * 16 + (q & 1) * 8) = make_uint2(lo, hi);
      *reinterpret_cast<uint2*>(codes + (chunk * 64 + zlane) * 16 + (q & 1) * 8) = make_uint2(0u, 0u);
      if (q == 0) {
        dx[chunk * 16 + i] = d;
        nsx[chunk * 16 + i] = -8 * sum;
      }
      return;
    }
    *reinterpret_cast<uint2*>(codes + (r * kbp + b) * 32 + q * 8) = make_uint2(lo, hi);
    if (q == 0) {
      dx[r * kbp + b] = d;
      nsx[r * kbp + b] = -8 * sum;
    }
  }
};

// Four lanes per 32-block over kbp blocks per row; pad blocks come out all
// zero (scale 0, codes 0).
__global__ __launch_bounds__(256) void prepare_kernel(const float* __restrict__ x, int64_t k, int kb, int xrows,
                                                      PrepDst dst) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = t >> 2;
  const int q = (int)(t & 3);
  const bool active = blk < (int64_t)dst.rows * dst.kbp;  // whole quads are active or not
  const int64_t r = active ? blk / dst.kbp : 0, b = active ? blk % dst.kbp : 0;
  float v[8];
  load_quarter(x, k, r, b, kb, q, active && r < xrows, v);  // pad rows quantize to zeros
  unsigned lo, hi;
  float d;
  int sum;
  quantize_quarter(v, lo, hi, d, sum);
  if (active) dst.put(r, b, q, lo, hi, d, sum);
}

// Same for several activation sets; blockIdx.y picks the set.
struct PrepSet {
  const float* x[QG_MAX_SET];
  PrepDst dst[QG_MAX_SET];
  int64_t k[QG_MAX_SET];
  int count;
  int xrows;
};

__global__ __launch_bounds__(256) void prepare_set_kernel(PrepSet s) {
  const int p = blockIdx.y;
  const int64_t k = s.k[p];
  const PrepDst& dst = s.dst[p];
  const int kb = (int)kb_of(k);
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = t >> 2;
  const int q = (int)(t & 3);
  const bool active = blk < (int64_t)dst.rows * dst.kbp;
  const int64_t r = active ? blk / dst.kbp : 0, b = active ? blk % dst.kbp : 0;
  float v[8];
  load_quarter(s.x[p], k, r, b, kb, q, active && r < s.xrows, v);
  unsigned lo, hi;
  float d;
  int sum;
  quantize_quarter(v, lo, hi, d, sum);
  if (active) dst.put(r, b, q, lo, hi, d, sum);
}

// Plain layout [rows][k] with the code sum (test hook).
__global__ __launch_bounds__(256) void quantize_plain_kernel(const float* __restrict__ x, int rows, int64_t k, int kb,
                                                             int8_t* __restrict__ qx, float* __restrict__ dx,
                                                             int* __restrict__ sx) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = t >> 2;
  const int q = (int)(t & 3);
  const bool active = blk < (int64_t)rows * kb;
  const int64_t r = active ? blk / kb : 0, b = active ? blk % kb : 0;
  float v[8];
  load_quarter(x, k, r, b, kb, q, active, v);
  unsigned lo, hi;
  float d;
  int sum;
  quantize_quarter(v, lo, hi, d, sum);
  if (!active) return;
  *reinterpret_cast<uint2*>(qx + r * k + b * 32 + q * 8) = make_uint2(lo, hi);
  if (q == 0) {
    dx[r * kb + b] = d;
    sx[r * kb + b] = sum;
  }
}

// One thread per (row, block) of the padded image.  d = fp16(amax/qmax) with
// round-to-nearest-even, codes by IEEE division by the stored scale.
template <int FMT>
__global__ __launch_bounds__(256) void quantize_weights_kernel(const float* __restrict__ w, int64_t n, int64_t k,
                                                               int kb, int kbp, uint8_t* __restrict__ code,
                                                               uint16_t* __restrict__ scale) {
  const int64_t np = np_of(n);
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= np * kbp) return;
  const int64_t o = t / kbp, b = t % kbp;
  unsigned packed[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  uint16_t d16 = 0;
  if (o < n && b < kb) {
    float v[32];
    const float4* src = reinterpret_cast<const float4*>(w + o * k + b * QK);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float4 f = src[i];
      v[4 * i] = f.x, v[4 * i + 1] = f.y, v[4 * i + 2] = f.z, v[4 * i + 3] = f.w;
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(v[i]));
    const _Float16 h = (_Float16)(amax / (FMT == FMT_Q8 ? 127.0f : 7.0f));
    __builtin_memcpy(&d16, &h, 2);
    const float dq = (float)h;
    if (FMT == FMT_Q8) {
      if (dq != 0.0f) {
#pragma unroll
        for (int i = 0; i < 32; i++) {
          const int q = (int)fminf(fmaxf(roundf(v[i] / dq), -127.0f), 127.0f);
          packed[i >> 2] |= ((unsigned)(q & 0xff)) << (8 * (i & 3));
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; i++) {
        int lo = 8, hi = 8;  // code 8 stands for 0
        if (dq != 0.0f) {
          lo = (int)fminf(fmaxf(roundf(v[i] / dq), -8.0f), 7.0f) + 8;
          hi = (int)fminf(fmaxf(roundf(v[i + 16] / dq), -8.0f), 7.0f) + 8;
        }
        // the image keeps c XOR 8 (the 4-bit two's complement of c - 8)
        packed[i >> 2] |= ((unsigned)((lo ^ 8) | ((hi ^ 8) << 4))) << (8 * (i & 3));
      }
    }
  }
  uint8_t* dst = code + cell_row_offset(FMT, o, b, kbp);
  *reinterpret_cast<uint4*>(dst) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  if (FMT == FMT_Q8) *reinterpret_cast<uint4*>(dst + 256) = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  scale[scale_index(o, b, kbp)] = d16;
}

// Q4_K superblock quantizer, one thread per (row, superblock) of the padded
// image: per sub-block j (lo = min(0, min w), hi = max w) s_j = (hi - lo) / 15
// and mn_j = -lo; d = fp16(max s / 63), dmin = fp16(max mn / 63); sc_j =
// min(63, round(s_j / d)), m_j = min(63, round(mn_j / dmin)) (0 for a zero
// scale); codes clamp(round((w + dmin*m_j) / (d*sc_j)), 0, 15) (0 when
// d*sc_j == 0).  IEEE divisions, round half away from zero.  Pad rows and
// superblocks are written as zeros.
__global__ __launch_bounds__(256) void quantize_q4k_weights_kernel(const float* __restrict__ w, int64_t n, int64_t k,
                                                                   int kbp, uint8_t* __restrict__ code,
                                                                   uint8_t* __restrict__ hdr) {
  const int sbp = kbp / 8, ns = (int)(k / QK_K);
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= np_of(n) * sbp) return;
  const int64_t o = t / sbp;
  const int s = (int)(t % sbp);
  uint4 h = make_uint4(0u, 0u, 0u, 0u);
  unsigned cells[8][4];
#pragma unroll
  for (int j = 0; j < 8; j++) cells[j][0] = cells[j][1] = cells[j][2] = cells[j][3] = 0u;
  if (o < n && s < ns) {
    const float* v = w + o * k + (int64_t)s * QK_K;
    float sj[8], mnj[8], smax = 0.0f, mmax = 0.0f;
    for (int j = 0; j < 8; j++) {
      float lo = 0.0f, hi = v[32 * j];
      for (int i = 0; i < 32; i++) {
        const float x = v[32 * j + i];
        lo = x < lo ? x : lo;
        hi = x > hi ? x : hi;
      }
      sj[j] = (hi - lo) / 15.0f;
      mnj[j] = -lo;
      smax = sj[j] > smax ? sj[j] : smax;
      mmax = mnj[j] > mmax ? mnj[j] : mmax;
    }
    const _Float16 dh = (_Float16)(smax / 63.0f), mh = (_Float16)(mmax / 63.0f);
    const float d = (float)dh, dmin = (float)mh;
    unsigned sc[8], m[8];
    for (int j = 0; j < 8; j++) {
      sc[j] = d != 0.0f ? (unsigned)fminf(fmaxf(roundf(sj[j] / d), 0.0f), 63.0f) : 0u;
      m[j] = dmin != 0.0f ? (unsigned)fminf(fmaxf(roundf(mnj[j] / dmin), 0.0f), 63.0f) : 0u;
    }
    uint16_t d16, m16;
    __builtin_memcpy(&d16, &dh, 2);
    __builtin_memcpy(&m16, &mh, 2);
    unsigned b[12];
    for (int j = 0; j < 4; j++) {
      b[j] = (sc[j] & 63u) | ((sc[j + 4] >> 4) << 6);
      b[j + 4] = (m[j] & 63u) | ((m[j + 4] >> 4) << 6);
      b[j + 8] = (sc[j + 4] & 15u) | ((m[j + 4] & 15u) << 4);
    }
    h.x = (unsigned)d16 | ((unsigned)m16 << 16);
    h.y = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    h.z = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
    h.w = b[8] | (b[9] << 8) | (b[10] << 16) | (b[11] << 24);
    for (int j = 0; j < 8; j++) {
      const float D = d * (float)sc[j], M = dmin * (float)m[j];
      for (int i = 0; i < 32; i++) {
        const unsigned q = D != 0.0f ? (unsigned)fminf(fmaxf(roundf((v[32 * j + i] + M) / D), 0.0f), 15.0f) : 0u;
        const int l = i & 15;  // byte l of the cell: code l low, code l + 16 high
        cells[j][l >> 2] |= (q << ((i >> 4) * 4)) << (8 * (l & 3));
      }
    }
  }
  *reinterpret_cast<uint4*>(hdr + q4k_header_offset(o, s, kbp)) = h;
#pragma unroll
  for (int j = 0; j < 8; j++)
    *reinterpret_cast<uint4*>(code + cell_row_offset(FMT_Q4K, o, 8 * s + j, kbp)) =
        make_uint4(cells[j][0], cells[j][1], cells[j][2], cells[j][3]);
}

// isum[r][o][b]: the exact block dot of the image's codes with qx (plain).
template <int FMT>
__global__ __launch_bounds__(256) void blockdots_kernel(const uint8_t* __restrict__ code, int64_t n, int kbp, int kb,
                                                        const int8_t* __restrict__ qx, int rows, int64_t k,
                                                        int* __restrict__ isum) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)rows * n * kb) return;
  const int64_t b = t % kb, o = (t / kb) % n, r = t / ((int64_t)kb * n);
  const int8_t* xq = qx + r * k + b * QK;
  const uint4 xl = ld16(xq), xh = ld16(xq + 16);
  const uint8_t* p = code + cell_row_offset(FMT, o, b, kbp);
  int s;
  if (FMT == FMT_Q8) {
    s = dot_q8(ld16(p), ld16(p + 256), xl, xh);
  } else if (FMT == FMT_Q4K) {
    s = dot_q4(ld16(p), xl, xh, 0);  // raw codes: the sub-min's share is not part of the integer dot
  } else {
    s = dot_q4s16(ld16(p), xl, xh) >> 4;  // sixteen times the dot, exactly
  }
  isum[t] = s;
}

static unsigned grid1(int64_t threads, int per) { return (unsigned)((threads + per - 1) / per); }

static PrepDst prep_dst(void* ws, const PrepLayout& L, int rows, int64_t k) {
  uint8_t* w = (uint8_t*)ws;
  return PrepDst{(int8_t*)(w + L.codes), (float*)(w + L.dx), (int*)(w + L.nsx), L.pairs ? L.groups * 8 : rows,
                 (int)kbp_of(k), L.pairs ? L.groups : 0};
}

// ------------------------------------------------------ add + RMS norm ---
//
// The step before a projection group: h = x + residual, y = h * inv * gamma
// with inv = 1 / sqrt(mean(h^2) + eps), and A1 of y into the workspace in the
// layout the GEMV reads -- the bytes prepare_kernel writes for the same fp32
// y.  One workgroup per workspace row (pair order pads to 8-row groups; pad
// rows come out zero).  The sum of squares has a fixed order: each thread adds
// its float4 chunks t, t + 1024, ... element by element, the waves reduce by a
// DPP tree, and the sixteen wave sums add left to right.  x, residual, h and
// y may alias (each element is read and written by one thread, and y is
// written only after every thread has finished reading for the sum).
constexpr int NORM_WG = 1024;

__device__ __forceinline__ float norm_wave_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // pairs
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quads
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // 8-lane mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // 16-lane mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

__global__ __launch_bounds__(NORM_WG) void add_rmsnorm_prepare_kernel(const float* x, const float* res,
                                                                      const float* __restrict__ gamma, float eps,
                                                                      int xrows, int64_t k, int kb, float* h_out,
                                                                      float* y_out, PrepDst dst, bool write_ws) {
  __shared__ float s_part[NORM_WG / WAVE];
  const int r = blockIdx.x, tid = threadIdx.x, wave = tid / WAVE, lane = tid % WAVE;
  const bool real = r < xrows;  // uniform over the workgroup
  const float* xr = x + (int64_t)r * k;
  const float* rr = res ? res + (int64_t)r * k : nullptr;
  float inv = 0.0f;
  if (real) {
    float ss = 0.0f;
    const int64_t nc = k / 4;
    for (int64_t c0 = tid; c0 < nc; c0 += 2 * NORM_WG) {  // two chunks' loads in flight
      float4 hv[2], rv[2];
#pragma unroll
      for (int u = 0; u < 2; u++) {
        const int64_t c = c0 + u * NORM_WG;
        hv[u] = c < nc ? reinterpret_cast<const float4*>(xr)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
        rv[u] = rr && c < nc ? reinterpret_cast<const float4*>(rr)[c] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 2; u++) {
        const int64_t c = c0 + u * NORM_WG;
        if (c >= nc) break;
        float4 h = hv[u];
        if (rr) {
          h.x += rv[u].x;
          h.y += rv[u].y;
          h.z += rv[u].z;
          h.w += rv[u].w;
        }
        if (h_out) reinterpret_cast<float4*>(h_out + (int64_t)r * k)[c] = h;
        ss += h.x * h.x;
        ss += h.y * h.y;
        ss += h.z * h.z;
        ss += h.w * h.w;
      }
    }
    ss = norm_wave_sum(ss);
    if (lane == 0) s_part[wave] = ss;
    __syncthreads();
    float tot = s_part[0];
    for (int w = 1; w < NORM_WG / WAVE; w++) tot += s_part[w];
    inv = 1.0f / sqrtf(tot / (float)k + eps);
  }
  // four lanes per 32-block; kbp * 4 is a multiple of 64, so whole waves leave the loop together
  // (a thread's pass-1 chunks and its blocks here differ, hence the barrier above)
  for (int64_t t = tid; t < (int64_t)dst.kbp * 4; t += NORM_WG) {
    const int64_t b = t >> 2;
    const int q = (int)(t & 3);
    float v[8];
    if (real && b < kb) {
      const int64_t e0 = b * QK + q * 8;
      // h again: from h_out when it was written (it may alias x or the residual), else recomputed
      const float* hs = h_out ? h_out + (int64_t)r * k : xr;
      const float4 a0 = *reinterpret_cast<const float4*>(hs + e0), a1 = *reinterpret_cast<const float4*>(hs + e0 + 4);
      float h[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      if (rr && !h_out) {
        const float4 b0 = *reinterpret_cast<const float4*>(rr + e0), b1 = *reinterpret_cast<const float4*>(rr + e0 + 4);
        const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
        for (int j = 0; j < 8; j++) h[j] += bb[j];
      }
      const float4 g0 = *reinterpret_cast<const float4*>(gamma + e0), g1 = *reinterpret_cast<const float4*>(gamma + e0 + 4);
      const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
      for (int j = 0; j < 8; j++) v[j] = (h[j] * inv) * gg[j];
      if (y_out) {
        float* yo = y_out + (int64_t)r * k + e0;
        *reinterpret_cast<float4*>(yo) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(yo + 4) = make_float4(v[4], v[5], v[6], v[7]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; j++) v[j] = 0.0f;
    }
    unsigned lo, hi;
    float d;
    int sum;
    quantize_quarter(v, lo, hi, d, sum);
    if (write_ws) dst.put(r, b, q, lo, hi, d, sum);
  }
}

int launch_add_rmsnorm_prepare(const float* x, const float* res, const float* gamma, float eps, int rows, int64_t k,
                               float* h_out, float* y_out, void* ws, hipStream_t s) {
  const PrepLayout L = prep_layout(rows, k);
  PrepDst dst = prep_dst(ws, L, rows, k);
  const bool write_ws = ws != nullptr;
  if (!write_ws) dst.rows = rows;  // no workspace: the real rows only
  hipLaunchKernelGGL(add_rmsnorm_prepare_kernel, dim3((unsigned)dst.rows), dim3(NORM_WG), 0, s, x, res, gamma, eps,
                     rows, k, (int)kb_of(k), h_out, y_out, dst, write_ws);
  return hip_status(hipGetLastError(), "add_rmsnorm_prepare_kernel");
}

int launch_prepare(const float* x, int rows, int64_t k, void* ws, const PrepLayout& L, hipStream_t s) {
  const PrepDst dst = prep_dst(ws, L, rows, k);
  hipLaunchKernelGGL(prepare_kernel, dim3(grid1((int64_t)dst.rows * dst.kbp * 4, 256)), dim3(256), 0, s, x, k,
                     (int)kb_of(k), rows, dst);
  return hip_status(hipGetLastError(), "prepare_kernel");
}

int launch_prepare_set(const qg_act* acts, int count, int rows, hipStream_t s) {
  PrepSet ps;
  memset(&ps, 0, sizeof ps);
  ps.count = count;
  ps.xrows = rows;
  int64_t maxblk = 0;
  for (int i = 0; i < count; i++) {
    ps.x[i] = acts[i].x;
    ps.k[i] = acts[i].k;
    ps.dst[i] = prep_dst(acts[i].ws, prep_layout(rows, acts[i].k), rows, acts[i].k);
    const int64_t blk = (int64_t)ps.dst[i].rows * ps.dst[i].kbp;
    if (blk > maxblk) maxblk = blk;
  }
  hipLaunchKernelGGL(prepare_set_kernel, dim3(grid1(maxblk * 4, 256), count), dim3(256), 0, s, ps);
  return hip_status(hipGetLastError(), "prepare_set_kernel");
}

int launch_quantize_plain(const float* x, int rows, int64_t k, int8_t* qx, float* dx, int32_t* sx, hipStream_t s) {
  const int kb = (int)kb_of(k);
  hipLaunchKernelGGL(quantize_plain_kernel, dim3(grid1((int64_t)rows * kb * 4, 256)), dim3(256), 0, s, x, rows, k, kb,
                     qx, dx, sx);
  return hip_status(hipGetLastError(), "quantize_plain_kernel");
}

int launch_quantize_weights(int fmt, const float* w, int64_t n, int64_t k, void* image, hipStream_t s) {
  uint8_t* img = (uint8_t*)image;
  uint16_t* scale = (uint16_t*)(img + image_scale_offset(fmt, n, k));
  const int kb = (int)kb_of(k), kbp = (int)kbp_of(k);
  if (fmt == FMT_Q4K) {
    hipLaunchKernelGGL(quantize_q4k_weights_kernel, dim3(grid1(np_of(n) * (kbp / 8), 256)), dim3(256), 0, s, w, n, k,
                       kbp, img, (uint8_t*)scale);
    return hip_status(hipGetLastError(), "quantize_q4k_weights_kernel");
  }
  const unsigned g = grid1(np_of(n) * kbp, 256);
  if (fmt == FMT_Q8)
    hipLaunchKernelGGL(quantize_weights_kernel<FMT_Q8>, dim3(g), dim3(256), 0, s, w, n, k, kb, kbp, img, scale);
  else
    hipLaunchKernelGGL(quantize_weights_kernel<FMT_Q4>, dim3(g), dim3(256), 0, s, w, n, k, kb, kbp, img, scale);
  return hip_status(hipGetLastError(), "quantize_weights_kernel");
}

int launch_blockdots(int fmt, const void* image, int64_t n, int64_t k, const int8_t* qx, int rows, int32_t* isum,
                     hipStream_t s) {
  const int kb = (int)kb_of(k), kbp = (int)kbp_of(k);
  const unsigned g = grid1((int64_t)rows * n * kb, 256);
  const uint8_t* img = (const uint8_t*)image;
  if (fmt == FMT_Q8)
    hipLaunchKernelGGL(blockdots_kernel<FMT_Q8>, dim3(g), dim3(256), 0, s, img, n, kbp, kb, qx, rows, k, isum);
  else if (fmt == FMT_Q4K)
    hipLaunchKernelGGL(blockdots_kernel<FMT_Q4K>, dim3(g), dim3(256), 0, s, img, n, kbp, kb, qx, rows, k, isum);
  else
    hipLaunchKernelGGL(blockdots_kernel<FMT_Q4>, dim3(g), dim3(256), 0, s, img, n, kbp, kb, qx, rows, k, isum);
  return hip_status(hipGetLastError(), "blockdots_kernel");
}

}  // namespace qg
