// qg_device.h -- device primitives shared by the libqgemv kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qg_layout.h"

namespace qg {

constexpr int WAVE = 64;
constexpr int FMT_Q8 = 1, FMT_Q4 = 2, FMT_Q4K = 5;  // the QG_FMT_* values of the formats

// Whether a format's codes are 4-bit nibbles (Q4_0: c - 8; Q4_K: raw q).
__host__ __device__ constexpr bool nibble_fmt(int fmt) { return fmt == FMT_Q4 || fmt == FMT_Q4K; }

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// Streaming loads of weight bytes that are read exactly once: the
// non-temporal hint keeps them from displacing activation rows in the caches.
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld8_stream(const void* p) {
  const v2u v = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint16_t ld2_stream(const uint16_t* p) { return __builtin_nontemporal_load(p); }

// f32(half `hi` of the two fp16 in h2) * b, rounded once (the product h2f(h) * b), in one
// mixed-precision FMA with a negative-zero addend.
__device__ __forceinline__ float mul_h_f(uint32_t h2, int hi, float b) {
  float d;
  if (hi)
    asm("v_fma_mix_f32 %0, %1, %2, neg(0) op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(h2), "v"(b));
  else
    asm("v_fma_mix_f32 %0, %1, %2, neg(0) op_sel:[0,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(h2), "v"(b));
  return d;
}

__device__ __forceinline__ float h2f(uint16_t h) {
  _Float16 v;
  __builtin_memcpy(&v, &h, 2);
  return (float)v;
}

// Exact int32 dot of one Q8_0 block (low/high 16 codes) with one q8 block.
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

// Exact int32 dot of 16 packed bytes of raw 4-bit codes c in [0,15] (Q4_K's)
// with one q8 block, from the start value nsx.
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

// Sixteen times the exact int32 dot of one Q4_0 image block with one q8 block.
// The image keeps each code c as c XOR 8, the 4-bit two's complement of
// c - 8; moved to the high half of its byte, a nibble is the int8 16 (c - 8).
// (The products stay exact: |16 * 32 * 8 * 127| < 2^24.)
__device__ __forceinline__ int dot_q4s16(uint4 p, uint4 xl, uint4 xh) {
  const unsigned H = 0xF0F0F0F0u;
  int s = 0;
  s = __builtin_amdgcn_sdot4((int)((p.x << 4) & H), (int)xl.x, s, false);
  s = __builtin_amdgcn_sdot4((int)((p.y << 4) & H), (int)xl.y, s, false);
  s = __builtin_amdgcn_sdot4((int)((p.z << 4) & H), (int)xl.z, s, false);
  s = __builtin_amdgcn_sdot4((int)((p.w << 4) & H), (int)xl.w, s, false);
  s = __builtin_amdgcn_sdot4((int)(p.x & H), (int)xh.x, s, false);
  s = __builtin_amdgcn_sdot4((int)(p.y & H), (int)xh.y, s, false);
  s = __builtin_amdgcn_sdot4((int)(p.z & H), (int)xh.z, s, false);
  s = __builtin_amdgcn_sdot4((int)(p.w & H), (int)xh.w, s, false);
  return s;
}

// Q4_K: sub-block j's (0..7) scale D = d * sc[j] and offset M = dmin * m[j]
// from its superblock header h (h.x = d | dmin << 16, then the twelve bytes
// of 6-bit fields: for j < 4, sc = byte j & 63 and m = byte j+4 & 63; for
// j >= 4, sc = (byte j+4 & 15) | (byte j-4 >> 6) << 4 and m = (byte j+4 >> 4)
// | (byte j >> 6) << 4).  Both products are exact in fp32.
__device__ __forceinline__ void q4k_dm(uint4 h, int j, float& D, float& M) {
  const int sh = (j & 3) * 8;
  const unsigned a = (h.y >> sh) & 255u, b = (h.z >> sh) & 255u, c = (h.w >> sh) & 255u;
  const unsigned sc = j < 4 ? (a & 63u) : ((c & 15u) | ((a >> 6) << 4));
  const unsigned m = j < 4 ? (b & 63u) : ((c >> 4) | ((b >> 6) << 4));
  D = mul_h_f(h.x, 0, (float)sc);
  M = mul_h_f(h.x, 1, (float)m);
}

// Q4_K: sub-block j's 6-bit sub-scale and sub-min from a header (as q4k_dm).
__device__ __forceinline__ void q4k_scm(uint4 h, int j, unsigned& sc, unsigned& m) {
  const int sh = (j & 3) * 8;
  const unsigned a = (h.y >> sh) & 255u, b = (h.z >> sh) & 255u, c = (h.w >> sh) & 255u;
  sc = j < 4 ? (a & 63u) : ((c & 15u) | ((a >> 6) << 4));
  m = j < 4 ? (b & 63u) : ((c >> 4) | ((b >> 6) << 4));
}

// One Q4_K sub-block's share of an output: acc + dx * (D * isum - M * xsum),
// isum the integer dot of the raw codes with the q8 codes and xsum the sum of
// those q8 codes; the same operations in every kernel, so a row's bits do not
// depend on which kernel or how many rows.
__device__ __forceinline__ float q4k_acc(float acc, int isum, int xsum, float D, float M, float dx) {
  const float t = __builtin_fmaf((float)isum, D, -((float)xsum * M));
  return __builtin_fmaf(t, dx, acc);
}

// Cross-lane moves inside groups of four lanes (DPP quad permutes).
__device__ __forceinline__ int quad_xor1(int v) { return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ int quad_xor2(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false); }

// q8 quantization of one 32-block held by the four lanes of a quad, eight
// elements each (lane 4m+q holds elements 8q..8q+7): d = amax/127 by IEEE
// division, q = round-half-away(x/d) clamped to [-127, 127], all 0 when d == 0.
// Every lane of the quad gets d and the block's code sum; each lane returns its
// eight codes packed in element order.
__device__ __forceinline__ void quantize_quarter(const float (&v)[8], unsigned& lo, unsigned& hi, float& d,
                                                 int& block_sum) {
  float am = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; e++) am = fmaxf(am, fabsf(v[e]));
  am = fmaxf(am, __int_as_float(quad_xor1(__float_as_int(am))));
  am = fmaxf(am, __int_as_float(quad_xor2(__float_as_int(am))));
  d = am / 127.0f;
  int s = 0;
  unsigned w[2] = {0u, 0u};
  if (d != 0.0f) {
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const int q = (int)fminf(fmaxf(roundf(v[e] / d), -127.0f), 127.0f);
      s += q;
      w[e >> 2] |= ((unsigned)(q & 0xff)) << (8 * (e & 3));
    }
  }
  lo = w[0];
  hi = w[1];
  s += quad_xor1(s);
  s += quad_xor2(s);
  block_sum = s;
}

// E4M3 code of f: round to nearest even on the fp32 mantissa, magnitudes from
// 448 up saturate to 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_code(float f) {
  const uint32_t sign = (__float_as_uint(f) >> 24) & 0x80u;
  const float a = fabsf(f);
  if (!(a < 448.0f)) return sign | 0x7Eu;
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.0f);  // subnormal: multiples of 2^-9 (8: min normal)
  const uint32_t ab = __float_as_uint(a);
  int e = (int)(ab >> 23) - 127;
  uint32_t keep = (ab >> 20) & 7u;
  const uint32_t rest = ab & 0xFFFFFu;
  keep += (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ? 1u : 0u;
  if (keep == 8u) {
    keep = 0u;
    e += 1;
  }
  if (e > 8 || (e == 8 && keep > 6u)) return sign | 0x7Eu;
  return sign | ((uint32_t)(e + 7) << 3) | keep;
}

// One 1 x 128 group by one wave, columns 2*lane and 2*lane + 1 in v: scale
// amax / 448 to *scale, codes e4m3(v / scale) to codes[0..127].
__device__ __forceinline__ void fp8_group_store(float2 v, int lane, uint8_t* __restrict__ codes,
                                                float* __restrict__ scale) {
  float am = fmaxf(fabsf(v.x), fabsf(v.y));
  for (int off = 32; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
  const float s = am / 448.0f;
  const uint32_t c0 = s != 0.0f ? e4m3_code(v.x / s) : 0u, c1 = s != 0.0f ? e4m3_code(v.y / s) : 0u;
  reinterpret_cast<uint16_t*>(codes)[lane] = (uint16_t)(c0 | (c1 << 8));
  if (lane == 0) *scale = s;
}

// Work items of a grouped GEMV of at most this many rows run in the
// small-item kernel (few registers, many workgroups per CU); larger ones in
// the kernel built for up to 16 rows.
constexpr int GROUPED_SMALL_ROWS = 2;

// The last step of a grouped plan (one workgroup, every thread calls it):
// work item it < ni is (s_ie[it], s_is[it], s_ic[it]) = (expert, first sorted
// position, rows).  The items go to `items` with those of at most
// GROUPED_SMALL_ROWS rows first (in no fixed order within a class: each
// item's outputs are its own); header[0] and header[2] receive the item count
// and the small-item count.  s_slot: LDS scratch of ni ints; s_cnt: two LDS
// ints.
__device__ inline void store_items_small_first(const int* s_ie, const int* s_is, const int* s_ic, int ni, int* s_slot,
                                               int* s_cnt, int* __restrict__ items, int* __restrict__ header) {
  const int tid = threadIdx.x, nt = blockDim.x;
  if (tid == 0) s_cnt[0] = s_cnt[1] = 0;
  __syncthreads();
  for (int it = tid; it < ni; it += nt) {
    const bool small = s_ic[it] <= GROUPED_SMALL_ROWS;
    const int c = atomicAdd(&s_cnt[small ? 0 : 1], 1);
    s_slot[it] = small ? c : -1 - c;
  }
  __syncthreads();
  const int nsmall = s_cnt[0];
  for (int it = tid; it < ni; it += nt) {
    const int sl = s_slot[it], dst = sl >= 0 ? sl : nsmall - 1 - sl;
    items[3 * dst] = s_ie[it];
    items[3 * dst + 1] = s_is[it];
    items[3 * dst + 2] = s_ic[it];
  }
  if (tid == 0) {
    header[0] = ni;
    header[2] = nsmall;
  }
}

// Workgroup `wg` of those that quantize a launch's input rows beside its
// other work: the rows' A1 in row order, four lanes per 32-block (item
// wg * blockDim.x + threadIdx.x of rows * kbp * 4; pad blocks quantize zeros).
__device__ __forceinline__ void plan_prepare_q8(const float* __restrict__ x, int rows, int64_t k,
                                                int8_t* __restrict__ xq, float* __restrict__ xd,
                                                int* __restrict__ xn, int wg) {
  const int kb = (int)kb_of(k), kbp = (int)kbp_of(k);
  const int64_t e = (int64_t)wg * blockDim.x + threadIdx.x;
  if (e >= (int64_t)rows * kbp * 4) return;  // a multiple of 64: whole waves leave
  const int q = (int)(e & 3);
  const int64_t blk = e >> 2, r = blk / kbp;
  const int b = (int)(blk - r * kbp);
  float v[8];
  if (b < kb) {
    const float4* src = reinterpret_cast<const float4*>(x + (int64_t)r * k + (int64_t)b * QK + q * 8);
    const float4 a = src[0], c = src[1];
    v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = c.x, v[5] = c.y, v[6] = c.z, v[7] = c.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; i++) v[i] = 0.0f;
  }
  unsigned lo, hi;
  float d;
  int sum;
  quantize_quarter(v, lo, hi, d, sum);
  *reinterpret_cast<uint2*>(xq + ((int64_t)r * kbp + b) * 32 + q * 8) = make_uint2(lo, hi);
  if (q == 0) {
    xd[r * kbp + b] = d;
    xn[r * kbp + b] = -8 * sum;
  }
}

// The same for the FP8 lane: the input rows' 1 x 128 groups, a wave per
// (row, group).
__device__ __forceinline__ void plan_prepare_fp8(const float* __restrict__ x, int rows, int64_t k,
                                                 uint8_t* __restrict__ fcodes, float* __restrict__ fscales, int wg) {
  const int lane = threadIdx.x % WAVE;
  const int64_t kg = k / 128, e = (int64_t)wg * (blockDim.x / WAVE) + threadIdx.x / WAVE;
  if (e >= (int64_t)rows * kg) return;  // whole waves
  const int64_t r = e / kg, g = e - r * kg;
  const float2 v = reinterpret_cast<const float2*>(x + r * k + g * 128)[lane];
  fp8_group_store(v, lane, fcodes + r * k + g * 128, fscales + e);
}

}  // namespace qg
