/*
 * qgemv_oracle.c -- plain, slow CPU definition of the few-row block-quantized
 * GEMV and its lanes.  TEST INFRASTRUCTURE ONLY: the parity tests, the smoke
 * check and the benchmark's CPU-baseline leg call it; the HIP library never
 * links, includes or calls anything here, and this file includes nothing of it.
 *
 * Sources (the pages describe the computation; none prints its arithmetic):
 *   [A] "dasLLAMA: the audio towers on the CUDA home, q8 + f16 on every GPU
 *       home" (daScript PR 4473).  Feature commit: every GPU home serves a q8
 *       lane by default and an f16 reference lane whose weights are halfwords
 *       accumulated in f32.  Router-GEMV commit: a launch holds at most eight
 *       activation rows ("columns"); longer tails must be tiled, never read
 *       past the kernel's rows.
 *   [B] "drama: the tower's one-row projections on drama_tower_gemv, in
 *       cuBLASLt's summation order" (TensorFold PR 926).  Series commits: the
 *       one-row projection streams its weights through a shared ring; the MoE
 *       combine keeps each sum in its order; routed rows are quantized in the
 *       same launch that produces them.
 *   [C] "dasLLAMA llama leg: ... batched steps past eight rows group ..."
 *       (daScript PR 4293).  Commit 16880fe: more rows than one command holds
 *       run as balanced groups in one weight pass each; commit 8624bce: the
 *       one-row form of a block format needs K in whole blocks; Not-done
 *       section: the SwiGLU step re-quantizes its output to q8.
 *
 * Formats (the plainest reading of the block format names the pages use):
 *   Q8_0: blocks of 32 weights, one fp16 scale d = fp16(max|w| / 127), codes
 *         q = round(w / d) in [-127, 127].  Canonical block: {u16 d; i8 q[32]},
 *         34 bytes, little endian.
 *   Q4_0: blocks of 32 weights, d = fp16(max|w| / 7), codes c = round(w/d)+8
 *         in [0, 15], two per byte.  Canonical block: {u16 d; u8 p[16]}, 18
 *         bytes; byte j holds c_j in its low nibble and c_{j+16} in its high one.
 *   q8 activations: each row is cut into 32-blocks; d_x = max|x| / 127 in fp32,
 *         q = round(x / d_x) clamped to [-127, 127], plus s_x = sum of q.
 *   "round" is round-half-away-from-zero; divisions are correctly rounded
 *   IEEE binary32 divisions; subnormals are kept.
 *
 * Floating-point results are accumulated in double and rounded once to float.
 * Build: gcc -O2 -ffp-contract=off, no -ffast-math (keeps IEEE division and
 * subnormals).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_Q8_0 1
#define ORC_Q4_0 2
#define ORC_Q4_K 3

#define QK 32
#define Q8_BLOCK_BYTES 34
#define Q4_BLOCK_BYTES 18
#define QK_K 256
#define Q4K_BLOCK_BYTES 144

/* ---------------------------------------------------------------- fp16 --- */
/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */

float orc_f16_to_f32(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24); /* subnormal: f * 2^-24 */
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
  }
  return (float)(sign ? -v : v);
}

/* Round a non-negative double holding a value with few significant bits to
 * the nearest integer, ties to even. */
static double round_half_even(double v) {
  double fl = floor(v);
  double diff = v - fl;
  if (diff > 0.5) return fl + 1.0;
  if (diff < 0.5) return fl;
  return fmod(fl, 2.0) == 0.0 ? fl : fl + 1.0;
}

/* fp32 -> fp16, round to nearest even.  Values past the largest finite half
 * round to infinity and set *overflow. */
uint16_t orc_f32_to_f16(float f, int* overflow) {
  if (isnan(f)) return 0x7e00;
  uint16_t sign = signbit(f) ? 0x8000 : 0;
  double a = fabs((double)f);
  if (a == 0.0) return sign;
  if (a < ldexp(1.0, -14)) {
    /* subnormal range: count units of 2^-24 */
    double q = round_half_even(a / ldexp(1.0, -24));
    return (uint16_t)(sign | (uint16_t)q); /* q == 1024 encodes the smallest normal */
  }
  int e2;
  double m = frexp(a, &e2); /* a = m * 2^e2, m in [0.5, 1) */
  int e = e2 - 1;           /* a = (2m) * 2^e, 2m in [1, 2) */
  double q = round_half_even(2.0 * m * 1024.0); /* in [1024, 2048] */
  if (q == 2048.0) {
    q = 1024.0;
    e += 1;
  }
  if (e + 15 >= 31) {
    if (overflow) *overflow = 1;
    return (uint16_t)(sign | 0x7c00);
  }
  return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(q - 1024.0));
}

void orc_f32_to_f16_array(const float* in, uint16_t* out, int64_t count, int* overflow) {
  for (int64_t i = 0; i < count; i++) out[i] = orc_f32_to_f16(in[i], overflow);
}

void orc_f16_to_f32_array(const uint16_t* in, float* out, int64_t count) {
  for (int64_t i = 0; i < count; i++) out[i] = orc_f16_to_f32(in[i]);
}

/* ------------------------------------------------------------- helpers --- */

static float block_amax(const float* v) {
  float m = 0.0f;
  for (int i = 0; i < QK; i++) {
    float a = fabsf(v[i]);
    if (a > m) m = a;
  }
  return m;
}

static int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

static void put_u16(uint8_t* p, uint16_t v) {
  p[0] = (uint8_t)(v & 0xff);
  p[1] = (uint8_t)(v >> 8);
}

static uint16_t get_u16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* ------------------------------------------------- weight quantization --- */

/* Q8_0 per 32-block: d = fp16(amax/127); q = clamp(round(w/d), -127, 127). */
int orc_quantize_q8_0(const float* w, int64_t n, int64_t k, uint8_t* blocks) {
  if (k % QK) return -1;
  int overflow = 0;
  int64_t nb = k / QK;
  for (int64_t r = 0; r < n; r++) {
    for (int64_t b = 0; b < nb; b++) {
      const float* v = w + r * k + b * QK;
      uint8_t* out = blocks + (r * nb + b) * Q8_BLOCK_BYTES;
      float d = block_amax(v) / 127.0f;
      uint16_t d16 = orc_f32_to_f16(d, &overflow);
      float dq = orc_f16_to_f32(d16);
      put_u16(out, d16);
      for (int i = 0; i < QK; i++) {
        int q = 0;
        if (dq != 0.0f) q = clampi((int)roundf(v[i] / dq), -127, 127);
        out[2 + i] = (uint8_t)(int8_t)q;
      }
    }
  }
  return overflow ? -2 : 0;
}

/* Q4_0 per 32-block: d = fp16(amax/7); c = clamp(round(w/d), -8, 7) + 8. */
int orc_quantize_q4_0(const float* w, int64_t n, int64_t k, uint8_t* blocks) {
  if (k % QK) return -1;
  int overflow = 0;
  int64_t nb = k / QK;
  for (int64_t r = 0; r < n; r++) {
    for (int64_t b = 0; b < nb; b++) {
      const float* v = w + r * k + b * QK;
      uint8_t* out = blocks + (r * nb + b) * Q4_BLOCK_BYTES;
      float d = block_amax(v) / 7.0f;
      uint16_t d16 = orc_f32_to_f16(d, &overflow);
      float dq = orc_f16_to_f32(d16);
      put_u16(out, d16);
      int c[QK];
      for (int i = 0; i < QK; i++) {
        int q = 0;
        if (dq != 0.0f) q = clampi((int)roundf(v[i] / dq), -8, 7);
        c[i] = q + 8;
      }
      for (int j = 0; j < 16; j++) out[2 + j] = (uint8_t)(c[j] | (c[j + 16] << 4));
    }
  }
  return overflow ? -2 : 0;
}

/* ------------------------------------------------ K-quant superblocks --- */
/* Q4_K ([C] commit 8624bce: a superblock format's one-row form whose K comes
 * in whole superblocks; the race bed of [C]'s body runs Q4_K_M weights).  The
 * pages do not print the format; this is the published ggml K-quant Q4_K
 * superblock, restated:
 *   256 weights = 8 sub-blocks of 32.  Bytes: fp16 d at 0, fp16 dmin at 2,
 *   twelve bytes at 4 holding eight 6-bit sub-scales sc[j] and eight 6-bit
 *   sub-mins m[j], then 128 bytes of 4-bit codes q.
 *   Scales byte s[0..11]: for j < 4, sc[j] = s[j] & 63 and m[j] = s[j+4] & 63;
 *   for j >= 4, sc[j] = (s[j+4] & 15) | (s[j-4] >> 6) << 4 and
 *   m[j] = (s[j+4] >> 4) | (s[j] >> 6) << 4.
 *   Codes: weight 64p + l (p < 4, l < 32) in the low nibble of code byte
 *   32p + l, weight 64p + 32 + l in its high nibble.
 *   Weight value: w = d * sc[j] * q - dmin * m[j], j = the weight's sub-block.
 * How a weight matrix is quantized into this format is a choice of the
 * writer's (it does not change the format): the plainest one is taken here,
 * per sub-block j (lo = min(0, min w), hi = max w):
 *   s_j = (hi - lo) / 15, mn_j = -lo                       (fp32)
 *   d = fp16(max_j s_j / 63), dmin = fp16(max_j mn_j / 63)
 *   sc[j] = min(63, round(s_j / d)) (0 when d == 0), m[j] likewise with dmin
 *   q = clamp(round((w + dmin*m[j]) / (d*sc[j])), 0, 15) (0 when d*sc[j] == 0)
 * with IEEE fp32 divisions, round half away from zero, d*sc and dmin*m exact
 * in fp32 (11-bit by 6-bit products). */

static void q4k_scale_min(const uint8_t* sb, int j, int* sc, int* m) {
  const uint8_t* s = sb + 4;
  if (j < 4) {
    *sc = s[j] & 63;
    *m = s[j + 4] & 63;
  } else {
    *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
    *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
  }
}

static void q4k_put_scales(uint8_t* sb, const int sc[8], const int m[8]) {
  uint8_t* s = sb + 4;
  for (int j = 0; j < 4; j++) {
    s[j] = (uint8_t)((sc[j] & 63) | ((sc[j + 4] >> 4) << 6));
    s[j + 4] = (uint8_t)((m[j] & 63) | ((m[j + 4] >> 4) << 6));
    s[j + 8] = (uint8_t)((sc[j + 4] & 15) | ((m[j + 4] & 15) << 4));
  }
}

/* Code (0..15) of weight i (0..255) of a superblock. */
static int q4k_code(const uint8_t* sb, int i) {
  const int p = i >> 6, l = i & 31, hi = (i >> 5) & 1;
  const uint8_t byte = sb[16 + 32 * p + l];
  return hi ? (byte >> 4) : (byte & 15);
}

int orc_quantize_q4_k(const float* w, int64_t n, int64_t k, uint8_t* blocks) {
  if (k % QK_K) return -1;
  int overflow = 0;
  const int64_t ns = k / QK_K;
  for (int64_t r = 0; r < n; r++)
    for (int64_t b = 0; b < ns; b++) {
      const float* v = w + r * k + b * QK_K;
      uint8_t* out = blocks + (r * ns + b) * Q4K_BLOCK_BYTES;
      float s[8], mn[8], smax = 0.0f, mmax = 0.0f;
      for (int j = 0; j < 8; j++) {
        float lo = 0.0f, hi = v[32 * j];
        for (int i = 0; i < 32; i++) {
          const float x = v[32 * j + i];
          if (x < lo) lo = x;
          if (x > hi) hi = x;
        }
        s[j] = (hi - lo) / 15.0f;
        mn[j] = -lo;
        if (s[j] > smax) smax = s[j];
        if (mn[j] > mmax) mmax = mn[j];
      }
      const uint16_t d16 = orc_f32_to_f16(smax / 63.0f, &overflow);
      const uint16_t m16 = orc_f32_to_f16(mmax / 63.0f, &overflow);
      const float d = orc_f16_to_f32(d16), dmin = orc_f16_to_f32(m16);
      int sc[8], m[8];
      for (int j = 0; j < 8; j++) {
        sc[j] = d != 0.0f ? clampi((int)roundf(s[j] / d), 0, 63) : 0;
        m[j] = dmin != 0.0f ? clampi((int)roundf(mn[j] / dmin), 0, 63) : 0;
      }
      put_u16(out, d16);
      put_u16(out + 2, m16);
      q4k_put_scales(out, sc, m);
      for (int j = 0; j < 8; j++) {
        const float D = d * (float)sc[j], M = dmin * (float)m[j];
        for (int i = 0; i < 32; i++) {
          const int e = 32 * j + i;
          const int q = D != 0.0f ? clampi((int)roundf((v[e] + M) / D), 0, 15) : 0;
          const int p = e >> 6, l = e & 31;
          uint8_t* byte = out + 16 + 32 * p + l;
          *byte = (uint8_t)((e & 32) ? ((*byte & 15) | (q << 4)) : ((*byte & 0xF0) | q));
        }
      }
    }
  return overflow ? -2 : 0;
}

/* Sub-block j's scale d * sc[j] and offset dmin * m[j] of a superblock (exact). */
static void q4k_dm(const uint8_t* sb, int j, double* D, double* M) {
  int sc, m;
  q4k_scale_min(sb, j, &sc, &m);
  *D = (double)orc_f16_to_f32(get_u16(sb)) * (double)sc;
  *M = (double)orc_f16_to_f32(get_u16(sb + 2)) * (double)m;
}

/* Code i of a canonical block, as the signed integer it stands for. */
static int block_code(int fmt, const uint8_t* blk, int i) {
  if (fmt == ORC_Q8_0) return (int)(int8_t)blk[2 + i];
  int byte = blk[2 + (i & 15)];
  int c = (i < 16) ? (byte & 0xf) : (byte >> 4);
  return c - 8;
}

static int block_bytes(int fmt) { return fmt == ORC_Q8_0 ? Q8_BLOCK_BYTES : Q4_BLOCK_BYTES; }

/* Dequantized weights w_hat = d * code (Q4_K: d*sc*q - dmin*m), in double (exact). */
int orc_dequantize(int fmt, const uint8_t* blocks, int64_t n, int64_t k, double* w_hat) {
  if (fmt == ORC_Q4_K) {
    if (k % QK_K) return -1;
    const int64_t ns = k / QK_K;
    for (int64_t r = 0; r < n; r++)
      for (int64_t b = 0; b < ns; b++) {
        const uint8_t* sb = blocks + (r * ns + b) * Q4K_BLOCK_BYTES;
        for (int i = 0; i < QK_K; i++) {
          double D, M;
          q4k_dm(sb, i >> 5, &D, &M);
          w_hat[r * k + b * QK_K + i] = D * (double)q4k_code(sb, i) - M;
        }
      }
    return 0;
  }
  if (k % QK || (fmt != ORC_Q8_0 && fmt != ORC_Q4_0)) return -1;
  int64_t nb = k / QK;
  int bb = block_bytes(fmt);
  for (int64_t r = 0; r < n; r++)
    for (int64_t b = 0; b < nb; b++) {
      const uint8_t* blk = blocks + (r * nb + b) * bb;
      double d = (double)orc_f16_to_f32(get_u16(blk));
      for (int i = 0; i < QK; i++) w_hat[r * k + b * QK + i] = d * (double)block_code(fmt, blk, i);
    }
  return 0;
}

/* ------------------------------------------- activation quantization --- */

/* Per row and 32-block: d_x = amax/127 (fp32 division); q = 0 when d_x == 0,
 * else clamp(round(x / d_x), -127, 127) with a true fp32 division; s_x = sum q. */
int orc_quantize_acts(const float* x, int rows, int64_t k, int8_t* qx, float* dx, int32_t* sx) {
  if (k % QK) return -1;
  int64_t nb = k / QK;
  for (int r = 0; r < rows; r++)
    for (int64_t b = 0; b < nb; b++) {
      const float* v = x + (int64_t)r * k + b * QK;
      float d = block_amax(v) / 127.0f;
      int32_t s = 0;
      for (int i = 0; i < QK; i++) {
        int q = 0;
        if (d != 0.0f) q = clampi((int)roundf(v[i] / d), -127, 127);
        qx[(int64_t)r * k + b * QK + i] = (int8_t)q;
        s += q;
      }
      dx[(int64_t)r * nb + b] = d;
      if (sx) sx[(int64_t)r * nb + b] = s;
    }
  return 0;
}

/* ---------------------------------------------------------- block dots --- */

/* isum[r][n][b] = sum_i code(w[n], b, i) * qx[r][32b + i], exact in int64,
 * stored as int32 (|isum| <= 32 * 127 * 127 fits).  Q4_K: b is a 32-weight
 * sub-block and the code its raw 4-bit q (0..15); the sub-min's share,
 * dmin * m * sum(qx), is not part of the integer dot. */
int orc_blockdots(int fmt, const uint8_t* blocks, int64_t n, int64_t k, const int8_t* qx, int rows,
                  int32_t* isum) {
  if (fmt == ORC_Q4_K) {
    if (k % QK_K) return -1;
    const int64_t ns = k / QK_K, nb = k / QK;
    for (int r = 0; r < rows; r++)
      for (int64_t o = 0; o < n; o++)
        for (int64_t b = 0; b < nb; b++) {
          const uint8_t* sb = blocks + (o * ns + b / 8) * Q4K_BLOCK_BYTES;
          int64_t s = 0;
          for (int i = 0; i < QK; i++)
            s += (int64_t)q4k_code(sb, (int)(b % 8) * 32 + i) * (int64_t)qx[(int64_t)r * k + b * QK + i];
          isum[((int64_t)r * n + o) * nb + b] = (int32_t)s;
        }
    return 0;
  }
  if (k % QK || (fmt != ORC_Q8_0 && fmt != ORC_Q4_0)) return -1;
  int64_t nb = k / QK;
  int bb = block_bytes(fmt);
  for (int r = 0; r < rows; r++)
    for (int64_t o = 0; o < n; o++)
      for (int64_t b = 0; b < nb; b++) {
        const uint8_t* blk = blocks + (o * nb + b) * bb;
        int64_t s = 0;
        for (int i = 0; i < QK; i++)
          s += (int64_t)block_code(fmt, blk, i) * (int64_t)qx[(int64_t)r * k + b * QK + i];
        isum[((int64_t)r * n + o) * nb + b] = (int32_t)s;
      }
  return 0;
}

/* -------------------------------------------------------- thread pool --- */

typedef void (*range_fn)(void* ctx, int64_t lo, int64_t hi);
typedef struct {
  range_fn fn;
  void* ctx;
  int64_t lo, hi;
} range_job;

static void* range_thread(void* p) {
  range_job* j = (range_job*)p;
  j->fn(j->ctx, j->lo, j->hi);
  return NULL;
}

/* Split [0, count) into `threads` contiguous parts, one per pthread. */
static void parallel_for(int64_t count, int threads, range_fn fn, void* ctx) {
  if (threads <= 1 || count < 2) {
    fn(ctx, 0, count);
    return;
  }
  if (threads > count) threads = (int)count;
  pthread_t* tid = (pthread_t*)malloc(sizeof(pthread_t) * threads);
  range_job* jobs = (range_job*)malloc(sizeof(range_job) * threads);
  for (int t = 0; t < threads; t++) {
    jobs[t].fn = fn;
    jobs[t].ctx = ctx;
    jobs[t].lo = count * t / threads;
    jobs[t].hi = count * (t + 1) / threads;
    pthread_create(&tid[t], NULL, range_thread, &jobs[t]);
  }
  for (int t = 0; t < threads; t++) pthread_join(tid[t], NULL);
  free(tid);
  free(jobs);
}

/* --------------------------------------------------- quantized GEMV --- */

typedef struct {
  int fmt;
  const uint8_t* blocks;
  int64_t n, k, nb;
  const int8_t* qx;
  const float* dx;
  int rows;
  const int64_t* sel; /* output rows to compute, or NULL for all */
  int64_t out_n;      /* row stride of y */
  float* y;
} qgemv_ctx;

/* y[r][o] = sum_b d_w[o][b] * d_x[r][b] * isum[r][o][b], ascending b, in
 * double, rounded once to float.  Q4_K: the sum over 32-weight sub-blocks b of
 * d_x[r][b] * (D_b * isum_b - M_b * sum(qx of block b)), D_b = d * sc, M_b =
 * dmin * m of b's superblock -- the dot of the dequantized weights with the
 * dequantized activations, sub-block by sub-block. */
static void qgemv_range(void* p, int64_t lo, int64_t hi) {
  qgemv_ctx* c = (qgemv_ctx*)p;
  int bb = block_bytes(c->fmt);
  for (int64_t t = lo; t < hi; t++) {
    int64_t o = c->sel ? c->sel[t] : t;
    if (c->fmt == ORC_Q4_K) {
      const int64_t ns = c->k / QK_K;
      for (int r = 0; r < c->rows; r++) {
        double acc = 0.0;
        for (int64_t b = 0; b < c->nb; b++) {
          const uint8_t* sb = c->blocks + (o * ns + b / 8) * Q4K_BLOCK_BYTES;
          const int8_t* q = c->qx + (int64_t)r * c->k + b * QK;
          int64_t s = 0, xs = 0;
          for (int i = 0; i < QK; i++) {
            s += (int64_t)q4k_code(sb, (int)(b % 8) * 32 + i) * (int64_t)q[i];
            xs += q[i];
          }
          double D, M;
          q4k_dm(sb, (int)(b % 8), &D, &M);
          acc += (double)c->dx[(int64_t)r * c->nb + b] * (D * (double)s - M * (double)xs);
        }
        c->y[(int64_t)r * c->out_n + t] = (float)acc;
      }
      continue;
    }
    for (int r = 0; r < c->rows; r++) {
      double acc = 0.0;
      for (int64_t b = 0; b < c->nb; b++) {
        const uint8_t* blk = c->blocks + (o * c->nb + b) * bb;
        const int8_t* q = c->qx + (int64_t)r * c->k + b * QK;
        int64_t s = 0;
        for (int i = 0; i < QK; i++) s += (int64_t)block_code(c->fmt, blk, i) * (int64_t)q[i];
        double dw = (double)orc_f16_to_f32(get_u16(blk));
        double dxv = (double)c->dx[(int64_t)r * c->nb + b];
        acc += dw * dxv * (double)s;
      }
      c->y[(int64_t)r * c->out_n + t] = (float)acc;
    }
  }
}

static int qgemv_common(int fmt, const uint8_t* blocks, int64_t n, int64_t k, const float* x, int rows,
                        const int64_t* sel, int64_t nsel, float* y, int threads) {
  if (k % QK || (fmt != ORC_Q8_0 && fmt != ORC_Q4_0 && fmt != ORC_Q4_K) || rows < 0) return -1;
  if (fmt == ORC_Q4_K && k % QK_K) return -1;
  int64_t nb = k / QK;
  int8_t* qx = (int8_t*)malloc((size_t)(rows * k) + 1);
  float* dx = (float*)malloc(sizeof(float) * (size_t)(rows * nb) + 1);
  orc_quantize_acts(x, rows, k, qx, dx, NULL);
  qgemv_ctx c = {fmt, blocks, n, k, nb, qx, dx, rows, sel, sel ? nsel : n, y};
  parallel_for(sel ? nsel : n, threads, qgemv_range, &c);
  free(qx);
  free(dx);
  return 0;
}

/* Quantized GEMV from fp32 activations: A1 then A3/A4 per output element. */
int orc_gemv_q(int fmt, const uint8_t* blocks, int64_t n, int64_t k, const float* x, int rows, float* y,
               int threads) {
  return qgemv_common(fmt, blocks, n, k, x, rows, NULL, 0, y, threads);
}

/* Same, for a chosen subset of output rows: y is [rows][nsel]. */
int orc_gemv_q_rows(int fmt, const uint8_t* blocks, int64_t n, int64_t k, const float* x, int rows,
                    const int64_t* sel, int64_t nsel, float* y, int threads) {
  for (int64_t i = 0; i < nsel; i++)
    if (sel[i] < 0 || sel[i] >= n) return -1;
  return qgemv_common(fmt, blocks, n, k, x, rows, sel, nsel, y, threads);
}

/* ------------------------------------------------------------ FP8 lane --- */
/* Block-FP8 ([B] backbone section: block-FP8 expert weights, dynamic 1 x 128
 * FP8 activation groups; neither the element format nor the weight block is
 * printed there -- the plainest reading is the OCP 8-bit format E4M3 (4
 * exponent bits, bias 7, 3 mantissa bits, largest finite 448, no infinities),
 * fp32 scales amax / 448, activation groups of 128 consecutive k of one row,
 * and weight blocks of 128 rows x 128 k).  Encoding: round to nearest, ties
 * to even, magnitudes past 448 saturate to 448. */
#define FP8_GROUP 128
#define FP8_MAX 448.0

uint8_t orc_e4m3_encode(float f) {
  const uint8_t sign = signbit(f) ? 0x80 : 0x00;
  double a = fabs((double)f);
  if (a >= FP8_MAX) return sign | 0x7E; /* saturate (0x7F is NaN) */
  if (a < ldexp(1.0, -6)) {             /* subnormal: multiples of 2^-9 */
    int m = (int)round_half_even(a * 512.0);
    return sign | (uint8_t)m; /* m == 8 is the smallest normal, 0x08 */
  }
  int e;
  double fr = frexp(a, &e); /* a = fr * 2^e, fr in [0.5, 1) */
  e -= 1;                   /* a = (2 fr) * 2^e, 2 fr in [1, 2) */
  int m = (int)round_half_even((2.0 * fr - 1.0) * 8.0);
  if (m == 8) {
    m = 0;
    e += 1;
  }
  if (e > 8 || (e == 8 && m > 6)) return sign | 0x7E;
  return sign | (uint8_t)(((e + 7) << 3) | m);
}

void orc_e4m3_encode_array(const float* in, uint8_t* out, int64_t count) {
  for (int64_t i = 0; i < count; i++) out[i] = orc_e4m3_encode(in[i]);
}

double orc_e4m3_decode(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  const double v = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* Quantize a group: s = amax / 448 (IEEE fp32 division), codes = e4m3(v / s)
 * with the fp32 quotient; all zero when amax == 0. */
static float fp8_group(const float* v, int64_t count, int64_t stride, uint8_t* codes, int64_t cstride) {
  float am = 0.0f;
  for (int64_t i = 0; i < count; i++) {
    float a = fabsf(v[i * stride]);
    if (a > am) am = a;
  }
  volatile float s = am / 448.0f;
  for (int64_t i = 0; i < count; i++) codes[i * cstride] = s != 0.0f ? orc_e4m3_encode(v[i * stride] / s) : 0;
  return s;
}

/* Weights [n][k] -> codes [n][k] + scales [ceil(n/128)][k/128] (row-major),
 * one scale per 128 x 128 block (the last block row may be shorter). */
int orc_quantize_fp8_weights(const float* w, int64_t n, int64_t k, uint8_t* codes, float* scales) {
  if (k % FP8_GROUP || n < 1) return -1;
  const int64_t kg = k / FP8_GROUP, nb = (n + FP8_GROUP - 1) / FP8_GROUP;
  for (int64_t bi = 0; bi < nb; bi++)
    for (int64_t g = 0; g < kg; g++) {
      const int64_t r0 = bi * FP8_GROUP, r1 = r0 + FP8_GROUP < n ? r0 + FP8_GROUP : n;
      float am = 0.0f;
      for (int64_t o = r0; o < r1; o++)
        for (int64_t i = 0; i < FP8_GROUP; i++) {
          float a = fabsf(w[o * k + g * FP8_GROUP + i]);
          if (a > am) am = a;
        }
      volatile float s = am / 448.0f;
      scales[bi * kg + g] = s;
      for (int64_t o = r0; o < r1; o++)
        for (int64_t i = 0; i < FP8_GROUP; i++) {
          const int64_t e = o * k + g * FP8_GROUP + i;
          codes[e] = s != 0.0f ? orc_e4m3_encode(w[e] / s) : 0;
        }
    }
  return 0;
}

/* Activations [rows][k] -> codes [rows][k] + scales [rows][k/128]. */
int orc_quantize_fp8_acts(const float* x, int rows, int64_t k, uint8_t* codes, float* scales) {
  if (k % FP8_GROUP) return -1;
  const int64_t kg = k / FP8_GROUP;
  for (int r = 0; r < rows; r++)
    for (int64_t g = 0; g < kg; g++)
      scales[r * kg + g] = fp8_group(x + r * k + g * FP8_GROUP, FP8_GROUP, 1, codes + r * k + g * FP8_GROUP, 1);
  return 0;
}

typedef struct {
  const uint8_t* wc;
  const float* ws;
  int64_t n, k, kg;
  const uint8_t* xc;
  const float* xs;
  int rows;
  const int64_t* sel;
  int64_t out_n;
  float* y;
} fp8_ctx;

/* y[r][o] = sum_g s_w[o/128][g] * s_x[r][g] * sum_{k in g} w(o,k) x(r,k),
 * the group sums exact (products of two E4M3 values and their sum of 128 fit
 * a double exactly), ascending g in double, rounded once to float. */
static void fp8_range(void* p, int64_t lo, int64_t hi) {
  fp8_ctx* c = (fp8_ctx*)p;
  for (int64_t t = lo; t < hi; t++) {
    const int64_t o = c->sel ? c->sel[t] : t;
    for (int r = 0; r < c->rows; r++) {
      double acc = 0.0;
      for (int64_t g = 0; g < c->kg; g++) {
        double dot = 0.0;
        for (int i = 0; i < FP8_GROUP; i++) {
          const int64_t e = g * FP8_GROUP + i;
          dot += orc_e4m3_decode(c->wc[o * c->k + e]) * orc_e4m3_decode(c->xc[(int64_t)r * c->k + e]);
        }
        acc += (double)c->ws[(o / FP8_GROUP) * c->kg + g] * (double)c->xs[(int64_t)r * c->kg + g] * dot;
      }
      c->y[(int64_t)r * c->out_n + t] = (float)acc;
    }
  }
}

/* FP8 GEMV from fp32 activations (quantized per 1 x 128 group first); with
 * sel, only the output rows sel[0..nsel) (y is [rows][nsel]). */
int orc_gemv_fp8(const uint8_t* wcodes, const float* wscales, int64_t n, int64_t k, const float* x, int rows,
                 const int64_t* sel, int64_t nsel, float* y, int threads) {
  if (k % FP8_GROUP || rows < 0) return -1;
  for (int64_t i = 0; sel && i < nsel; i++)
    if (sel[i] < 0 || sel[i] >= n) return -1;
  const int64_t kg = k / FP8_GROUP;
  uint8_t* xc = (uint8_t*)malloc((size_t)(rows * k) + 1);
  float* xs = (float*)malloc(sizeof(float) * (size_t)(rows * kg) + 1);
  orc_quantize_fp8_acts(x, rows, k, xc, xs);
  fp8_ctx c = {wcodes, wscales, n, k, kg, xc, xs, rows, sel, sel ? nsel : n, y};
  parallel_for(sel ? nsel : n, threads, fp8_range, &c);
  free(xc);
  free(xs);
  return 0;
}

/* ------------------------------------------------------------ f16 lane --- */

typedef struct {
  const uint16_t* w;
  int64_t n, k;
  const float* x;
  int rows;
  const int64_t* sel;
  int64_t out_n;
  float* y;
} f16_ctx;

/* y[r][o] = sum_k f32(w16[o][k]) * x[r][k], in double, rounded once. */
static void f16_range(void* p, int64_t lo, int64_t hi) {
  f16_ctx* c = (f16_ctx*)p;
  for (int64_t t = lo; t < hi; t++) {
    int64_t o = c->sel ? c->sel[t] : t;
    for (int r = 0; r < c->rows; r++) {
      double acc = 0.0;
      for (int64_t i = 0; i < c->k; i++)
        acc += (double)orc_f16_to_f32(c->w[o * c->k + i]) * (double)c->x[(int64_t)r * c->k + i];
      c->y[(int64_t)r * c->out_n + t] = (float)acc;
    }
  }
}

int orc_gemv_f16(const uint16_t* w, int64_t n, int64_t k, const float* x, int rows, float* y, int threads) {
  f16_ctx c = {w, n, k, x, rows, NULL, n, y};
  parallel_for(n, threads, f16_range, &c);
  return 0;
}

int orc_gemv_f16_rows(const uint16_t* w, int64_t n, int64_t k, const float* x, int rows, const int64_t* sel,
                      int64_t nsel, float* y, int threads) {
  for (int64_t i = 0; i < nsel; i++)
    if (sel[i] < 0 || sel[i] >= n) return -1;
  f16_ctx c = {w, n, k, x, rows, sel, nsel, y};
  parallel_for(nsel, threads, f16_range, &c);
  return 0;
}

/* ------------------------------------------- grouped routed experts --- */

/* For each assignment j: y[j] = W_{expert[j]} . q8(x[x_index[j]]).  Experts
 * are stacked [E][n][k/32] canonical Q8_0 blocks.  An assignment naming an
 * expert or an activation row out of range is skipped (its y row untouched);
 * the count of such entries is returned. */
int orc_gemv_q8_0_grouped(const uint8_t* blocks, int64_t n_experts, int64_t n, int64_t k, const float* x,
                          int x_rows, const int32_t* expert, const int32_t* x_index, int m, float* y) {
  if (k % QK) return -1;
  int bad = 0;
  int64_t expert_bytes = n * (k / QK) * Q8_BLOCK_BYTES;
  for (int j = 0; j < m; j++) {
    if (expert[j] < 0 || expert[j] >= n_experts || x_index[j] < 0 || x_index[j] >= x_rows) {
      bad++;
      continue;
    }
    qgemv_common(ORC_Q8_0, blocks + expert[j] * expert_bytes, n, k, x + (int64_t)x_index[j] * k, 1, NULL, 0,
                 y + (int64_t)j * n, 1);
  }
  return bad;
}

/* ---------------------------------------------------------- MoE glue --- */

/* Softmax over the E logits of each row (double, max subtracted), then the
 * topk experts by logit, ties to the lower expert index, in descending order.
 * The combine weight of a pick is its softmax probability over all E. */
int orc_route_topk(const float* logits, int rows, int64_t E, int topk, int32_t* expert, double* p) {
  if (topk > E) return -1;
  double* pr = (double*)malloc(sizeof(double) * (size_t)E);
  char* taken = (char*)malloc((size_t)E);
  for (int r = 0; r < rows; r++) {
    const float* l = logits + (int64_t)r * E;
    double mx = -INFINITY;
    for (int64_t e = 0; e < E; e++)
      if ((double)l[e] > mx) mx = (double)l[e];
    double sum = 0.0;
    for (int64_t e = 0; e < E; e++) {
      pr[e] = exp((double)l[e] - mx);
      sum += pr[e];
    }
    for (int64_t e = 0; e < E; e++) pr[e] /= sum;
    memset(taken, 0, (size_t)E);
    for (int s = 0; s < topk; s++) {
      int64_t best = -1;
      for (int64_t e = 0; e < E; e++) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict: ties keep the lower index */
      }
      taken[best] = 1;
      expert[(int64_t)r * topk + s] = (int32_t)best;
      p[(int64_t)r * topk + s] = pr[best];
    }
  }
  free(pr);
  free(taken);
  return 0;
}

/* h = silu(g) * u with silu(g) = g / (1 + exp(-g)), in double, cast to float. */
void orc_swiglu(const float* g, const float* u, int64_t count, float* h) {
  for (int64_t i = 0; i < count; i++) {
    double gv = (double)g[i];
    h[i] = (float)(gv / (1.0 + exp(-gv)) * (double)u[i]);
  }
}

/* Residual add and RMS norm, the step before a projection group ([B] series
 * commits: the add + norm launch also emits the activation quantization that
 * a separate pass used to produce, with equal results; [C] "Not done" names a
 * requant arm in its add+rms family).
 *   h = x + residual (fp32 add; residual may be NULL: h = x)
 *   y = h / sqrt(mean(h^2) + eps) * gamma, evaluated in double.
 * h is returned in fp32 (one correctly rounded add, the same on any device),
 * y in double; the q8 codes of the normed rows are A1 of the fp32 y. */
void orc_add_rmsnorm(const float* x, const float* residual, const float* gamma, double eps, int rows, int64_t k,
                     float* h, double* y) {
  for (int r = 0; r < rows; r++) {
    const float* xr = x + (int64_t)r * k;
    float* hr = h + (int64_t)r * k;
    double ss = 0.0;
    for (int64_t i = 0; i < k; i++) {
      hr[i] = residual ? xr[i] + residual[(int64_t)r * k + i] : xr[i];
      ss += (double)hr[i] * (double)hr[i];
    }
    const double inv = 1.0 / sqrt(ss / (double)k + eps);
    for (int64_t i = 0; i < k; i++) y[(int64_t)r * k + i] = (double)hr[i] * inv * (double)gamma[i];
  }
}

/* One expert's FFN on one activation row: gate and up (n=ffn, k=hidden),
 * SwiGLU, q8 re-quantization of h, down (n=hidden, k=ffn). */
static void expert_ffn(const uint8_t* gate, const uint8_t* up, const uint8_t* down, int64_t hidden, int64_t ffn,
                       const float* xrow, float* out, float* g, float* u, float* h) {
  qgemv_common(ORC_Q8_0, gate, ffn, hidden, xrow, 1, NULL, 0, g, 1);
  qgemv_common(ORC_Q8_0, up, ffn, hidden, xrow, 1, NULL, 0, u, 1);
  orc_swiglu(g, u, ffn, h);
  qgemv_common(ORC_Q8_0, down, hidden, ffn, h, 1, NULL, 0, out, 1);
}

/* Routed MoE decode step with one ungated shared expert.
 *   logits = f16 GEMV(router, x); topk picks per row; each pick's expert FFN;
 *   y[r] = sum over picks (in slot order) of p * o, then + the shared FFN. */
int orc_moe_step(const float* x, int rows, int64_t hidden, const uint16_t* router, int64_t E, int topk,
                 const uint8_t* gate, const uint8_t* up, const uint8_t* down, int64_t ffn, const uint8_t* sgate,
                 const uint8_t* sup, const uint8_t* sdown, float* y, int32_t* sel_expert, double* sel_p,
                 float* logits_out) {
  if (hidden % QK || ffn % QK) return -1;
  float* logits = (float*)malloc(sizeof(float) * (size_t)(rows * E));
  orc_gemv_f16(router, E, hidden, x, rows, logits, 1);
  if (logits_out) memcpy(logits_out, logits, sizeof(float) * (size_t)(rows * E));
  orc_route_topk(logits, rows, E, topk, sel_expert, sel_p);
  int64_t gu_bytes = ffn * (hidden / QK) * Q8_BLOCK_BYTES;
  int64_t dn_bytes = hidden * (ffn / QK) * Q8_BLOCK_BYTES;
  float* g = (float*)malloc(sizeof(float) * (size_t)ffn);
  float* u = (float*)malloc(sizeof(float) * (size_t)ffn);
  float* h = (float*)malloc(sizeof(float) * (size_t)ffn);
  float* o = (float*)malloc(sizeof(float) * (size_t)hidden);
  double* acc = (double*)malloc(sizeof(double) * (size_t)hidden);
  for (int r = 0; r < rows; r++) {
    const float* xr = x + (int64_t)r * hidden;
    for (int64_t i = 0; i < hidden; i++) acc[i] = 0.0;
    for (int s = 0; s < topk; s++) {
      int64_t e = sel_expert[(int64_t)r * topk + s];
      double pe = sel_p[(int64_t)r * topk + s];
      expert_ffn(gate + e * gu_bytes, up + e * gu_bytes, down + e * dn_bytes, hidden, ffn, xr, o, g, u, h);
      for (int64_t i = 0; i < hidden; i++) acc[i] += pe * (double)o[i];
    }
    expert_ffn(sgate, sup, sdown, hidden, ffn, xr, o, g, u, h);
    for (int64_t i = 0; i < hidden; i++) y[(int64_t)r * hidden + i] = (float)(acc[i] + (double)o[i]);
  }
  free(logits);
  free(g);
  free(u);
  free(h);
  free(o);
  free(acc);
  return 0;
}
