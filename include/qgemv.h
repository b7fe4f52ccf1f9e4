/*
 * qgemv.h -- C ABI of the few-row block-quantized GEMV library for MI355X
 * (gfx950), built as block_quantized_few_amd/libqgemv.so.
 *
 * What it computes.  The decode-time projection of 1..16 activation rows
 * against one weight matrix W [n][k], y[r][o] = sum_k W[o][k] * x[r][k], in the
 * two device lanes of the dasLLAMA audio-towers page (feature commit): the q8
 * lane, where block-quantized weights meet q8-quantized activations through
 * exact integer block dots, and the f16 lane, halfword weights accumulated in
 * fp32.  Rows past eight are tiled inside the callee, in one weight pass, so a
 * caller can never launch rows past the kernel's tile (router-GEMV commit of
 * the same page; balanced groups past eight rows, commit 16880fe of the
 * dasLLAMA llama-leg page).  A grouped variant streams each routed expert
 * once for all rows routed to it (llama-leg page: the routed model's N-row
 * command).
 *
 * Formats.
 *   Q8_0: 32-weight blocks, fp16 scale d = fp16(max|w|/127), int8 codes
 *         q = round-half-away(w/d) in [-127, 127].  Canonical block
 *         {uint16 d; int8 q[32]} = 34 bytes.
 *   Q4_0: 32-weight blocks, d = fp16(max|w|/7), 4-bit codes c = q + 8 in
 *         [0, 15]; canonical block {uint16 d; uint8 p[16]} = 18 bytes, byte j
 *         holding c_j (low nibble) and c_{j+16} (high nibble).
 *   q8 activations: per row and 32-block, d_x = max|x|/127 (IEEE fp32
 *         division), q = round-half-away(x/d_x) clamped to [-127, 127] (0 when
 *         d_x == 0), s_x = sum q.  Quantized on the device, bit-exact with a
 *         plain CPU evaluation of that definition.
 *   y[r][o] = sum_b d_w[o][b] * d_x[r][b] * isum[r][o][b], where isum is the
 *         exact int32 dot of block b's codes (Q4_0 codes stand for c - 8).
 *         The fp32 summation order is fixed per output and does not depend on
 *         `rows`: a row computed inside a batch of 16 has the same bits as the
 *         row computed alone.
 *
 *   Q4_K: K-quant superblocks of 256 weights (the llama-leg page's Q4_K_M
 *         race bed and its commit 8624bce, a superblock format's one-row form
 *         with K in whole superblocks; the pages do not print the format, so
 *         the published ggml Q4_K layout is taken): canonical block
 *         {uint16 d; uint16 dmin; uint8 scales[12]; uint8 qs[128]} = 144
 *         bytes, eight 32-weight sub-blocks j with 6-bit sub-scale sc[j] and
 *         sub-min m[j] (for j < 4: sc = scales[j] & 63, m = scales[j+4] & 63;
 *         for j >= 4: sc = (scales[j+4] & 15) | (scales[j-4] >> 6) << 4,
 *         m = (scales[j+4] >> 4) | (scales[j] >> 6) << 4), weight 64p + l in
 *         the low nibble of qs[32p + l] and weight 64p + 32 + l in its high
 *         nibble (p < 4, l < 32); w = d * sc[j] * q - dmin * m[j].  y adds per
 *         sub-block d_x * (d*sc * isum - dmin*m * s_x), isum the exact int32
 *         dot of the raw codes q (0..15).  k must be a multiple of 256.
 *
 * Device image.  Weights live on the device in the library's own layout,
 * made either by qg_pack_image (from canonical blocks, on the host) or by
 * qg_quantize_weights (from fp32 weights, on the device): rows in tiles of 16,
 * each tile storing its blocks one after another with the 16 rows of a block
 * side by side, codes and fp16 scales in separate planes.  Rows are padded to
 * a multiple of 16 and blocks to a multiple of 16 (512 weights) with zeros;
 * for n % 16 == 0 and k % 512 == 0 the image holds exactly the canonical bytes
 * per weight.
 *
 * F16 image.  The f16 lane reads halfword weights from an image too, made by
 * qg_f16_image (device) or qg_pack_image(QG_FMT_F16, ...) (host) from the
 * row-major [n][k] halfword matrix: rows in tiles of 16, columns in steps of
 * 32; tile t, step s is one 1 KB block whose 16-byte chunk l = i + 16*j holds
 * w[16t + i][32s + 8j .. 32s + 8j + 7] (j = 0..3), steps of a tile in order,
 * tiles in order, rows past n and columns past k zero.  That is the operand
 * order of the matrix core's 16x16x32 halfword product, so one wave load is
 * 1 KB of consecutive bytes.  Size: ceil(n/16) * ceil(k/32) * 1024 bytes.
 *
 * FP8 lane (block-FP8 weights, dynamic 1 x 128 FP8 activation groups: the
 * drama page's backbone section).  Elements are OCP E4M3 (largest finite 448;
 * round to nearest even, saturating).  Weights: one fp32 scale amax/448 per
 * block of 128 rows x 128 columns, codes e4m3(w / scale); canonical form
 * codes [n][k] bytes followed by the scales [ceil(n/128)][k/128] fp32.
 * Activations: per row and group of 128 columns, scale amax/448 and codes
 * e4m3(x / scale) (qg_prepare_fp8; workspace codes [rows][k], then, 256-byte
 * aligned, scales [rows][k/128]).  y[r][o] = sum_g s_w s_x (sum over the
 * group's 128 code products), the group sum from the matrix core's 16x16x128
 * FP8 product in fp32.  Image: 16-row tiles of 128-column groups, 2 KB per
 * (tile, group) in which lane l = i + 16j finds the codes of row 16t + i,
 * columns 128g + 32j .. + 31, the first 16 at byte 16l and the other 16 at
 * byte 1024 + 16l; then (256-byte aligned) the scales as in the canonical
 * form.  k must be a multiple of 128.
 *
 * Conventions.
 *   - Pointers are device pointers unless marked (host).  `stream` is a
 *     hipStream_t (NULL = the null stream).  Device calls enqueue work on
 *     `stream` and return without synchronizing, except the functions marked
 *     "synchronizes".
 *   - The caller owns every buffer; the library allocates no device memory,
 *     frees nothing and keeps no pointer past a return.
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     negative status means nothing was launched and no output was touched;
 *     qg_last_error_detail() then names the argument and its value (per
 *     thread).  QG_ELAUNCH reports a HIP launch failure.
 *   - rows == 0 is a successful no-op.  rows > 16 is QG_EROWS, never a
 *     silently truncated tile.
 *   - Shapes: n >= 1; k % 32 == 0 (q8 lane) or k % 8 == 0 (f16 lane).
 *   - Alignment: images and workspaces 256 bytes; x, f16 weights and q8 row
 *     buffers 16 bytes; y 4 bytes.
 *   - x must be finite; the result for NaN/Inf inputs is unspecified.
 *   - Calls are stateless and re-entrant; two calls that share a workspace
 *     must be ordered on one stream.
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* qg_stream; /* a hipStream_t */

enum {
  QG_OK = 0,
  QG_EINVAL = -1,     /* null pointer, unknown format, bad count */
  QG_ESHAPE = -2,     /* n, k or another extent out of range */
  QG_EROWS = -3,      /* rows outside 0..16 */
  QG_EALIGN = -4,     /* a pointer misses its alignment */
  QG_EWORKSPACE = -5, /* workspace smaller than the size query returned */
  QG_ELAUNCH = -6,    /* a HIP call or kernel launch failed */
  QG_EDEVICE = -7     /* the current device is not a gfx950 GPU */
};

enum { QG_FMT_Q8_0 = 1, QG_FMT_Q4_0 = 2, QG_FMT_F16 = 3, QG_FMT_FP8 = 4, QG_FMT_Q4_K = 5 };

#define QG_MAX_ROWS 16        /* activation rows per GEMV call */
#define QG_MAX_PREP_ROWS 8192 /* rows one qg_prepare_rows call quantizes */
#define QG_MAX_ASSIGN 2048    /* assignments per grouped call */
#define QG_MAX_SET 8          /* projections per qgemv_set call */
#define QG_FUSED_ROWS 2       /* up to this many rows are quantized inside the GEMV launch */
#define QG_NOALLOC_SCRATCH_BYTES (1u << 20) /* the static workspace of qgemv_q8_0_noalloc, per GPU */

/* ------------------------------------------------------------ host only --- */

/* Bytes of the device image of an n x k matrix in `fmt` (Q8_0, Q4_0, F16,
 * FP8: the padded layouts above).  Returns 0 for an invalid format or shape,
 * k included: K must come in whole blocks of the format (the llama-leg page,
 * commit 8624bce: a block format's one-row form needs K in whole blocks). */
size_t qg_image_bytes(int fmt, int64_t n, int64_t k);

/* Host -> host.  Converts canonical blocks (Q8_0 / Q4_0, n * k/32 blocks, row
 * major; F16: the row-major [n][k] halfwords, k % 8 == 0) to the device
 * layout in `image` (qg_image_bytes bytes, host memory; copy it to the device
 * afterwards).  Padding is written as zeros.  Both buffers belong to the
 * caller; QG_EINVAL / QG_ESHAPE on a null pointer, unknown format or bad
 * shape, nothing written then. */
int qg_pack_image(int fmt, const void* blocks, int64_t n, int64_t k, void* image);

/* Host -> host inverse of qg_pack_image (padding is dropped). */
int qg_unpack_image(int fmt, const void* image, int64_t n, int64_t k, void* blocks);

/* Bytes of the FP8 workspace of `rows` activation rows of length k (k a
 * multiple of 128); 0 for an invalid shape. */
size_t qg_fp8_workspace_bytes(int rows, int64_t k);

/* Bytes of the workspace that holds `rows` quantized activation rows of
 * length k (codes, scales and code sums) in the order a GEMV of `rows` rows
 * reads (row order at 1-2 rows, pair order at 3-16).  q8 activations are the
 * audio-towers page's q8 lane (feature commit): int8 codes in 32-blocks with
 * one scale each.  0 for an invalid shape (k not whole blocks, rows < 1). */
size_t qg_workspace_bytes(int rows, int64_t k);

/* Bytes of the workspace of qgemv_q8_0_grouped for x_rows activation rows of
 * length k and m assignments: the plan (assignments sorted by expert, work
 * items of at most 16 of one expert) and the q8 rows.  0 for an invalid
 * shape (m > QG_MAX_ASSIGN included). */
size_t qg_grouped_workspace_bytes(int x_rows, int64_t k, int m);

/* Static description of a status code. */
const char* qg_status_string(int status);

/* Copies this thread's detail of the last failed call into buf (host),
 * NUL-terminated; returns the status of that call (QG_OK if none failed). */
int qg_last_error_detail(char* buf, size_t len);

/* Capability probe: 1 when HIP device `device` is a gfx950 on which this
 * library's code object carries its marker, a device global that stands for
 * the image layouts and kernels declared here; 0 otherwise.  Any driver
 * failure, the marker's name missing included, answers 0, never an error
 * status (the drama page's series commits: a promise a code object carries
 * in a device global, checked by the host before it relies on it).  Host
 * only; launches nothing and leaves the calling thread's current device as
 * it found it. */
int qg_device_supported(int device);

/* ---------------------------------------------------------------- device --- */

/* Quantizes fp32 weights w [n][k] (device) into a device image of `fmt`
 * (Q8_0, Q4_0, Q4_K or FP8) by the block rules above (Q4_K, per 32-weight
 * sub-block j with lo = min(0, min w) and hi = max w: s_j = (hi - lo)/15,
 * mn_j = -lo; d = fp16(max s / 63), dmin = fp16(max mn / 63); sc = min(63,
 * round(s_j / d)), m = min(63, round(mn_j / dmin)); q = clamp(round((w +
 * dmin*m) / (d*sc)), 0, 15) -- the format does not fix a quantizer; this is
 * the plainest one).  Requires max|w|/qmax to fit fp16.
 * Offline preparation, not part of the per-token path. */
int qg_quantize_weights(int fmt, const float* w, int64_t n, int64_t k, void* image, qg_stream stream);

/* A1 of the q8 lane: quantizes rows x [rows][k] (1 <= rows <= QG_MAX_PREP_ROWS)
 * into the workspace `ws` (qg_workspace_bytes(rows, k) bytes) in the layout the
 * GEMV kernels read for that row count (so a workspace serves GEMV calls with
 * the same rows and k). */
int qg_prepare_rows(const float* x, int rows, int64_t k, void* ws, size_t ws_bytes, qg_stream stream);

/* The step before a projection group, in one launch: residual add, RMS norm
 * and A1.  The drama page (series commits) folds the activation quantization
 * of the next projection into its add + norm launch with results equal to a
 * separate quantization pass; the llama-leg page ("Not done") names a requant
 * arm of its add+rms family.  Per row r of x [rows][k] (fp32):
 *   h = x + residual                    (residual may be null: h = x)
 *   y = h * (1 / sqrt(mean(h^2) + eps)) * gamma   (gamma [k])
 * in fp32: the sum of squares in a fixed order (per thread, then a wave tree,
 * then the sixteen waves left to right), so y is reproducible bit for bit.
 * Writes h to h_out and y to y_out when they are not null (both [rows][k];
 * they may alias x or residual), and, when ws is not null, A1 of y into ws
 * (qg_workspace_bytes(rows, k) bytes) in the layout the GEMV reads for `rows`
 * rows -- the same bytes qg_prepare_rows writes for y.  1 <= rows <= 8192
 * (0 is a no-op), k a multiple of 32, eps >= 0; at least one of ws, h_out,
 * y_out must be given. */
int qg_add_rmsnorm_prepare(const float* x, const float* residual, const float* gamma, float eps, int rows, int64_t k,
                           float* h_out, float* y_out, void* ws, size_t ws_bytes, qg_stream stream);

/* q8 lane GEMV on rows already prepared in `ws` (by qg_prepare_rows with the
 * same rows and k): y [rows][n] fp32, row stride n.  fmt = Q8_0, Q4_0 or Q4_K.
 * ws_bytes is the workspace's size: smaller than qg_workspace_bytes(rows, k)
 * is refused (QG_EWORKSPACE) rather than read past (the audio-towers page,
 * router-GEMV commit: a launch never reads past what it was given). */
int qgemv_prepared(int fmt, const void* w_image, int64_t n, int64_t k, const void* ws, size_t ws_bytes, int rows,
                   float* y, qg_stream stream);

/* Q8_0 weights x q8 activations: y [rows][n] = W . x for 0 <= rows <= 16.
 * The q8 lane of the audio-towers page (feature commit: the default device
 * lane; block-quantized weights against q8 activations, integer block dots);
 * rows past eight tiled inside this one call and weight pass, each row equal
 * to the row computed alone (the same page's router-GEMV commit; the
 * llama-leg page, commit 16880fe: balanced groups past eight rows rather
 * than one more read of the weights for every extra row); k in whole
 * 32-blocks (llama-leg page, commit 8624bce).
 *   w_image  device image (qg_quantize_weights / qg_pack_image), 256-aligned
 *   x        [rows][k] fp32, device, 16-aligned, finite
 *   y        [rows][n] fp32, device, written whole, nothing else written
 *   ws       device scratch of ws_bytes >= qg_workspace_bytes(rows, k),
 *            256-aligned, owned by the caller (rows 1-2 are quantized inside
 *            the GEMV launch when they fit its staging area, as for
 *            qgemv_set_rows; the workspace is checked either way)
 * Errors (nothing launched): QG_EROWS for rows outside 0..16, QG_ESHAPE for
 * n < 1 or k not whole blocks, QG_EINVAL / QG_EALIGN for null or misaligned
 * pointers, QG_EWORKSPACE for a short workspace, QG_EDEVICE off gfx950. */
int qgemv_q8_0(const void* w_image, int64_t n, int64_t k, const float* x, int rows, float* y, void* ws,
               size_t ws_bytes, qg_stream stream);

/* Q4_K superblocks x q8 activations; arguments, rows, tiling and errors as
 * qgemv_q8_0, with k a multiple of 256 (QG_ESHAPE otherwise): the one-row and
 * N-row form of a K-quant superblock format whose K comes in whole
 * superblocks (the llama-leg page, commit 8624bce; its race bed's Q4_K_M
 * weights, body and Validation).  Per 32-weight sub-block the exact int32 dot
 * of the raw codes with the q8 codes, then d_x * (d*sc * isum - dmin*m * s_x)
 * in fp32, in a fixed order that does not depend on `rows`. */
int qgemv_q4_k(const void* w_image, int64_t n, int64_t k, const float* x, int rows, float* y, void* ws,
               size_t ws_bytes, qg_stream stream);

/* qgemv_q8_0 for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernels and the same bits, with the q8
 * activation rows (3..16 rows) in a static device array of
 * QG_NOALLOC_SCRATCH_BYTES per GPU, held from the first call on that GPU until
 * the process ends.  The call allocates and frees nothing.  A call whose
 * qg_workspace_bytes(rows, k) exceeds that size is refused with
 * QG_EWORKSPACE (every k <= 28672 fits at any row count); 1-2 rows use no
 * workspace.  All calls on one GPU share the array: two calls that may
 * overlap on one GPU (different streams, or different host threads without
 * an ordering) race on it and must not be issued; calls ordered on one
 * stream are safe.  Other arguments and errors as qgemv_q8_0. */
int qgemv_q8_0_noalloc(const void* w_image, int64_t n, int64_t k, const float* x, int rows, float* y,
                       qg_stream stream);

/* Q4_0 weights x q8 activations; arguments, rows, tiling and errors as
 * qgemv_q8_0 (the q8 lane of the audio-towers page's feature commit, with
 * 4-bit weight blocks).  The codes stand for c - 8; each block dot starts
 * from -8 * (sum of the activation codes). */
int qgemv_q4_0(const void* w_image, int64_t n, int64_t k, const float* x, int rows, float* y, void* ws,
               size_t ws_bytes, qg_stream stream);

/* Device -> device: the F16 image (qg_image_bytes(QG_FMT_F16, n, k) bytes,
 * 256-byte aligned) of the row-major [n][k] halfword matrix w (16-byte
 * aligned, k % 8 == 0). */
int qg_f16_image(const uint16_t* w, int64_t n, int64_t k, void* image, qg_stream stream);

/* f16 lane: y [rows][n] = W [n][k] (fp16, as the F16 image w_image) . x
 * [rows][k] (fp32), fp32 products and sums -- the reference lane of the
 * audio-towers page (feature commit: halfword weights, f32 accumulate).
 * x enters the halfword products as two halfword terms per value (about 22
 * significant bits, scaled by a power of two per row and k range), so the
 * result is fp32-accurate.  A row's bits do not depend on the other rows of
 * the call (router-GEMV commit).  The weights come as the F16 image
 * (qg_f16_image from row-major halfwords, once, offline) rather than as the
 * row-major matrix: a wave then reads 1 KB of consecutive bytes per load.
 * rows 0..16, k % 8 == 0; errors as qgemv_q8_0 (no workspace). */
int gemv_f16(const void* w_image, int64_t n, int64_t k, const float* x, int rows, float* y, qg_stream stream);

/* FP8 lane, activation groups: x [rows][k] fp32 (1 <= rows <= 8192) into the
 * FP8 workspace ws (qg_fp8_workspace_bytes(rows, k) bytes). */
int qg_prepare_fp8(const float* x, int rows, int64_t k, void* ws, size_t ws_bytes, qg_stream stream);

/* FP8 lane GEMV on rows prepared by qg_prepare_fp8 (same rows and k):
 * y [rows][n] fp32, 0 <= rows <= 16.  w_image: the FP8 image (qg_pack_image
 * or qg_quantize_weights with QG_FMT_FP8).  ws_bytes smaller than
 * qg_fp8_workspace_bytes(rows, k) is refused (QG_EWORKSPACE). */
int qgemv_fp8_prepared(const void* w_image, int64_t n, int64_t k, const void* ws, size_t ws_bytes, int rows,
                       float* y, qg_stream stream);

/* qg_prepare_fp8 then qgemv_fp8_prepared: x [rows][k] fp32, y [rows][n]. */
int qgemv_fp8(const void* w_image, int64_t n, int64_t k, const float* x, int rows, float* y, void* ws,
              size_t ws_bytes, qg_stream stream);

/* Several independent q8-lane projections with the same row count in one
 * launch (a decode layer's Q/K/V/O/gate/up/down).  Each entry's rows must
 * already be prepared in its `ws` (ws_bytes >= qg_workspace_bytes(rows, k),
 * else QG_EWORKSPACE).  1 <= count <= QG_MAX_SET. */
typedef struct {
  const void* w_image;
  int64_t n;
  int64_t k;
  const void* ws;  /* prepared rows for this projection's input */
  size_t ws_bytes; /* its size */
  float* y;        /* [rows][n] */
} qg_proj;
int qgemv_set(int fmt, const qg_proj* projs /*host*/, int count, int rows, qg_stream stream);

/* Several projections with the same row count straight from fp32 rows, the
 * whole decode-layer step in as few launches as the row count allows: for
 * rows <= QG_FUSED_ROWS whose q8 blocks fit the launch's 80 KiB staging area
 * (every projection's k up to 72704 at one row and 36352 at two in Q8_0,
 * 65536 and 32768 in Q4_0) the rows are quantized inside the GEMV launch (one
 * launch, ws unused and may be null); otherwise one launch quantizes every
 * distinct (x, ws) pair into its ws (qg_workspace_bytes(rows, k) bytes;
 * projections that share x may share ws) and a second runs all GEMVs.  Q4_0
 * and Q4_K at two rows take the two launches whenever every projection
 * brings a 256-aligned ws of at least qg_workspace_bytes(rows, k) (faster
 * there), and the one launch when any does not; the outputs are the same
 * bits either way.
 * 1 <= count <= QG_MAX_SET. */
typedef struct {
  const void* w_image;
  int64_t n;
  int64_t k;
  const float* x; /* [rows][k] fp32 */
  void* ws;
  size_t ws_bytes;
  float* y; /* [rows][n] */
} qg_proj_rows;
int qgemv_set_rows(int fmt, const qg_proj_rows* projs /*host*/, int count, int rows, qg_stream stream);

/* Prepares several activation sets in one launch (count <= QG_MAX_SET). */
typedef struct {
  const float* x; /* [rows][k] */
  int64_t k;
  void* ws;
  size_t ws_bytes;
} qg_act;
int qg_prepare_rows_set(const qg_act* acts /*host*/, int count, int rows, qg_stream stream);

/* Grouped routed-expert GEMV, Q8_0 (the llama-leg page, commit 2243ccc and
 * "Observable behavior": a routed model steps several rows' picks in one
 * N-row command; the drama page's backbone section: a 256-expert top-8 MoE
 * with a shared expert).  w_images holds n_experts device images
 * back to back, each qg_image_bytes(Q8_0, n, k) bytes.  For assignment j < m:
 * y[j] = W_{expert[j]} . q8(x[x_index[j]]).  Each touched expert's weights are
 * streamed once for up to 16 of its assignments.  expert and x_index are
 * device int32 arrays; an entry out of range is skipped (y[j] untouched) and
 * counted in the workspace, readable with qg_grouped_status.  x [x_rows][k],
 * 1 <= x_rows <= QG_MAX_PREP_ROWS, 0 <= m <= QG_MAX_ASSIGN; with m == 0, y, expert
 * and x_index may be null and only the workspace is written.  Two launches:
 * the plan (which also quantizes x into ws), then the GEMV. */
int qgemv_q8_0_grouped(const void* w_images, int64_t n_experts, int64_t n, int64_t k, const float* x, int x_rows,
                       const int32_t* expert, const int32_t* x_index, int m, float* y, void* ws, size_t ws_bytes,
                       qg_stream stream);

/* Grouped routed-expert GEMV, FP8 lane (the drama page's backbone runs its
 * routed experts in block-FP8 with 1 x 128 FP8 activation groups): as
 * qgemv_q8_0_grouped, with w_images n_experts FP8 images back to back, each
 * qg_image_bytes(QG_FMT_FP8, n, k) bytes (k a multiple of 128), and the rows
 * of x quantized into FP8 groups as qg_prepare_fp8 does.  Each assignment's
 * y[j] has the bits of qgemv_fp8 on its row alone.  ws:
 * qg_fp8_grouped_workspace_bytes(x_rows, k, m) bytes; qg_grouped_status reads
 * its skipped count. */
size_t qg_fp8_grouped_workspace_bytes(int x_rows, int64_t k, int m);
int qgemv_fp8_grouped(const void* w_images, int64_t n_experts, int64_t n, int64_t k, const float* x, int x_rows,
                      const int32_t* expert, const int32_t* x_index, int m, float* y, void* ws, size_t ws_bytes,
                      qg_stream stream);

/* Synchronizes `stream`, then reads the count of skipped assignments of the
 * last grouped call on `ws` into *bad (host). */
int qg_grouped_status(const void* ws, int32_t* bad, qg_stream stream);

/* MoE glue around the grouped GEMV (routed decode step with an ungated shared
 * expert).
 * qg_moe_route: per row, softmax over n_experts logits (max subtracted) and
 *   the topk experts by logit, ties to the lower index, in descending order;
 *   writes rows*slots assignments, slots = topk + (shared_expert >= 0): slot
 *   s < topk is (expert, x_index = r, weight = softmax probability), the last
 *   slot is (shared_expert, r, 1.0).  1 <= topk <= 32, n_experts <= 1024. */
int qg_moe_route(const float* logits, int rows, int n_experts, int topk, int shared_expert, int32_t* expert,
                 int32_t* x_index, float* weight, qg_stream stream);

/* h[j][i] = silu(gu[j][i]) * gu[j][ffn + i], silu(g) = g / (1 + exp(-g)),
 * for j < m, i < ffn (gate rows first, then up rows, in one output row). */
int qg_swiglu(const float* gu, int m, int64_t ffn, float* h, qg_stream stream);

/* y[r] = sum over s < slots, in slot order, of weight[r*slots+s] * o[r*slots+s]
 * (o rows of length hidden). */
int qg_moe_combine(const float* o, const float* weight, int rows, int slots, int64_t hidden, float* y,
                   qg_stream stream);

/* A routed-MoE decode step, the composition of the calls above: router
 * logits (f16 lane: router_image is the F16 image of the n_experts x hidden
 * router), routing as qg_moe_route, grouped gate/up GEMV, SwiGLU quantized
 * for the down projection, grouped down GEMV, weighted combine.  Six
 * launches at 9-16 rows; four at 3-8 rows, where the gate/up launch routes
 * the rows itself and the down launch quantizes the SwiGLU of the gate/up
 * rows in its staging (on the work items cut to two rows, so an expert that
 * c rows meet is read ceil(c/2) times); three at 1-2 rows, where the down
 * launch does the same and, when the assignments fit one workgroup, combines
 * them (four when they do not).  gu_images holds
 * n_experts + shared Q8_0 images of [2*ffn][hidden] (gate rows, then up rows)
 * back to back; down_images the same experts' [hidden][ffn]; with shared = 1
 * image n_experts is an ungated shared expert joining every row with weight
 * 1 (the last slot).  x [rows][hidden], y [rows][hidden] fp32, 1 <= rows <= 16
 * (0 is a no-op), 1 <= topk <= min(32, n_experts), n_experts <= 1024, hidden
 * and ffn multiples of 32.  logits [rows][n_experts], expert and weight
 * [rows][slots] (slots = topk + shared) receive the routing when not null.
 * ws: qg_moe_workspace_bytes bytes.  Rows of 9..16 run in the same launches.
 * The step follows the routed feed-forward of the llama-leg page's routed-slot
 * commit 2243ccc and the drama page's MoE series commits. */
size_t qg_moe_workspace_bytes(int rows, int n_experts, int64_t hidden, int64_t ffn, int topk, int shared);
int qg_moe_step(const void* router_image, int n_experts, int64_t hidden, int64_t ffn, int topk, int shared,
                const void* gu_images, const void* down_images, const float* x, int rows, float* y, float* logits,
                int32_t* expert, float* weight, void* ws, size_t ws_bytes, qg_stream stream);

/* The routed-MoE step in the FP8 lane (the drama page's backbone: a 256-expert
 * top-8 block-FP8 MoE with a shared expert, activations in dynamic 1 x 128
 * FP8 groups): as qg_moe_step, with gu_images and down_images FP8 images
 * (qg_image_bytes(QG_FMT_FP8, ...) each, back to back), the input rows and
 * the SwiGLU rows quantized into FP8 groups, and the expert GEMVs those of
 * qgemv_fp8_grouped.  hidden and ffn multiples of 128.  Six launches; five
 * when the rows fit the gate/up launch's waves (up to 8 rows on the usual
 * shapes), which then plans for itself beside the router launch's FP8 input
 * groups; four at one row, where the down launch also takes the SwiGLU of the
 * gate/up rows in its staging (ffn up to 2048).  The
 * bits are those of the composition: the f16 router GEMV, qg_moe_route,
 * qgemv_fp8_grouped on the gate/up images, qg_swiglu, qgemv_fp8_grouped on
 * the down images (assignment j reading SwiGLU row j), qg_moe_combine.
 * ws: qg_moe_fp8_workspace_bytes bytes. */
size_t qg_moe_fp8_workspace_bytes(int rows, int n_experts, int64_t hidden, int64_t ffn, int topk, int shared);
int qg_moe_step_fp8(const void* router_image, int n_experts, int64_t hidden, int64_t ffn, int topk, int shared,
                    const void* gu_images, const void* down_images, const float* x, int rows, float* y,
                    float* logits, int32_t* expert, float* weight, void* ws, size_t ws_bytes, qg_stream stream);

/* ------------------------------------------------------ test-only hooks --- */

/* A1 in the plain layout: qx [rows][k] int8, dx [rows][k/32] fp32, sx
 * [rows][k/32] int32 (sum of the block's codes). */
int qg_quantize_rows_q8(const float* x, int rows, int64_t k, int8_t* qx, float* dx, int32_t* sx, qg_stream stream);

/* A3 alone: isum [rows][n][k/32] int32 = exact block dots of the image's codes
 * with qx [rows][k] (plain layout), rows <= 16 (Q4_K: the raw 4-bit codes of
 * each 32-weight sub-block). */
int qgemv_blockdots(int fmt, const void* w_image, int64_t n, int64_t k, const int8_t* qx, int rows, int32_t* isum,
                    qg_stream stream);

/* A3 as the 3..16-row kernel forms it: isum [rows][n][k/32] int32, the exact
 * block dots of the image's codes with rows prepared in ws by
 * qg_prepare_rows(x, rows, k, ...) (pair order, ws_bytes >= its size), each
 * from the same block-pair matrix product that kernel scales and sums
 * (Q4_0: codes c - 8).  3 <= rows <= 16. */
int qgemv_blockdots_pairs(int fmt, const void* w_image, int64_t n, int64_t k, const void* ws, size_t ws_bytes,
                          int rows, int32_t* isum, qg_stream stream);

/* ------------------------------------------------------ measurement hook --- */

/* The achievable-read ceiling: reads `bytes` (a nonzero multiple of 16) at
 * src (16-byte aligned) once with 16-byte non-temporal loads, the GEMV
 * kernels' weight-load form, in `grid` workgroups of 512 threads (1..65536),
 * each reading one contiguous range with `inflight` (1, 2, 4 or 8) loads per
 * thread in flight, and stores an xor fold of what it read to sink
 * (grid * 8 uint32, device; its values mean nothing).  Timing it over the
 * same bytes as a GEMV's weight image gives the bare-read bandwidth that the
 * GEMV is compared with beside the HBM data-sheet peak (the pages' one-row
 * projections are weight-streaming passes: llama-leg page, commit 16880fe;
 * drama page, series commits). */
int qg_read_probe(const void* src, size_t bytes, int grid, int inflight, uint32_t* sink, qg_stream stream);

#ifdef __cplusplus
}
#endif
#endif /* QGEMV_H */
