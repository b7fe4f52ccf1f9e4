// qg_api.hip -- the C ABI's device entry points: argument validation on the
// host (a negative status means nothing was enqueued), then the launchers.
#include <hip/hip_runtime.h>
#include <string.h>

#include "qg_internal.h"
#include "qg_launch.h"
#include "qg_layout.h"

using namespace qg;

namespace {

int check_fmt(int fmt) {
  if (fmt != QG_FMT_Q8_0 && fmt != QG_FMT_Q4_0 && fmt != QG_FMT_Q4_K)
    return fail(QG_EINVAL, "fmt=%d is not Q8_0 (1), Q4_0 (2) or Q4_K (5)", fmt);
  return QG_OK;
}

int check_nk(int64_t n, int64_t k) {
  if (n < 1 || n > (1LL << 31) - 16) return fail(QG_ESHAPE, "n=%lld outside 1..2^31-16", (long long)n);
  if (k < QK || k % QK || k > (1LL << 24))
    return fail(QG_ESHAPE, "k=%lld is not a positive multiple of 32 up to 2^24", (long long)k);
  return QG_OK;
}

// k in whole blocks of the format: 32 weights, or a 256-weight superblock for
// Q4_K (the llama-leg page, commit 8624bce).
int check_nk_fmt(int fmt, int64_t n, int64_t k) {
  if (int st = check_nk(n, k)) return st;
  if (fmt == QG_FMT_Q4_K && k % QK_K)
    return fail(QG_ESHAPE, "k=%lld is not a multiple of 256 (Q4_K superblocks)", (long long)k);
  return QG_OK;
}

int check_fp8_nk(int64_t n, int64_t k) {
  if (n < 1 || n > (1LL << 31) - 16) return fail(QG_ESHAPE, "n=%lld outside 1..2^31-16", (long long)n);
  if (k < 128 || k % 128 || k > (1LL << 24))
    return fail(QG_ESHAPE, "k=%lld is not a positive multiple of 128 up to 2^24", (long long)k);
  return QG_OK;
}

int check_rows(int rows) {
  if (rows < 0 || rows > QG_MAX_ROWS) return fail(QG_EROWS, "rows=%d outside 0..%d", rows, QG_MAX_ROWS);
  return QG_OK;
}

int check_image(const void* image, const char* name) {
  if (!image) return fail(QG_EINVAL, "%s is null", name);
  if (!aligned(image, 256)) return fail(QG_EALIGN, "%s %p is not 256-byte aligned", name, image);
  return QG_OK;
}

int check_y(const float* y) {
  if (!y) return fail(QG_EINVAL, "y is null");
  if (!aligned(y, 4)) return fail(QG_EALIGN, "y %p is not 4-byte aligned", (const void*)y);
  return QG_OK;
}

int check_x(const float* x, int rows, int64_t k, int max_rows) {
  if (!x) return fail(QG_EINVAL, "x is null");
  if (!aligned(x, 16)) return fail(QG_EALIGN, "x %p is not 16-byte aligned", (const void*)x);
  if (rows < 1 || rows > max_rows) return fail(QG_EROWS, "rows=%d outside 1..%d", rows, max_rows);
  if (k < QK || k % QK || k > (1LL << 24))
    return fail(QG_ESHAPE, "k=%lld is not a positive multiple of 32 up to 2^24", (long long)k);
  return QG_OK;
}

int check_ws(const void* ws, size_t have, size_t need, const char* what) {
  if (!ws) return fail(QG_EINVAL, "%s workspace is null", what);
  if (!aligned(ws, 256)) return fail(QG_EALIGN, "%s workspace %p is not 256-byte aligned", what, ws);
  if (have < need) return fail(QG_EWORKSPACE, "ws_bytes=%zu < %zu needed for %s", have, need, what);
  return QG_OK;
}

// Q8_0 / Q4_0 GEMV from fp32 rows: rows small enough are quantized inside the
// GEMV launch, otherwise a quantize launch fills the workspace first.
int qgemv_fmt(int fmt, const void* w_image, int64_t n, int64_t k, const float* x, int rows, float* y, void* ws,
              size_t ws_bytes, qg_stream stream) {
  if (int st = check_rows(rows)) return st;
  if (int st = check_nk_fmt(fmt, n, k)) return st;
  if (int st = check_image(w_image, "w_image")) return st;
  if (int st = check_y(y)) return st;
  if (rows == 0) return ok();
  if (int st = check_x(x, rows, k, QG_MAX_ROWS)) return st;
  if (int st = check_ws(ws, ws_bytes, prep_layout(rows, k).total, "the activation rows")) return st;
  if (int st = check_device()) return st;
  hipStream_t s = (hipStream_t)stream;
  ProjArg pa{w_image, n, k, ws, nullptr, y};
  if (fuses_quantization(fmt, rows, k)) {
    pa.x = x;
  } else if (int st = launch_prepare(x, rows, k, ws, prep_layout(rows, k), s)) {
    return st;
  }
  if (int st = launch_qgemv_set(fmt, &pa, 1, rows, s)) return st;
  return ok();
}

}  // namespace

extern "C" {

int qg_quantize_weights(int fmt, const float* w, int64_t n, int64_t k, void* image, qg_stream stream) {
  if (fmt != QG_FMT_FP8)
    if (int st = check_fmt(fmt)) return st;
  if (int st = fmt == QG_FMT_FP8 ? check_fp8_nk(n, k) : check_nk_fmt(fmt, n, k)) return st;
  if (!w) return fail(QG_EINVAL, "w is null");
  if (!aligned(w, 16)) return fail(QG_EALIGN, "w %p is not 16-byte aligned", (const void*)w);
  if (int st = check_image(image, "image")) return st;
  if (int st = check_device()) return st;
  if (fmt == QG_FMT_FP8) {
    if (int st = launch_fp8_quantize_weights(w, n, k, image, (hipStream_t)stream)) return st;
    return ok();
  }
  if (int st = launch_quantize_weights(fmt, w, n, k, image, (hipStream_t)stream)) return st;
  return ok();
}

int qg_prepare_fp8(const float* x, int rows, int64_t k, void* ws, size_t ws_bytes, qg_stream stream) {
  if (int st = check_x(x, rows, k, QG_MAX_PREP_ROWS)) return st;
  if (k % 128) return fail(QG_ESHAPE, "k=%lld is not a multiple of 128", (long long)k);
  if (int st = check_ws(ws, ws_bytes, fp8_ws_bytes(rows, k), "the FP8 activation rows")) return st;
  if (int st = check_device()) return st;
  if (int st = launch_fp8_prepare(x, rows, k, ws, (hipStream_t)stream)) return st;
  return ok();
}

int qgemv_fp8_prepared(const void* w_image, int64_t n, int64_t k, const void* ws, size_t ws_bytes, int rows, float* y,
                       qg_stream stream) {
  if (int st = check_rows(rows)) return st;
  if (int st = check_fp8_nk(n, k)) return st;
  if (int st = check_image(w_image, "w_image")) return st;
  if (int st = check_y(y)) return st;
  if (rows == 0) return ok();
  if (int st = check_ws(ws, ws_bytes, fp8_ws_bytes(rows, k), "the FP8 activation rows")) return st;
  if (int st = check_device()) return st;
  if (int st = launch_gemv_fp8(w_image, n, k, ws, rows, y, (hipStream_t)stream)) return st;
  return ok();
}

int qgemv_fp8(const void* w_image, int64_t n, int64_t k, const float* x, int rows, float* y, void* ws,
              size_t ws_bytes, qg_stream stream) {
  if (int st = check_rows(rows)) return st;
  if (int st = check_fp8_nk(n, k)) return st;
  if (int st = check_image(w_image, "w_image")) return st;
  if (int st = check_y(y)) return st;
  if (rows == 0) return ok();
  if (int st = check_x(x, rows, k, QG_MAX_ROWS)) return st;
  if (int st = check_ws(ws, ws_bytes, fp8_ws_bytes(rows, k), "the FP8 activation rows")) return st;
  if (int st = check_device()) return st;
  hipStream_t s = (hipStream_t)stream;
  if (int st = launch_fp8_prepare(x, rows, k, ws, s)) return st;
  if (int st = launch_gemv_fp8(w_image, n, k, ws, rows, y, s)) return st;
  return ok();
}

int qg_prepare_rows(const float* x, int rows, int64_t k, void* ws, size_t ws_bytes, qg_stream stream) {
  if (int st = check_x(x, rows, k, QG_MAX_PREP_ROWS)) return st;
  if (int st = check_ws(ws, ws_bytes, prep_layout(rows, k).total, "the activation rows")) return st;
  if (int st = check_device()) return st;
  if (int st = launch_prepare(x, rows, k, ws, prep_layout(rows, k), (hipStream_t)stream)) return st;
  return ok();
}

int qg_add_rmsnorm_prepare(const float* x, const float* residual, const float* gamma, float eps, int rows, int64_t k,
                           float* h_out, float* y_out, void* ws, size_t ws_bytes, qg_stream stream) {
  if (rows == 0) return ok();
  if (int st = check_x(x, rows, k, QG_MAX_PREP_ROWS)) return st;
  if (!gamma) return fail(QG_EINVAL, "gamma is null");
  if (!aligned(gamma, 16)) return fail(QG_EALIGN, "gamma %p is not 16-byte aligned", (const void*)gamma);
  if (residual && !aligned(residual, 16))
    return fail(QG_EALIGN, "residual %p is not 16-byte aligned", (const void*)residual);
  if (h_out && !aligned(h_out, 16)) return fail(QG_EALIGN, "h_out %p is not 16-byte aligned", (const void*)h_out);
  if (y_out && !aligned(y_out, 16)) return fail(QG_EALIGN, "y_out %p is not 16-byte aligned", (const void*)y_out);
  if (!(eps >= 0.0f) || eps > 1e30f) return fail(QG_EINVAL, "eps=%g is not a finite value >= 0", (double)eps);
  if (ws) {
    if (int st = check_ws(ws, ws_bytes, prep_layout(rows, k).total, "the normed rows")) return st;
  } else if (!h_out && !y_out) {
    return fail(QG_EINVAL, "no output: ws, h_out and y_out are all null");
  }
  if (int st = check_device()) return st;
  if (int st = launch_add_rmsnorm_prepare(x, residual, gamma, eps, rows, k, h_out, y_out, ws, (hipStream_t)stream))
    return st;
  return ok();
}

int qg_prepare_rows_set(const qg_act* acts, int count, int rows, qg_stream stream) {
  if (!acts || count < 1 || count > QG_MAX_SET) return fail(QG_EINVAL, "count=%d outside 1..%d", count, QG_MAX_SET);
  for (int i = 0; i < count; i++) {
    if (int st = check_x(acts[i].x, rows, acts[i].k, QG_MAX_PREP_ROWS)) return fail(st, "acts[%d]: x/rows/k", i);
    if (int st = check_ws(acts[i].ws, acts[i].ws_bytes, prep_layout(rows, acts[i].k).total, "acts[i]"))
      return fail(st, "acts[%d]: workspace", i);
  }
  if (int st = check_device()) return st;
  if (int st = launch_prepare_set(acts, count, rows, (hipStream_t)stream)) return st;
  return ok();
}

int qgemv_prepared(int fmt, const void* w_image, int64_t n, int64_t k, const void* ws, size_t ws_bytes, int rows,
                   float* y, qg_stream stream) {
  if (int st = check_fmt(fmt)) return st;
  if (int st = check_rows(rows)) return st;
  if (int st = check_nk_fmt(fmt, n, k)) return st;
  if (int st = check_image(w_image, "w_image")) return st;
  if (int st = check_y(y)) return st;
  if (rows == 0) return ok();
  // the layout read depends on rows (row order at 1-2, pair order at 3-16): the
  // workspace must hold that layout whole, or the kernel would read past it
  if (int st = check_ws(ws, ws_bytes, prep_layout(rows, k).total, "the prepared rows")) return st;
  if (int st = check_device()) return st;
  ProjArg pa{w_image, n, k, ws, nullptr, y};
  if (int st = launch_qgemv_set(fmt, &pa, 1, rows, (hipStream_t)stream)) return st;
  return ok();
}

int qgemv_q8_0(const void* w_image, int64_t n, int64_t k, const float* x, int rows, float* y, void* ws,
               size_t ws_bytes, qg_stream stream) {
  return qgemv_fmt(QG_FMT_Q8_0, w_image, n, k, x, rows, y, ws, ws_bytes, stream);
}

int qgemv_q4_0(const void* w_image, int64_t n, int64_t k, const float* x, int rows, float* y, void* ws,
               size_t ws_bytes, qg_stream stream) {
  return qgemv_fmt(QG_FMT_Q4_0, w_image, n, k, x, rows, y, ws, ws_bytes, stream);
}

int qgemv_q4_k(const void* w_image, int64_t n, int64_t k, const float* x, int rows, float* y, void* ws,
               size_t ws_bytes, qg_stream stream) {
  return qgemv_fmt(QG_FMT_Q4_K, w_image, n, k, x, rows, y, ws, ws_bytes, stream);
}

int qgemv_set(int fmt, const qg_proj* projs, int count, int rows, qg_stream stream) {
  if (int st = check_fmt(fmt)) return st;
  if (!projs || count < 1 || count > QG_MAX_SET) return fail(QG_EINVAL, "count=%d outside 1..%d", count, QG_MAX_SET);
  if (int st = check_rows(rows)) return st;
  ProjArg pa[QG_MAX_SET];
  for (int i = 0; i < count; i++) {
    const qg_proj& p = projs[i];
    if (int st = check_nk_fmt(fmt, p.n, p.k)) return fail(st, "projs[%d]: n=%lld k=%lld", i, (long long)p.n, (long long)p.k);
    if (int st = check_image(p.w_image, "w_image")) return fail(st, "projs[%d].w_image null or misaligned", i);
    if (int st = check_y(p.y)) return fail(st, "projs[%d].y null or misaligned", i);
    if (rows) {
      if (int st = check_ws(p.ws, p.ws_bytes, prep_layout(rows, p.k).total, "the prepared rows"))
        return fail(st, "projs[%d].ws null, misaligned or small (%zu bytes)", i, p.ws_bytes);
    }
    pa[i] = ProjArg{p.w_image, p.n, p.k, p.ws, nullptr, p.y};
  }
  if (rows == 0) return ok();
  if (int st = check_device()) return st;
  if (int st = launch_qgemv_set(fmt, pa, count, rows, (hipStream_t)stream)) return st;
  return ok();
}

int qgemv_set_rows(int fmt, const qg_proj_rows* projs, int count, int rows, qg_stream stream) {
  if (int st = check_fmt(fmt)) return st;
  if (!projs || count < 1 || count > QG_MAX_SET) return fail(QG_EINVAL, "count=%d outside 1..%d", count, QG_MAX_SET);
  if (int st = check_rows(rows)) return st;
  // quantized inside the GEMV launch only when every projection's rows fit its staging area
  bool fuse = true;
  for (int i = 0; i < count; i++) fuse = fuse && fuses_quantization(fmt, rows, projs[i].k);
  // Q4_0 and Q4_K at two rows: when every projection brings a workspace large
  // enough and aligned (else, as at one row, ws is not used), one quantize
  // launch and the GEMV on prepared rows beat quantizing inside the set
  // launch, whose workgroups (about one tile each) each stage their
  // projection's two rows against few weight bytes (3B-shaped set: Q4_0
  // 18.2 -> 17.2 us, Q4_K 23.1 -> 20.4); the results are the same bits
  if (fuse && rows == 2 && fmt != QG_FMT_Q8_0) {
    bool all_ws = true;
    for (int i = 0; i < count; i++)
      all_ws = all_ws && projs[i].ws && aligned(projs[i].ws, 256) &&
               projs[i].ws_bytes >= prep_layout(rows, projs[i].k).total;
    fuse = !all_ws;
  }
  ProjArg pa[QG_MAX_SET];
  for (int i = 0; i < count; i++) {
    const qg_proj_rows& p = projs[i];
    if (int st = check_nk_fmt(fmt, p.n, p.k)) return fail(st, "projs[%d]: n=%lld k=%lld", i, (long long)p.n, (long long)p.k);
    if (int st = check_image(p.w_image, "w_image")) return fail(st, "projs[%d].w_image null or misaligned", i);
    if (int st = check_y(p.y)) return fail(st, "projs[%d].y null or misaligned", i);
    if (rows) {
      if (int st = check_x(p.x, rows, p.k, QG_MAX_ROWS)) return fail(st, "projs[%d].x null, misaligned or bad", i);
    }
    if (!fuse && rows) {
      if (int st = check_ws(p.ws, p.ws_bytes, prep_layout(rows, p.k).total, "projs[i]"))
        return fail(st, "projs[%d].ws missing or small (%zu bytes)", i, p.ws_bytes);
    }
    pa[i] = ProjArg{p.w_image, p.n, p.k, p.ws, nullptr, p.y};
  }
  if (rows == 0) return ok();
  if (int st = check_device()) return st;
  hipStream_t s = (hipStream_t)stream;
  if (fuse) {
    for (int i = 0; i < count; i++) pa[i].x = projs[i].x;
  } else {
    // one quantize launch for all distinct inputs
    qg_act acts[QG_MAX_SET];
    int na = 0;
    for (int i = 0; i < count; i++) {
      bool seen = false;
      for (int j = 0; j < i; j++) seen = seen || (projs[j].x == projs[i].x && projs[j].ws == projs[i].ws);
      if (!seen) acts[na++] = qg_act{projs[i].x, projs[i].k, projs[i].ws, projs[i].ws_bytes};
    }
    if (int st = launch_prepare_set(acts, na, rows, s)) return st;
  }
  if (int st = launch_qgemv_set(fmt, pa, count, rows, s)) return st;
  return ok();
}

static int check_f16_nk(int64_t n, int64_t k) {
  if (n < 1 || n > (1LL << 31) - 1) return fail(QG_ESHAPE, "n=%lld outside 1..2^31-1", (long long)n);
  if (k < 8 || k % 8 || k > (1LL << 24))
    return fail(QG_ESHAPE, "k=%lld is not a positive multiple of 8 up to 2^24", (long long)k);
  return QG_OK;
}

int qg_f16_image(const uint16_t* w, int64_t n, int64_t k, void* image, qg_stream stream) {
  if (int st = check_f16_nk(n, k)) return st;
  if (!w) return fail(QG_EINVAL, "w is null");
  if (!aligned(w, 16)) return fail(QG_EALIGN, "w %p is not 16-byte aligned", (const void*)w);
  if (int st = check_image(image, "image")) return st;
  if (int st = check_device()) return st;
  if (int st = launch_f16_pack(w, n, k, image, (hipStream_t)stream)) return st;
  return ok();
}

int gemv_f16(const void* w_image, int64_t n, int64_t k, const float* x, int rows, float* y, qg_stream stream) {
  if (int st = check_rows(rows)) return st;
  if (int st = check_f16_nk(n, k)) return st;
  if (int st = check_image(w_image, "w_image")) return st;
  if (int st = check_y(y)) return st;
  if (rows == 0) return ok();
  if (!x) return fail(QG_EINVAL, "x is null");
  if (!aligned(x, 16)) return fail(QG_EALIGN, "x %p is not 16-byte aligned", (const void*)x);
  if (int st = check_device()) return st;
  if (int st = launch_gemv_f16(w_image, n, k, x, rows, y, (hipStream_t)stream)) return st;
  return ok();
}

int qgemv_q8_0_grouped(const void* w_images, int64_t n_experts, int64_t n, int64_t k, const float* x, int x_rows,
                       const int32_t* expert, const int32_t* x_index, int m, float* y, void* ws, size_t ws_bytes,
                       qg_stream stream) {
  if (n_experts < 1 || n_experts > (1 << 30)) return fail(QG_ESHAPE, "n_experts=%lld", (long long)n_experts);
  if (m < 0 || m > QG_MAX_ASSIGN) return fail(QG_ESHAPE, "m=%d outside 0..%d", m, QG_MAX_ASSIGN);
  if (int st = check_nk(n, k)) return st;
  if (int st = check_image(w_images, "w_images")) return st;
  if (m && check_y(y)) return check_y(y);
  if (int st = check_x(x, x_rows, k, QG_MAX_PREP_ROWS)) return st;
  if (m && (!expert || !x_index)) return fail(QG_EINVAL, "expert or x_index is null");
  if (int st = check_ws(ws, ws_bytes, grouped_layout(x_rows, k, m).total, "the grouped call")) return st;
  if (int st = check_device()) return st;
  hipStream_t s = (hipStream_t)stream;
  const GroupedLayout G = grouped_layout(x_rows, k, m);
  if (int st = launch_grouped(w_images, n_experts, n, k, x, x_rows, expert, x_index, m, y, ws, s)) return st;
  return ok();
}

int qgemv_fp8_grouped(const void* w_images, int64_t n_experts, int64_t n, int64_t k, const float* x, int x_rows,
                      const int32_t* expert, const int32_t* x_index, int m, float* y, void* ws, size_t ws_bytes,
                      qg_stream stream) {
  if (n_experts < 1 || n_experts > (1 << 30)) return fail(QG_ESHAPE, "n_experts=%lld", (long long)n_experts);
  if (m < 0 || m > QG_MAX_ASSIGN) return fail(QG_ESHAPE, "m=%d outside 0..%d", m, QG_MAX_ASSIGN);
  if (int st = check_fp8_nk(n, k)) return st;
  if (int st = check_image(w_images, "w_images")) return st;
  if (m && check_y(y)) return check_y(y);
  if (int st = check_x(x, x_rows, k, QG_MAX_PREP_ROWS)) return st;
  if (m && (!expert || !x_index)) return fail(QG_EINVAL, "expert or x_index is null");
  const GroupedLayout G = grouped_fp8_layout(x_rows, k, m);
  if (int st = check_ws(ws, ws_bytes, G.total, "the FP8 grouped call")) return st;
  if (int st = check_device()) return st;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* w = (uint8_t*)ws;
  int* header = (int*)(w + G.header);
  int* sorted = (int*)(w + G.sorted);
  int* items = (int*)(w + G.items);
  if (int st = launch_grouped_plan(expert, x_index, m, n_experts, x_rows, header, sorted, items, s, x, k, w + G.prep,
                                   true))
    return st;
  if (int st = launch_grouped_fp8(w_images, n, k, w + G.prep, x_rows, header, sorted, items, x_index, m, y, s))
    return st;
  return ok();
}

int qg_grouped_status(const void* ws, int32_t* bad, qg_stream stream) {
  if (!ws || !bad) return fail(QG_EINVAL, "null argument");
  if (int st = check_device()) return st;
  if (int st = hip_status(hipStreamSynchronize((hipStream_t)stream), "hipStreamSynchronize")) return st;
  int32_t h[2];
  if (int st = hip_status(hipMemcpy(h, ws, sizeof h, hipMemcpyDeviceToHost), "hipMemcpy")) return st;
  *bad = h[1];
  return ok();
}

int qg_moe_route(const float* logits, int rows, int n_experts, int topk, int shared_expert, int32_t* expert,
                 int32_t* x_index, float* weight, qg_stream stream) {
  if (!logits || !expert || !x_index || !weight) return fail(QG_EINVAL, "null buffer");
  if (rows < 0 || rows > 65535) return fail(QG_EROWS, "rows=%d outside 0..65535", rows);
  if (n_experts < 1 || n_experts > 1024) return fail(QG_ESHAPE, "n_experts=%d outside 1..1024", n_experts);
  if (topk < 1 || topk > 32 || topk > n_experts) return fail(QG_ESHAPE, "topk=%d outside 1..min(32, n_experts)", topk);
  if (rows == 0) return ok();
  if (int st = check_device()) return st;
  if (int st = launch_moe_route(logits, rows, n_experts, topk, shared_expert, expert, x_index, weight,
                                (hipStream_t)stream))
    return st;
  return ok();
}

int qg_swiglu(const float* gu, int m, int64_t ffn, float* h, qg_stream stream) {
  if (!gu || !h) return fail(QG_EINVAL, "null buffer");
  if (m < 0 || ffn < 1) return fail(QG_ESHAPE, "m=%d ffn=%lld", m, (long long)ffn);
  if (m == 0) return ok();
  if (int st = check_device()) return st;
  if (int st = launch_swiglu(gu, m, ffn, h, (hipStream_t)stream)) return st;
  return ok();
}

int qg_moe_combine(const float* o, const float* weight, int rows, int slots, int64_t hidden, float* y,
                   qg_stream stream) {
  if (!o || !weight || !y) return fail(QG_EINVAL, "null buffer");
  if (rows < 0 || rows > 65535 || slots < 1 || hidden < 4 || hidden % 4)
    return fail(QG_ESHAPE, "rows=%d slots=%d hidden=%lld (hidden must be a multiple of 4)", rows, slots,
                (long long)hidden);
  if (!aligned(o, 16) || !aligned(y, 16)) return fail(QG_EALIGN, "o and y must be 16-byte aligned");
  if (rows == 0) return ok();
  if (int st = check_device()) return st;
  if (int st = launch_moe_combine(o, weight, rows, slots, hidden, y, (hipStream_t)stream)) return st;
  return ok();
}

static int check_moe(int rows, int n_experts, int64_t hidden, int64_t ffn, int topk, int shared) {
  if (rows < 0 || rows > QG_MAX_ROWS) return fail(QG_EROWS, "rows=%d outside 0..%d", rows, QG_MAX_ROWS);
  if (n_experts < 1 || n_experts > 1024) return fail(QG_ESHAPE, "n_experts=%d outside 1..1024", n_experts);
  if (topk < 1 || topk > 32 || topk > n_experts) return fail(QG_ESHAPE, "topk=%d outside 1..min(32, n_experts)", topk);
  if (shared != 0 && shared != 1) return fail(QG_EINVAL, "shared=%d is not 0 or 1", shared);
  if (hidden < QK || hidden % QK) return fail(QG_ESHAPE, "hidden=%lld is not a positive multiple of 32", (long long)hidden);
  if (ffn < QK || ffn % QK) return fail(QG_ESHAPE, "ffn=%lld is not a positive multiple of 32", (long long)ffn);
  return QG_OK;
}

size_t qg_moe_workspace_bytes(int rows, int n_experts, int64_t hidden, int64_t ffn, int topk, int shared) {
  if (rows < 1 || check_moe(rows, n_experts, hidden, ffn, topk, shared)) return 0;
  return moe_layout(rows, n_experts, hidden, ffn, topk + shared).total;
}

int qg_moe_step(const void* router_image, int n_experts, int64_t hidden, int64_t ffn, int topk, int shared,
                const void* gu_images, const void* down_images, const float* x, int rows, float* y, float* logits,
                int32_t* expert, float* weight, void* ws, size_t ws_bytes, qg_stream stream) {
  if (int st = check_moe(rows, n_experts, hidden, ffn, topk, shared)) return st;
  if (!router_image || !gu_images || !down_images || !x || !y) return fail(QG_EINVAL, "null buffer");
  if (int st = check_image(router_image, "router_image")) return st;
  if (int st = check_image(gu_images, "gu_images")) return st;
  if (int st = check_image(down_images, "down_images")) return st;
  if (int st = check_y(y)) return st;
  if (!aligned(x, 16)) return fail(QG_EALIGN, "x %p is not 16-byte aligned", (const void*)x);
  if (rows == 0) return ok();
  const int slots = topk + shared, m = rows * slots;
  const MoeLayout M = moe_layout(rows, n_experts, hidden, ffn, slots);
  if (int st = check_ws(ws, ws_bytes, M.total, "the MoE step")) return st;
  if (int st = check_device()) return st;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* w = (uint8_t*)ws;
  float* lg = logits ? logits : (float*)(w + M.logits);
  int32_t* ex = expert ? expert : (int32_t*)(w + M.expert);
  float* wt = weight ? weight : (float*)(w + M.weight);
  int32_t* xi = (int32_t*)(w + M.x_index);
  int* header = (int*)(w + M.header);
  int* sorted = (int*)(w + M.sorted);
  int* items = (int*)(w + M.items);
  // 3-8 rows: the items cut to at most two rows as well (the gate/up launch's
  // plan stores them), for a down launch that takes the SwiGLU in its staging;
  // their header beside the plan's.  (With more rows the experts that many
  // rows meet would be read too many times over.)
  const bool split = rows > 2 && rows <= MOE_UP_PLAN_ROWS && grouped_glu_fits(ffn);
  int* dheader = split ? header + 16 : nullptr;
  int* ditems = split ? (int*)(w + M.ditems) : nullptr;
  float* gu = (float*)(w + M.gu);
  float* o = (float*)(w + M.o);
  const int n_images = n_experts + shared;
  // the router logits, and beside them the input rows' A1
  if (int st = launch_moe_router(router_image, n_experts, hidden, x, rows, lg, w + M.xprep, s)) return st;
  // the plan and the gate/up GEMV (an expert meets a row at most once:
  // distinct top-k picks, a separate shared image).  Up to 8 rows (a row a
  // wave) every workgroup of the gate/up launch routes the rows itself,
  // which costs less than a launch of its own; with more rows a plan launch
  // does it once.
  if (rows <= MOE_UP_PLAN_ROWS) {
    MoeUp up;
    up.logits = lg;
    up.rows = rows;
    up.E = n_experts;
    up.topk = topk;
    up.shared = shared;
    up.expert = ex;
    up.weight = wt;
    up.x_index = xi;
    up.header = header;
    up.sorted = sorted;
    up.items = items;
    up.dheader = dheader;
    up.ditems = ditems;
    up.plan_off = 0;
    if (int st = launch_moe_up(gu_images, 2 * ffn, hidden, w + M.xprep, up, gu, s)) return st;
  } else {
    if (int st = launch_moe_plan(lg, rows, n_experts, topk, shared ? n_experts : -1, ex, wt, xi, header, sorted,
                                 items, nullptr, 0, nullptr, false, s))
      return st;
    if (int st = launch_grouped_planned(gu_images, n_images, 2 * ffn, hidden, w + M.xprep, rows, header, sorted, items,
                                        xi, m, rows, gu, s))
      return st;
  }
  // the down launch takes the SwiGLU of the gate/up rows in its staging (one
  // launch fewer): at most two rows on the plan's items, and where the shape
  // allows it the combine too; 3-8 rows on the items cut to two rows (an
  // expert of c rows read ceil(c / 2) times); otherwise a launch quantizes
  // the SwiGLU first
  const bool glu = rows <= 2 && grouped_glu_fits(ffn);
  if (glu && moe_down_combine_fits(rows, slots, hidden, ffn)) {
    if (int st = launch_moe_down_combine(down_images, n_images, hidden, ffn, gu, ex, wt, rows, slots, y, s)) return st;
    return ok();
  }
  if (split) {
    if (int st = launch_grouped_planned(down_images, n_images, hidden, ffn, w + M.hprep, m, dheader, sorted, ditems,
                                        nullptr, m, 2, o, s, gu))
      return st;
  } else {
    if (!glu)
      if (int st = launch_swiglu_q8(gu, m, ffn, w + M.hprep, s)) return st;
    if (int st = launch_grouped_planned(down_images, n_images, hidden, ffn, w + M.hprep, m, header, sorted, items,
                                        nullptr, m, rows, o, s, glu ? gu : nullptr))
      return st;
  }
  if (int st = launch_moe_combine(o, wt, rows, slots, hidden, y, s)) return st;
  return ok();
}

size_t qg_moe_fp8_workspace_bytes(int rows, int n_experts, int64_t hidden, int64_t ffn, int topk, int shared) {
  if (rows < 1 || check_moe(rows, n_experts, hidden, ffn, topk, shared) || hidden % 128 || ffn % 128) return 0;
  return moe_layout(rows, n_experts, hidden, ffn, topk + shared, true).total;
}

int qg_moe_step_fp8(const void* router_image, int n_experts, int64_t hidden, int64_t ffn, int topk, int shared,
                    const void* gu_images, const void* down_images, const float* x, int rows, float* y, float* logits,
                    int32_t* expert, float* weight, void* ws, size_t ws_bytes, qg_stream stream) {
  if (int st = check_moe(rows, n_experts, hidden, ffn, topk, shared)) return st;
  if (hidden % 128 || ffn % 128)
    return fail(QG_ESHAPE, "hidden=%lld and ffn=%lld must be multiples of 128 (FP8 groups)", (long long)hidden,
                (long long)ffn);
  if (!router_image || !gu_images || !down_images || !x || !y) return fail(QG_EINVAL, "null buffer");
  if (int st = check_image(router_image, "router_image")) return st;
  if (int st = check_image(gu_images, "gu_images")) return st;
  if (int st = check_image(down_images, "down_images")) return st;
  if (int st = check_y(y)) return st;
  if (!aligned(x, 16)) return fail(QG_EALIGN, "x %p is not 16-byte aligned", (const void*)x);
  if (rows == 0) return ok();
  const int slots = topk + shared, m = rows * slots;
  const MoeLayout M = moe_layout(rows, n_experts, hidden, ffn, slots, true);
  if (int st = check_ws(ws, ws_bytes, M.total, "the FP8 MoE step")) return st;
  if (int st = check_device()) return st;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* w = (uint8_t*)ws;
  float* lg = logits ? logits : (float*)(w + M.logits);
  int32_t* ex = expert ? expert : (int32_t*)(w + M.expert);
  float* wt = weight ? weight : (float*)(w + M.weight);
  int32_t* xi = (int32_t*)(w + M.x_index);
  int* header = (int*)(w + M.header);
  int* sorted = (int*)(w + M.sorted);
  int* items = (int*)(w + M.items);
  float* gu = (float*)(w + M.gu);
  float* o = (float*)(w + M.o);
  if (rows <= MOE_UP_PLAN_ROWS && moe_up_fp8_fits(2 * ffn, hidden, rows)) {
    // the router launch with the input rows' FP8 groups beside it, then the
    // gate/up launch planning for itself (a row a wave): no plan launch
    if (int st = launch_moe_router(router_image, n_experts, hidden, x, rows, lg, w + M.xprep, s, true)) return st;
    MoeUp up;
    up.logits = lg;
    up.rows = rows;
    up.E = n_experts;
    up.topk = topk;
    up.shared = shared;
    up.expert = ex;
    up.weight = wt;
    up.x_index = xi;
    up.header = header;
    up.sorted = sorted;
    up.items = items;
    up.dheader = nullptr;
    up.ditems = nullptr;
    up.plan_off = 0;
    if (int st = launch_moe_up_fp8(gu_images, 2 * ffn, hidden, w + M.xprep, up, gu, s)) return st;
  } else {
    if (int st = launch_gemv_f16(router_image, n_experts, hidden, x, rows, lg, s)) return st;
    if (int st = launch_moe_plan(lg, rows, n_experts, topk, shared ? n_experts : -1, ex, wt, xi, header, sorted,
                                 items, x, hidden, w + M.xprep, true, s))
      return st;
    if (int st = launch_grouped_fp8(gu_images, 2 * ffn, hidden, w + M.xprep, rows, header, sorted, items, xi, m,
                                    gu, s))
      return st;
  }
  // one row: the down launch takes the SwiGLU of the gate/up rows in its
  // staging (the rows' FP8 groups in LDS; each unit makes its item's, so with
  // more rows that costs more than the launch it saves); else a launch
  // makes them
  const bool glu = rows == 1 && fp8_glu_fits(ffn);
  if (!glu)
    if (int st = launch_swiglu_fp8(gu, m, ffn, w + M.hprep, s)) return st;
  if (int st = launch_grouped_fp8(down_images, hidden, ffn, w + M.hprep, m, header, sorted, items, nullptr, m, o, s,
                                  glu ? gu : nullptr))
    return st;
  if (int st = launch_moe_combine(o, wt, rows, slots, hidden, y, s)) return st;
  return ok();
}

int qg_quantize_rows_q8(const float* x, int rows, int64_t k, int8_t* qx, float* dx, int32_t* sx, qg_stream stream) {
  if (int st = check_x(x, rows, k, QG_MAX_PREP_ROWS)) return st;
  if (!qx || !dx || !sx) return fail(QG_EINVAL, "null output");
  if (!aligned(qx, 16)) return fail(QG_EALIGN, "qx %p is not 16-byte aligned", (const void*)qx);
  if (int st = check_device()) return st;
  if (int st = launch_quantize_plain(x, rows, k, qx, dx, sx, (hipStream_t)stream)) return st;
  return ok();
}

int qgemv_blockdots(int fmt, const void* w_image, int64_t n, int64_t k, const int8_t* qx, int rows, int32_t* isum,
                    qg_stream stream) {
  if (int st = check_fmt(fmt)) return st;
  if (int st = check_rows(rows)) return st;
  if (int st = check_nk_fmt(fmt, n, k)) return st;
  if (int st = check_image(w_image, "w_image")) return st;
  if (!isum) return fail(QG_EINVAL, "isum is null");
  if (!qx) return fail(QG_EINVAL, "qx is null");
  if (!aligned(qx, 16)) return fail(QG_EALIGN, "qx %p is not 16-byte aligned", (const void*)qx);
  if (rows == 0) return ok();
  if (int st = check_device()) return st;
  if (int st = launch_blockdots(fmt, w_image, n, k, qx, rows, isum, (hipStream_t)stream)) return st;
  return ok();
}

int qgemv_blockdots_pairs(int fmt, const void* w_image, int64_t n, int64_t k, const void* ws, size_t ws_bytes,
                          int rows, int32_t* isum, qg_stream stream) {
  if (int st = check_fmt(fmt)) return st;
  if (rows < 3 || rows > QG_MAX_ROWS) return fail(QG_EROWS, "rows=%d outside 3..%d (pair order)", rows, QG_MAX_ROWS);
  if (int st = check_nk_fmt(fmt, n, k)) return st;
  if (int st = check_image(w_image, "w_image")) return st;
  if (!isum) return fail(QG_EINVAL, "isum is null");
  if (int st = check_ws(ws, ws_bytes, prep_layout(rows, k).total, "the prepared rows")) return st;
  if (int st = check_device()) return st;
  if (int st = launch_pair_blockdots(fmt, w_image, n, k, ws, rows, isum, (hipStream_t)stream)) return st;
  return ok();
}

}  // extern "C"
