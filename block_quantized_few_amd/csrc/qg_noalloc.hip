// qg_noalloc.hip -- qgemv_q8_0 for callers that cannot allocate (code under
// graph capture, serving loops, harnesses that forbid hipMalloc): the q8
// activation workspace is a fixed-size device array of this file, one per
// GPU, held until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "qg_internal.h"
#include "qg_launch.h"
#include "qg_layout.h"

namespace qg {

// The workspace.  In host code this name is only a stand-in for the symbol:
// every use goes through the device address hipGetSymbolAddress returns.
static __device__ __align__(256) uint8_t scratch[QG_NOALLOC_SCRATCH_BYTES];

// The calling thread's current device's address of `scratch`, looked up once
// per device with that device current.
static int scratch_address(void** out) {
  static std::mutex mu;
  static std::vector<void*> addr;
  int dev = -1;
  if (int st = hip_status(hipGetDevice(&dev), "hipGetDevice")) return st;
  std::lock_guard<std::mutex> lk(mu);
  if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
  if (!addr[dev]) {
    void* p = nullptr;
    if (int st = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)")) return st;
    if (!p) return fail(QG_ELAUNCH, "hipGetSymbolAddress(scratch) gave a null address");
    addr[dev] = p;
  }
  *out = addr[dev];
  return QG_OK;
}

}  // namespace qg

using namespace qg;

extern "C" int qgemv_q8_0_noalloc(const void* w_image, int64_t n, int64_t k, const float* x, int rows, float* y,
                                  qg_stream stream) {
  if (rows < 0 || rows > QG_MAX_ROWS) return fail(QG_EROWS, "rows=%d outside 0..%d", rows, QG_MAX_ROWS);
  if (n < 1 || n > (1LL << 31) - 16) return fail(QG_ESHAPE, "n=%lld outside 1..2^31-16", (long long)n);
  if (k < QK || k % QK || k > (1LL << 24))
    return fail(QG_ESHAPE, "k=%lld is not a positive multiple of 32 up to 2^24", (long long)k);
  if (!w_image) return fail(QG_EINVAL, "w_image is null");
  if (!aligned(w_image, 256)) return fail(QG_EALIGN, "w_image %p is not 256-byte aligned", w_image);
  if (!y) return fail(QG_EINVAL, "y is null");
  if (!aligned(y, 4)) return fail(QG_EALIGN, "y %p is not 4-byte aligned", (const void*)y);
  if (rows == 0) return ok();
  if (!x) return fail(QG_EINVAL, "x is null");
  if (!aligned(x, 16)) return fail(QG_EALIGN, "x %p is not 16-byte aligned", (const void*)x);
  // 1-2 rows that fit the launch's staging area are quantized inside the GEMV launch: no workspace
  const bool fused = fuses_quantization(QG_FMT_Q8_0, rows, k);
  const PrepLayout L = prep_layout(rows, k);
  if (!fused && L.total > (size_t)QG_NOALLOC_SCRATCH_BYTES)
    return fail(QG_EWORKSPACE, "rows=%d k=%lld need %zu workspace bytes, more than the %u of the static workspace",
                rows, (long long)k, L.total, (unsigned)QG_NOALLOC_SCRATCH_BYTES);
  if (int st = check_device()) return st;
  hipStream_t s = (hipStream_t)stream;
  ProjArg pa{w_image, n, k, nullptr, nullptr, y};
  if (fused) {
    pa.x = x;
  } else {
    void* ws = nullptr;
    if (int st = scratch_address(&ws)) return st;
    pa.ws = ws;
    // every byte the GEMV reads is written here (pair order clears the zero lanes; pad rows and blocks come out
    // zero), so nothing of the previous call's contents is read
    if (int st = launch_prepare(x, rows, k, ws, L, s)) return st;
  }
  if (int st = launch_qgemv_set(QG_FMT_Q8_0, &pa, 1, rows, s)) return st;
  return ok();
}
