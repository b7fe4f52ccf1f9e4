// qg_host.hip -- host side of libqgemv: status reporting, device check,
// size queries and the canonical-block <-> device-image packing.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "qg_internal.h"
#include "qg_layout.h"

namespace qg {

static thread_local int t_last_status = QG_OK;
static thread_local char t_detail[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(t_detail, sizeof t_detail, fmt, ap);
  va_end(ap);
  t_last_status = status;
  return status;
}

int ok() {
  t_last_status = QG_OK;
  t_detail[0] = 0;
  return QG_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return QG_OK;
  return fail(QG_ELAUNCH, "%s failed: %s", what, hipGetErrorString(e));
}

int check_device() {
  static std::mutex mu;
  static std::vector<int> arch_ok;  // per device: 0 unknown, 1 gfx950, -1 other
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(QG_EDEVICE, "no HIP device: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(mu);
  if ((int)arch_ok.size() <= dev) arch_ok.resize(dev + 1, 0);
  if (arch_ok[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(QG_EDEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    arch_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    if (arch_ok[dev] < 0) return fail(QG_EDEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  }
  if (arch_ok[dev] < 0) return fail(QG_EDEVICE, "device %d is not gfx950", dev);
  return QG_OK;
}

}  // namespace qg

using namespace qg;

// The marker qg_device_supported looks for: present in the device code object
// of every build of this library; its value is the version of the image
// layouts and kernels the header declares.
__device__ int qg_layout_marker = 1;

extern "C" {

const char* qg_status_string(int status) {
  switch (status) {
    case QG_OK: return "ok";
    case QG_EINVAL: return "invalid argument";
    case QG_ESHAPE: return "shape out of range";
    case QG_EROWS: return "rows outside 0..16";
    case QG_EALIGN: return "misaligned pointer";
    case QG_EWORKSPACE: return "workspace too small";
    case QG_ELAUNCH: return "HIP launch failed";
    case QG_EDEVICE: return "not a gfx950 device";
    default: return "unknown status";
  }
}

int qg_device_supported(int device) {
  int prev = -1, count = 0;
  if (hipGetDevice(&prev) != hipSuccess || hipGetDeviceCount(&count) != hipSuccess) return 0;
  if (device < 0 || device >= count) return 0;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess || strncmp(prop.gcnArchName, "gfx950", 6) != 0) return 0;
  if (device != prev && hipSetDevice(device) != hipSuccess) return 0;
  void* addr = nullptr;
  size_t bytes = 0;
  const bool ok = hipGetSymbolAddress(&addr, HIP_SYMBOL(qg_layout_marker)) == hipSuccess && addr != nullptr &&
                  hipGetSymbolSize(&bytes, HIP_SYMBOL(qg_layout_marker)) == hipSuccess &&
                  bytes == sizeof(qg_layout_marker);
  if (device != prev && hipSetDevice(prev) != hipSuccess) return 0;
  return ok ? 1 : 0;
}

int qg_last_error_detail(char* buf, size_t len) {
  if (buf && len) {
    strncpy(buf, t_detail, len - 1);
    buf[len - 1] = 0;
  }
  return t_last_status;
}

size_t qg_image_bytes(int fmt, int64_t n, int64_t k) {
  if (n < 1 || k < 1) return 0;
  if (fmt == QG_FMT_F16) return k % 8 ? 0 : (size_t)f16_image_bytes(n, k);
  if (fmt == QG_FMT_FP8) return k % 128 ? 0 : fp8_image_bytes(n, k);
  if (fmt == QG_FMT_Q4_K) return k % QK_K ? 0 : image_total_bytes(fmt, n, k);
  if (fmt != QG_FMT_Q8_0 && fmt != QG_FMT_Q4_0) return 0;
  if (k % QK) return 0;
  return image_total_bytes(fmt, n, k);
}

size_t qg_fp8_workspace_bytes(int rows, int64_t k) {
  if (rows < 1 || rows > QG_MAX_PREP_ROWS || k < 128 || k % 128) return 0;
  return fp8_ws_bytes(rows, k);
}

size_t qg_workspace_bytes(int rows, int64_t k) {
  if (rows < 1 || rows > QG_MAX_PREP_ROWS || k < QK || k % QK) return 0;
  return prep_layout(rows, k).total;
}

size_t qg_fp8_grouped_workspace_bytes(int x_rows, int64_t k, int m) {
  if (x_rows < 1 || x_rows > QG_MAX_PREP_ROWS || k < 128 || k % 128 || m < 0 || m > QG_MAX_ASSIGN) return 0;
  return grouped_fp8_layout(x_rows, k, m).total;
}

size_t qg_grouped_workspace_bytes(int x_rows, int64_t k, int m) {
  if (x_rows < 1 || x_rows > QG_MAX_PREP_ROWS || k < QK || k % QK || m < 0 || m > QG_MAX_ASSIGN) return 0;
  return grouped_layout(x_rows, k, m).total;
}

static int check_pack_args(int fmt, const void* a, int64_t n, int64_t k, const void* b) {
  if (fmt != QG_FMT_Q8_0 && fmt != QG_FMT_Q4_0 && fmt != QG_FMT_F16 && fmt != QG_FMT_FP8 && fmt != QG_FMT_Q4_K)
    return fail(QG_EINVAL, "fmt=%d is not Q8_0 (1), Q4_0 (2), F16 (3), FP8 (4) or Q4_K (5)", fmt);
  if (!a || !b) return fail(QG_EINVAL, "null buffer");
  if (fmt == QG_FMT_Q4_K) {
    if (n < 1 || k < QK_K || k % QK_K)
      return fail(QG_ESHAPE, "n=%lld k=%lld (need n >= 1, k a positive multiple of 256)", (long long)n, (long long)k);
    return QG_OK;
  }
  if (fmt == QG_FMT_FP8) {
    if (n < 1 || k < 128 || k % 128)
      return fail(QG_ESHAPE, "n=%lld k=%lld (need n >= 1, k a positive multiple of 128)", (long long)n, (long long)k);
    return QG_OK;
  }
  if (fmt == QG_FMT_F16) {
    if (n < 1 || k < 8 || k % 8)
      return fail(QG_ESHAPE, "n=%lld k=%lld (need n >= 1, k a positive multiple of 8)", (long long)n, (long long)k);
    return QG_OK;
  }
  if (n < 1 || k < QK || k % QK) return fail(QG_ESHAPE, "n=%lld k=%lld (need n >= 1, k a positive multiple of 32)",
                                             (long long)n, (long long)k);
  return QG_OK;
}

// F16 image chunk c (16 bytes) <-> row-major [n][k] halfwords: chunk l of the
// (tile, step) block holds 8 halfwords of row 16*tile + l % 16 at column
// 32*step + 8*(l / 16).
static void f16_pack_host(const uint16_t* w, int64_t n, int64_t k, uint16_t* img, bool unpack) {
  const int64_t ks = f16_steps(k), tiles = f16_tiles(n);
  for (int64_t t = 0; t < tiles; t++)
    for (int64_t s = 0; s < ks; s++)
      for (int l = 0; l < 64; l++) {
        const int64_t row = 16 * t + l % 16, k0 = 32 * s + 8 * (l / 16);
        uint16_t* chunk = img + ((t * ks + s) * 64 + l) * 8;
        if (row >= n || k0 >= k) continue;
        uint16_t* src = const_cast<uint16_t*>(w) + row * k + k0;
        if (unpack) memcpy(src, chunk, 16);
        else memcpy(chunk, src, 16);
      }
}

// FP8 image chunk <-> canonical codes [n][k] + scales [ceil(n/128)][k/128]:
// lane l = i + 16q of (tile t, group g) holds the codes of row 16t + i,
// columns 128g + 32q .. + 31, the first 16 at 16*l and the other 16 at
// 1024 + 16*l of the 2 KB block; the scales are copied as they are.
static void fp8_pack_host(uint8_t* canon, int64_t n, int64_t k, uint8_t* img, bool unpack) {
  const int64_t kg = k / 128, tiles = f16_tiles(n), nb = (n + 127) / 128;
  for (int64_t t = 0; t < tiles; t++)
    for (int64_t g = 0; g < kg; g++)
      for (int l = 0; l < 64; l++) {
        const int64_t row = 16 * t + l % 16, k0 = 128 * g + 32 * (l / 16);
        if (row >= n) continue;
        for (int h = 0; h < 2; h++) {
          uint8_t* chunk = img + (t * kg + g) * 2048 + h * 1024 + l * 16;
          if (unpack) memcpy(canon + row * k + k0 + 16 * h, chunk, 16);
          else memcpy(chunk, canon + row * k + k0 + 16 * h, 16);
        }
      }
  uint8_t* sc = img + fp8_scale_offset(n, k);
  if (unpack) memcpy(canon + n * k, sc, (size_t)(nb * kg * 4));
  else memcpy(sc, canon + n * k, (size_t)(nb * kg * 4));
}

// Q4_K image <-> canonical superblocks: sub-block j of superblock s of row o
// (canonical weights 32j .. 32j+31: the low nibbles of qs[32(j/2) ..] for even
// j, the high nibbles for odd j) goes to the code cell of block 8s + j in the
// Q4_0 nibble order; the 16-byte header to the header plane.
static void q4k_pack_host(uint8_t* canon, int64_t n, int64_t k, uint8_t* img, bool unpack) {
  const int64_t ns = k / QK_K, kbp = kbp_of(k);
  uint8_t* hdr = img + image_scale_offset(FMT_ID_Q4K, n, k);
  for (int64_t o = 0; o < n; o++)
    for (int64_t s = 0; s < ns; s++) {
      uint8_t* sb = canon + (o * ns + s) * Q4K_CANON;
      uint8_t* h = hdr + q4k_header_offset(o, s, kbp);
      if (unpack) memcpy(sb, h, 16);
      else memcpy(h, sb, 16);
      for (int j = 0; j < 8; j++) {
        uint8_t* cell = img + cell_row_offset(FMT_ID_Q4K, o, 8 * s + j, kbp);
        uint8_t* qs = sb + 16 + 32 * (j / 2);
        const int hi = j & 1;
        for (int l = 0; l < 16; l++) {
          if (unpack) {
            const int c0 = cell[l] & 15, c1 = cell[l] >> 4;  // codes l and l + 16 of the sub-block
            qs[l] = (uint8_t)(hi ? ((qs[l] & 15) | (c0 << 4)) : ((qs[l] & 0xF0) | c0));
            qs[l + 16] = (uint8_t)(hi ? ((qs[l + 16] & 15) | (c1 << 4)) : ((qs[l + 16] & 0xF0) | c1));
          } else {
            const int c0 = hi ? qs[l] >> 4 : qs[l] & 15, c1 = hi ? qs[l + 16] >> 4 : qs[l + 16] & 15;
            cell[l] = (uint8_t)(c0 | (c1 << 4));
          }
        }
      }
    }
}

int qg_pack_image(int fmt, const void* blocks, int64_t n, int64_t k, void* image) {
  int st = check_pack_args(fmt, blocks, n, k, image);
  if (st) return st;
  if (fmt == QG_FMT_Q4_K) {
    memset(image, 0, image_total_bytes(fmt, n, k));
    q4k_pack_host((uint8_t*)blocks, n, k, (uint8_t*)image, false);
    return ok();
  }
  if (fmt == QG_FMT_FP8) {
    memset(image, 0, fp8_image_bytes(n, k));
    fp8_pack_host((uint8_t*)blocks, n, k, (uint8_t*)image, false);
    return ok();
  }
  if (fmt == QG_FMT_F16) {
    memset(image, 0, (size_t)f16_image_bytes(n, k));
    f16_pack_host((const uint16_t*)blocks, n, k, (uint16_t*)image, false);
    return ok();
  }
  const uint8_t* src = (const uint8_t*)blocks;
  uint8_t* dst = (uint8_t*)image;
  memset(dst, 0, image_total_bytes(fmt, n, k));
  const int64_t kb = kb_of(k), kbp = kbp_of(k);
  uint16_t* scales = (uint16_t*)(dst + image_scale_offset(fmt, n, k));
  const int cb = fmt == QG_FMT_Q8_0 ? Q8_CANON : Q4_CANON;
  for (int64_t o = 0; o < n; o++)
    for (int64_t b = 0; b < kb; b++) {
      const uint8_t* blk = src + (o * kb + b) * cb;
      scales[scale_index(o, b, kbp)] = (uint16_t)(blk[0] | (blk[1] << 8));
      uint8_t* cell = dst + cell_row_offset(fmt, o, b, kbp);
      memcpy(cell, blk + 2, 16);
      if (fmt == QG_FMT_Q8_0) memcpy(cell + 256, blk + 18, 16);
      else
        for (int l = 0; l < 16; l++) cell[l] ^= 0x88;  // Q4_0 codes kept as c XOR 8
    }
  return ok();
}

int qg_unpack_image(int fmt, const void* image, int64_t n, int64_t k, void* blocks) {
  int st = check_pack_args(fmt, image, n, k, blocks);
  if (st) return st;
  if (fmt == QG_FMT_Q4_K) {
    memset(blocks, 0, (size_t)(n * (k / QK_K) * Q4K_CANON));
    q4k_pack_host((uint8_t*)blocks, n, k, const_cast<uint8_t*>((const uint8_t*)image), true);
    return ok();
  }
  if (fmt == QG_FMT_FP8) {
    fp8_pack_host((uint8_t*)blocks, n, k, (uint8_t*)image, true);
    return ok();
  }
  if (fmt == QG_FMT_F16) {
    f16_pack_host((uint16_t*)blocks, n, k, (uint16_t*)image, true);
    return ok();
  }
  const uint8_t* src = (const uint8_t*)image;
  uint8_t* dst = (uint8_t*)blocks;
  const int64_t kb = kb_of(k), kbp = kbp_of(k);
  const uint16_t* scales = (const uint16_t*)(src + image_scale_offset(fmt, n, k));
  const int cb = fmt == QG_FMT_Q8_0 ? Q8_CANON : Q4_CANON;
  for (int64_t o = 0; o < n; o++)
    for (int64_t b = 0; b < kb; b++) {
      uint8_t* blk = dst + (o * kb + b) * cb;
      const uint16_t d = scales[scale_index(o, b, kbp)];
      blk[0] = (uint8_t)(d & 0xff);
      blk[1] = (uint8_t)(d >> 8);
      const uint8_t* cell = src + cell_row_offset(fmt, o, b, kbp);
      memcpy(blk + 2, cell, 16);
      if (fmt == QG_FMT_Q8_0) memcpy(blk + 18, cell + 256, 16);
      else
        for (int l = 0; l < 16; l++) blk[2 + l] ^= 0x88;
    }
  return ok();
}

}  // extern "C"
