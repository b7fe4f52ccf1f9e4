// qg_probe.hip -- the achievable-read ceiling: a plain streaming read of a
// buffer (16-byte non-temporal loads, the weight loads' form), measured beside
// the GEMV kernels so that their bandwidth can be read against what a bare
// read of the same bytes reaches on the same GPU, not only against the
// 8 TB/s data-sheet figure.  Measurement hook, not part of the GEMV path.
#include <hip/hip_runtime.h>

#include "qg_device.h"
#include "qg_internal.h"

namespace qg {

constexpr int PROBE_WG = 512;

// Workgroup b reads the contiguous 16-byte pieces [b * per, min((b + 1) * per,
// n16)), each thread keeping LA loads in flight, and folds them with xor so
// the loads are not dead; lane 0 of each wave stores its wave's fold.
template <int LA>
__global__ __launch_bounds__(PROBE_WG) void read_probe_kernel(const uint4* __restrict__ src, size_t n16, size_t per,
                                                              uint32_t* __restrict__ sink) {
  const size_t start = (size_t)blockIdx.x * per;
  const size_t end = start + per < n16 ? start + per : n16;
  unsigned acc = 0;
  for (size_t i = start + threadIdx.x; i < end; i += (size_t)PROBE_WG * LA) {
    uint4 v[LA];
#pragma unroll
    for (int j = 0; j < LA; j++) {
      const size_t e = i + (size_t)j * PROBE_WG;
      v[j] = e < end ? ld16_stream(src + e) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int j = 0; j < LA; j++) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (int off = 1; off < WAVE; off <<= 1) acc ^= (unsigned)__shfl_xor((int)acc, off);
  if ((threadIdx.x & (WAVE - 1)) == 0) sink[(size_t)blockIdx.x * (PROBE_WG / WAVE) + threadIdx.x / WAVE] = acc;
}

}  // namespace qg

using namespace qg;

extern "C" int qg_read_probe(const void* src, size_t bytes, int grid, int inflight, uint32_t* sink,
                             qg_stream stream) {
  if (!src || !sink) return fail(QG_EINVAL, "src or sink is null");
  if (!aligned(src, 16) || bytes % 16 || bytes == 0)
    return fail(QG_EALIGN, "src %p / bytes=%zu must be 16-byte aligned, nonzero multiples of 16", src, bytes);
  if (!aligned(sink, 4)) return fail(QG_EALIGN, "sink %p is not 4-byte aligned", (const void*)sink);
  if (grid < 1 || grid > 65536) return fail(QG_EINVAL, "grid=%d outside 1..65536", grid);
  if (inflight != 1 && inflight != 2 && inflight != 4 && inflight != 8)
    return fail(QG_EINVAL, "inflight=%d is not 1, 2, 4 or 8", inflight);
  if (int st = check_device()) return st;
  const size_t n16 = bytes / 16;
  const size_t per = ((n16 + grid - 1) / grid + PROBE_WG - 1) / PROBE_WG * PROBE_WG;
  const unsigned g = (unsigned)((n16 + per - 1) / per);  // every launched workgroup has pieces to read
  hipStream_t s = (hipStream_t)stream;
  const uint4* p = reinterpret_cast<const uint4*>(src);
  switch (inflight) {
    case 1: hipLaunchKernelGGL(read_probe_kernel<1>, dim3(g), dim3(PROBE_WG), 0, s, p, n16, per, sink); break;
    case 2: hipLaunchKernelGGL(read_probe_kernel<2>, dim3(g), dim3(PROBE_WG), 0, s, p, n16, per, sink); break;
    case 4: hipLaunchKernelGGL(read_probe_kernel<4>, dim3(g), dim3(PROBE_WG), 0, s, p, n16, per, sink); break;
    default: hipLaunchKernelGGL(read_probe_kernel<8>, dim3(g), dim3(PROBE_WG), 0, s, p, n16, per, sink); break;
  }
  if (int st = hip_status(hipGetLastError(), "read_probe_kernel")) return st;
  return ok();
}
