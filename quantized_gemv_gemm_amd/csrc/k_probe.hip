// Measurement helper: one launch that only streams a buffer from memory, shaped
// like the decode GEMV's weight stream (1 KB per wave load, every load of a wave
// issued at once, no other work), so that a benchmark can put the GEMV beside the
// time a plain read of the same bytes takes in a single launch.
#include "tl_device.h"

namespace tl {
namespace {

constexpr int kProbeWaves = 4;     // waves per workgroup
constexpr int kProbeLoads = 2;     // 1 KB loads per wave

__global__ __launch_bounds__(64 * kProbeWaves) void read_probe_kernel(const uint4 *__restrict__ src, int64_t n16,
                                                                      uint32_t *__restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wv = int64_t(blockIdx.x) * kProbeWaves + (threadIdx.x >> 6);
  uint4 v[kProbeLoads];
#pragma unroll
  for (int i = 0; i < kProbeLoads; ++i) {
    const int64_t e = (wv * kProbeLoads + i) * 64 + lane;
    v[i] = e < n16 ? src[e] : make_uint4(0u, 0u, 0u, 0u);
  }
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < kProbeLoads; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  if (acc == 0x9E3779B9u) sink[0] = acc;  // keeps the loads; the value itself does not matter
}

}  // namespace

hipError_t launch_read_probe(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream) {
  const int64_t n16 = int64_t(bytes / 16);
  const int64_t per_wg = 64 * kProbeWaves * kProbeLoads;
  const int64_t grid = (n16 + per_wg - 1) / per_wg;
  if (grid <= 0 || grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  (void)hipGetLastError();
  hipLaunchKernelGGL(read_probe_kernel, dim3(unsigned(grid)), dim3(64 * kProbeWaves), 0, stream,
                     static_cast<const uint4 *>(src), n16, sink);
  set_last_kernel("read_probe");
  return hipGetLastError();
}

}  // namespace tl
