// Measurement helpers:
//  * one launch that only streams a buffer from memory, shaped like the decode
//    GEMV's weight stream (1 KB per wave load, every load of a wave issued at
//    once, no other work), so that a benchmark can put the GEMV beside the time a
//    plain read of the same bytes takes in a single launch;
//  * one launch that only issues the prefill GEMM's matrix instruction
//    (v_mfma_i32_32x32x32_i8) on eight independent accumulators per wave, two
//    workgroups of four waves per compute unit like the GEMM, with constant or
//    random-looking int8 operands: the rate the matrix cores sustain with each.
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

constexpr int kMfmaProbeGrid = 512;  // two workgroups per compute unit

typedef int v4i_p __attribute__((ext_vector_type(4)));
typedef int v16i_p __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  return x ^ (x >> 16);
}

template <bool kRandom>
__global__ __launch_bounds__(256, 2) void mfma_probe_kernel(int iters, uint32_t *__restrict__ sink) {
  const uint32_t id = blockIdx.x * 256u + threadIdx.x;
  // two operand sets, used by alternate instructions, so that with random
  // operands consecutive MFMAs of a wave see different bits, as in the GEMM
  v4i_p a[2], b[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[s][i] = kRandom ? (int)probe_hash(8 * id + 4 * s + i) : 0x01010101;
      b[s][i] = kRandom ? (int)probe_hash(0x10000000u + 8 * id + 4 * s + i) : 0x01010101;
    }
  v16i_p acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[m][r] = 0;
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[m & 1], b[m & 1], acc[m], 0, 0, 0);
  int x = 0;
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) x ^= acc[m][r];
  if (x == 0x2545F491) sink[0] = uint32_t(x);  // keeps the sums; the value itself does not matter
}

}  // namespace

hipError_t launch_mfma_probe(int random, int iters, uint32_t *sink, hipStream_t stream) {
  if (iters <= 0) return hipErrorInvalidValue;
  (void)hipGetLastError();
  if (random)
    hipLaunchKernelGGL(mfma_probe_kernel<true>, dim3(kMfmaProbeGrid), dim3(256), 0, stream, iters, sink);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<false>, dim3(kMfmaProbeGrid), dim3(256), 0, stream, iters, sink);
  set_last_kernel(random ? "mfma_probe_random" : "mfma_probe_constant");
  return hipGetLastError();
}

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
