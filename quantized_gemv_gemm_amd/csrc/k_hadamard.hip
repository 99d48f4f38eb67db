// Block Sylvester-Hadamard rotation of the layer input.
//
// Method: qiita.com/nakanokensetsu/items/ecc183fae033565af7cb, "前提" (Hadamard
// rotation on the input side) and "1. TP=2 への移植" (Sylvester type, 1024-wide
// blocks; the transform's last butterfly stage is the sum/difference of two
// 512-halves).  Scaling by 1/32 makes the block transform orthonormal.
//
// Design: one wavefront per (token, 1024-block) running the exact binary64
// butterfly routine of rotate_dev.h.  Traffic per element: 2 bytes in, 4 bytes
// out (plus 1 byte of signs per K).
#include "rotate_dev.h"

namespace tl {
namespace {

__global__ __launch_bounds__(64) void hadamard_blk_kernel(const uint16_t *__restrict__ x,
                                                          const int8_t *__restrict__ signs,
                                                          float *__restrict__ xr, int64_t K,
                                                          int nblk) {
  __shared__ double lds[kRotLds];
  const int lane = threadIdx.x;
  const int64_t t = blockIdx.x / nblk;
  const int blk = blockIdx.x - int(t * nblk);
  const int64_t base = t * K + int64_t(blk) * kHBlock;
  float r[kRotEPT];
  rotate_block_wave(x + base, signs ? signs + int64_t(blk) * kHBlock : nullptr, lds, lane, r);
  float *out = xr + base;
#pragma unroll
  for (int j = 0; j < kRotEPT; ++j) out[lane + 64 * j] = r[j];
}

}  // namespace

hipError_t launch_hadamard(const uint16_t *x, int64_t T, int64_t K, const int8_t *signs, float *xr,
                           hipStream_t stream) {
  const int nblk = int(K / kHBlock);
  const int64_t grid = T * nblk;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  (void)hipGetLastError();  // drop errors left by earlier, unrelated runtime calls
  hipLaunchKernelGGL(hadamard_blk_kernel, dim3(unsigned(grid)), dim3(64), 0, stream, x, signs, xr,
                     K, nblk);
  set_last_kernel("hadamard_blk_f64x16");
  return hipGetLastError();
}

}  // namespace tl
