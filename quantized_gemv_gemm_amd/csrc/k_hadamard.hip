// Block Sylvester-Hadamard rotation of the layer input.
//
// Method: qiita.com/nakanokensetsu/items/ecc183fae033565af7cb, "前提" (Hadamard
// rotation on the input side) and "1. TP=2 への移植" (Sylvester type, 1024-wide
// blocks; the transform's last butterfly stage is the sum/difference of two
// 512-halves).  Scaling by 1/32 makes the block transform orthonormal.
//
// Design: one wavefront per (token, 1024-block), 16 values per lane held as
// binary64.  A fast Walsh-Hadamard transform is 10 butterfly stages, one per
// index bit.  Lanes first own 16 consecutive elements (index bits 0-3 in
// registers), then a transpose through LDS gives them bits 4-7, and a second one
// bits 8-9; each phase runs its stages in registers.  binary64 keeps every partial
// sum exact for inputs that are multiples of 2^-31 below 2^8 (bf16 with small
// values flushed), so the f32 output is the exact rotation rounded once.
// Traffic per element: 2 bytes in, 4 bytes out (plus 1 byte of signs per K).
#include "tl_device.h"

namespace tl {
namespace {

constexpr int kEPT = 16;  // elements per lane

__device__ __forceinline__ int lds_pad(int i) { return i + (i >> 4); }

// in-register butterflies (a, b) -> (a + b, a - b) across slot-index bit S
template <int S>
__device__ __forceinline__ void stage(double (&v)[kEPT]) {
#pragma unroll
  for (int j = 0; j < kEPT; ++j) {
    if (!(j & S)) {
      const double a = v[j], b = v[j + S];
      v[j] = a + b;
      v[j + S] = a - b;
    }
  }
}

__global__ __launch_bounds__(64) void hadamard_blk_kernel(const uint16_t *__restrict__ x,
                                                          const int8_t *__restrict__ signs,
                                                          float *__restrict__ xr, int64_t K,
                                                          int nblk) {
  __shared__ double lds[kHBlock + kHBlock / 16];
  const int lane = threadIdx.x;
  const int64_t t = blockIdx.x / nblk;
  const int blk = blockIdx.x - int(t * nblk);
  const int64_t base = t * K + int64_t(blk) * kHBlock;

  // phase A: lane owns elements 16*lane + j
  double v[kEPT];
  {
    const uint4 *src = reinterpret_cast<const uint4 *>(x + base + kEPT * lane);
    const uint4 a = src[0], b = src[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[2 * j] = (double)bf16_bits_to_float(w[j] & 0xFFFFu);
      v[2 * j + 1] = (double)bf16_bits_to_float(w[j] >> 16);
    }
    if (signs) {
      const uint4 s = *reinterpret_cast<const uint4 *>(signs + int64_t(blk) * kHBlock + kEPT * lane);
      const uint32_t sw[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
      for (int j = 0; j < kEPT; ++j) {
        const int8_t d = (int8_t)((sw[j >> 2] >> (8 * (j & 3))) & 0xFF);
        if (d < 0) v[j] = -v[j];
      }
    }
  }
  stage<1>(v);
  stage<2>(v);
  stage<4>(v);
  stage<8>(v);
#pragma unroll
  for (int j = 0; j < kEPT; ++j) lds[lds_pad(kEPT * lane + j)] = v[j];
  __syncthreads();

  // phase B: slot j holds index bits 4-7
  const int ib = (lane & 15) | ((lane >> 4) << 8);
#pragma unroll
  for (int j = 0; j < kEPT; ++j) v[j] = lds[lds_pad(ib | (j << 4))];
  stage<1>(v);
  stage<2>(v);
  stage<4>(v);
  stage<8>(v);
#pragma unroll
  for (int j = 0; j < kEPT; ++j) lds[lds_pad(ib | (j << 4))] = v[j];
  __syncthreads();

  // phase C: element lane + 64 j; slot bits 2-3 are index bits 8-9
#pragma unroll
  for (int j = 0; j < kEPT; ++j) v[j] = lds[lds_pad(lane + 64 * j)];
  stage<4>(v);
  stage<8>(v);
  float *out = xr + base;
#pragma unroll
  for (int j = 0; j < kEPT; ++j) out[lane + 64 * j] = (float)(v[j] * 0.03125);
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
