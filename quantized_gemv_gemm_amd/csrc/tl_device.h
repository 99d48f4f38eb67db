// Device helpers shared by the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tl_internal.h"

namespace tl {
// ---------------------------------------------------------------------------
__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  _Float16 v;
  __builtin_memcpy(&v, &h, 2);
  return (float)v;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t h16) {
  return __uint_as_float(h16 << 16);
}

// round-to-nearest-even float -> bfloat16 bits (finite inputs)
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// int8 code of x for the per-token scale sx > 0: clamp(RNE(fl32(x / sx)), -127, 127).
// The quotient is the IEEE binary32 division (correctly rounded; no fast-math),
// which equals rounding the binary64 quotient once to binary32 (53 >= 2 * 24 + 2).
__device__ __forceinline__ int quant_code(float x, float sx) {
  const int q = (int)rintf(x / sx);
  return q > 127 ? 127 : (q < -127 ? -127 : q);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// block-wide max of non-negative values; every thread gets the result
template <int NT>
__device__ __forceinline__ float block_max(float v, float *red /* NT/64 floats */) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (NT > 64) {
    if (lane == 0) red[wave] = v;
    __syncthreads();
    v = red[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) v = fmaxf(v, red[w]);
    __syncthreads();
  }
  return v;
}

}  // namespace tl
