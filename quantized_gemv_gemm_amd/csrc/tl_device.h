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

// ---------------------------------------------------------------------------
// decode activation limbs
constexpr float kLimbRange = 32639.0f;  // 127 * 257: hi, lo of 256*hi + lo stay in int8

// The two int8 limbs of one 1024-block of token t, held by a wavefront in runs:
// v[4 s + c] is element k0 + 256 s + 4 lane + c (elements at or past len, a
// multiple of 128, are ignored).  The block's scale sigma = |v|max / 32639 goes
// to *sig; each value becomes q = clamp(RNE(fl32(v * fl32(32639 / |v|max))),
// +-32639) = 256 hi + lo with hi = floor((q + 128) / 256), so that lo lies in
// [-128, 127].  A run of four elements is one 4-byte store per limb, in the
// limb layout of the workspace (rows for b <= 8, operand order above).
__device__ __forceinline__ void store_block_limbs(const float (&v)[16], int lane, int t, int b, int64_t K,
                                                  int64_t Kp, int64_t k0, int len, int8_t *__restrict__ xhi,
                                                  float *__restrict__ sig) {
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (256 * (j >> 2) + 4 * lane < len) m = fmaxf(m, fabsf(v[j]));
  m = wave_max(m);
  if (lane == 0) *sig = m / kLimbRange;
  const float inv = m > 0.0f ? kLimbRange / m : 0.0f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int e = 256 * s + 4 * lane;
    if (e >= len) continue;
    uint32_t h = 0, l = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      int q = (int)rintf(v[4 * s + c] * inv);
      q = q > 32639 ? 32639 : (q < -32639 ? -32639 : q);
      const int hi = (q + 128) >> 8;
      h |= uint32_t(hi & 0xFF) << (8 * c);
      l |= uint32_t((q - 256 * hi) & 0xFF) << (8 * c);
    }
    const int64_t k = k0 + e;
    if (b > 8) {
      *reinterpret_cast<uint32_t *>(xhi + limb_frag_offset(t, k, 0, K)) = h;
      *reinterpret_cast<uint32_t *>(xhi + limb_frag_offset(t, k, 1, K)) = l;
    } else {
      *reinterpret_cast<uint32_t *>(xhi + int64_t(t) * Kp + k) = h;
      *reinterpret_cast<uint32_t *>(xhi + (int64_t(b) + t) * Kp + k) = l;
    }
  }
}

}  // namespace tl
