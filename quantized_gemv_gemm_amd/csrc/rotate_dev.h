// Exact block rotation of one 1024-wide block by one wavefront (device code shared
// by the rotation kernel and the fused rotation -> GEMV prep / quantisation
// kernels).
//
// Method: qiita.com/nakanokensetsu/items/ecc183fae033565af7cb, "前提" (Hadamard
// rotation on the input side) and "1. TP=2 への移植" (Sylvester type, 1024-wide
// blocks; the last butterfly stage is the sum/difference of two 512-halves).
// Scaling by 1/32 makes the block transform orthonormal.
//
// 16 values per lane held as binary64.  A fast Walsh-Hadamard transform is 10
// butterfly stages, one per index bit.  Lanes first own 16 consecutive elements
// (index bits 0-3 in registers), then a transpose through LDS gives them bits 4-7,
// and a second one bits 8-9.  binary64 keeps every partial sum exact for inputs
// that are multiples of 2^-31 below 2^8 (bf16 with small values flushed), so the
// f32 result is the exact rotation rounded once.
#pragma once

#include "tl_device.h"

namespace tl {

constexpr int kRotEPT = 16;                                  // elements per lane
constexpr int kRotLds = kHBlock + kHBlock / 16;              // doubles of LDS per wave

__device__ __forceinline__ int rot_lds_pad(int i) { return i + (i >> 4); }

// in-register butterflies (a, b) -> (a + b, a - b) across slot-index bit S
template <int S>
__device__ __forceinline__ void rot_stage(double (&v)[kRotEPT]) {
#pragma unroll
  for (int j = 0; j < kRotEPT; ++j) {
    if (!(j & S)) {
      const double a = v[j], b = v[j + S];
      v[j] = a + b;
      v[j + S] = a - b;
    }
  }
}

// LDS written by one lane and read by another of the same wavefront
__device__ __forceinline__ void rot_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The lane's raw inputs of one block: its 16 consecutive bf16 values and signs.
struct RotRaw {
  uint4 a, b;  // bf16 elements 16 lane .. 16 lane + 15
  uint4 s;     // their signs (when a sign table is given)
};

__device__ __forceinline__ void rotate_load(const uint16_t *__restrict__ xblk,
                                            const int8_t *__restrict__ sblk, int lane, RotRaw &r) {
  const uint4 *src = reinterpret_cast<const uint4 *>(xblk + kRotEPT * lane);
  r.a = src[0];
  r.b = src[1];
  if (sblk) r.s = *reinterpret_cast<const uint4 *>(sblk + kRotEPT * lane);
}

// Rotates one block from the lane's raw inputs (loaded by rotate_load; signs used
// when `signed_in`).  On return out[j] = fl32(rotation[lane + 64 j]), or with RUNS
// out[4 s + c] = fl32(rotation[256 s + 4 lane + c]): four runs of four consecutive
// elements per lane, for 4-byte and 16-byte stores.  The butterfly stages along
// different index bits commute and every partial sum is exact, so both layouts
// hold the same values.  lds: kRotLds doubles owned by the calling wavefront.
template <bool RUNS = false>
__device__ __forceinline__ void rotate_block_raw(const RotRaw &r, bool signed_in, double *lds, int lane,
                                                 float (&out)[kRotEPT]) {
  // phase A: lane owns elements 16*lane + j
  double v[kRotEPT];
  {
    const uint32_t w[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[2 * j] = (double)bf16_bits_to_float(w[j] & 0xFFFFu);
      v[2 * j + 1] = (double)bf16_bits_to_float(w[j] >> 16);
    }
    if (signed_in) {
      const uint32_t sw[4] = {r.s.x, r.s.y, r.s.z, r.s.w};
#pragma unroll
      for (int j = 0; j < kRotEPT; ++j) {
        const int8_t d = (int8_t)((sw[j >> 2] >> (8 * (j & 3))) & 0xFF);
        if (d < 0) v[j] = -v[j];
      }
    }
  }
  rot_stage<1>(v);
  rot_stage<2>(v);
  rot_stage<4>(v);
  rot_stage<8>(v);
#pragma unroll
  for (int j = 0; j < kRotEPT; ++j) lds[rot_lds_pad(kRotEPT * lane + j)] = v[j];
  rot_wave_sync();

  // phase B: slot j holds index bits 4-7
  const int ib = (lane & 15) | ((lane >> 4) << 8);
#pragma unroll
  for (int j = 0; j < kRotEPT; ++j) v[j] = lds[rot_lds_pad(ib | (j << 4))];
  rot_stage<1>(v);
  rot_stage<2>(v);
  rot_stage<4>(v);
  rot_stage<8>(v);
#pragma unroll
  for (int j = 0; j < kRotEPT; ++j) lds[rot_lds_pad(ib | (j << 4))] = v[j];  // the slots it read
  rot_wave_sync();

  // phase C: slot bits 2-3 are index bits 8-9; the other index bits are the lane's
  // (element lane + 64 j) or, with RUNS, lane bits 0-5 are index bits 2-7 and slot
  // bits 0-1 index bits 0-1 (element 256 (j / 4) + 4 lane + j % 4)
#pragma unroll
  for (int j = 0; j < kRotEPT; ++j)
    v[j] = lds[rot_lds_pad(RUNS ? (j & 3) | (lane << 2) | ((j >> 2) << 8) : lane + 64 * j)];
  rot_stage<4>(v);
  rot_stage<8>(v);
#pragma unroll
  for (int j = 0; j < kRotEPT; ++j) out[j] = (float)(v[j] * 0.03125);
  rot_wave_sync();  // the next block may overwrite lds
}

// Rotates the 1024 bf16 values at xblk (signs: NULL or the block's 1024 signs).
__device__ __forceinline__ void rotate_block_wave(const uint16_t *__restrict__ xblk,
                                                  const int8_t *__restrict__ sblk, double *lds,
                                                  int lane, float (&out)[kRotEPT]) {
  RotRaw r;
  rotate_load(xblk, sblk, lane, r);
  rotate_block_raw(r, sblk != nullptr, lds, lane, out);
}

}  // namespace tl
