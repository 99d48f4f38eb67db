// Rotation of a 1024-block that a K-shard boundary splits in the middle, in two
// stages with an exchange between the ranks in between.
//
// Method: qiita.com/nakanokensetsu/items/ecc183fae033565af7cb, "1. TP=2 への移植":
// down_proj's 17408 inputs split over two GPUs at 8704, the middle of a block, and
// the Sylvester recursion H1024 [a; b] = [H512 a + H512 b; H512 a - H512 b] lets
// each rank transform only its own 512 columns; after the exchange the rank with
// the first half keeps the sum and the other the difference.
//
// Stage (hadamard_half_kernel): one wavefront per token; lane l holds columns
// 8l..8l+7 as binary64 (sign applied), runs the three in-lane butterfly levels,
// then six cross-lane levels by lane-xor exchanges.  With the generator's inputs
// every partial sum is exact in binary64 (multiples of 2^-31 below 2^17), so the
// stage result is exact and the join reproduces the unsplit rotation bit for bit.
// Join (hadamard_join_kernel): (u_lo +- u_hi) / 32, rounded once to f32, four
// values per thread.
#include "tl_device.h"

namespace tl {
namespace {

constexpr int kHalf = kHBlock / 2;

__device__ __forceinline__ double shfl_xor_f64(double v, int m) {
  const int64_t b = __double_as_longlong(v);
  const int lo = __shfl_xor(int(b & 0xFFFFFFFF), m, 64);
  const int hi = __shfl_xor(int(b >> 32), m, 64);
  return __longlong_as_double((int64_t(hi) << 32) | uint32_t(lo));
}

__global__ __launch_bounds__(64) void hadamard_half_kernel(const uint16_t *__restrict__ x, int64_t ldx,
                                                           const int8_t *__restrict__ signs,
                                                           double *__restrict__ u) {
  const int lane = threadIdx.x;
  const int64_t t = blockIdx.x;
  const uint4 raw = *reinterpret_cast<const uint4 *>(x + t * ldx + 8 * lane);
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  double v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t h = (w[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
    v[j] = (double)bf16_bits_to_float(h);
    if (signs) v[j] *= (double)signs[8 * lane + j];
  }
  // columns 8 lane + j: levels 1, 2, 4 pair values inside the lane
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if ((j & h) == 0) {
        const double a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
  // levels 8 m pair lane l with lane l ^ m: the lower column takes the sum, the upper the difference
#pragma unroll
  for (int m = 1; m < 64; m <<= 1)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const double o = shfl_xor_f64(v[j], m);
      v[j] = (lane & m) ? o - v[j] : v[j] + o;
    }
  double2 *out = reinterpret_cast<double2 *>(u + t * kHalf + 8 * lane);
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = make_double2(v[2 * j], v[2 * j + 1]);
}

constexpr int kJoinThreads = 128;  // 4 values each: one token row per workgroup

__global__ __launch_bounds__(kJoinThreads) void hadamard_join_kernel(const double *__restrict__ u_lo,
                                                                     const double *__restrict__ u_hi,
                                                                     int half, float *__restrict__ xr,
                                                                     int64_t ldxr) {
  const int64_t t = blockIdx.x;
  const int i = 4 * threadIdx.x;
  const double2 *a = reinterpret_cast<const double2 *>(u_lo + t * kHalf + i);
  const double2 *b = reinterpret_cast<const double2 *>(u_hi + t * kHalf + i);
  const double2 a0 = a[0], a1 = a[1], b0 = b[0], b1 = b[1];
  const double s = half == 0 ? 1.0 : -1.0;  // exact: the sign flip changes no bit but the sign
  float4 r;
  r.x = (float)((a0.x + s * b0.x) * 0.03125);
  r.y = (float)((a0.y + s * b0.y) * 0.03125);
  r.z = (float)((a1.x + s * b1.x) * 0.03125);
  r.w = (float)((a1.y + s * b1.y) * 0.03125);
  *reinterpret_cast<float4 *>(xr + t * ldxr + i) = r;
}

static_assert(kJoinThreads * 4 == kHalf, "one token row per join workgroup");

}  // namespace

hipError_t launch_hadamard_half(const uint16_t *x, int64_t T, int64_t ldx, const int8_t *signs,
                                double *u, hipStream_t stream) {
  if (T > 0x7FFFFFFF) return hipErrorInvalidValue;
  (void)hipGetLastError();  // drop errors left by earlier, unrelated runtime calls
  hipLaunchKernelGGL(hadamard_half_kernel, dim3(unsigned(T)), dim3(64), 0, stream, x, ldx, signs, u);
  set_last_kernel("hadamard_half_f64x8");
  return hipGetLastError();
}

hipError_t launch_hadamard_join(const double *u_lo, const double *u_hi, int64_t T, int half, float *xr,
                                int64_t ldxr, hipStream_t stream) {
  if (T > 0x7FFFFFFF) return hipErrorInvalidValue;
  (void)hipGetLastError();  // drop errors left by earlier, unrelated runtime calls
  hipLaunchKernelGGL(hadamard_join_kernel, dim3(unsigned(T)), dim3(kJoinThreads), 0, stream, u_lo, u_hi,
                     half, xr, ldxr);
  set_last_kernel("hadamard_join_f64");
  return hipGetLastError();
}

}  // namespace tl
