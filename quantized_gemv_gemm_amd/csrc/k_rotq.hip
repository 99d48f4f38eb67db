// Fused layer-input kernels: block rotation -> GEMV activation limbs (decode) and
// block rotation -> per-token int8 quantisation (prefill), so that the rotated
// activations are never written to memory.
//
// Method: qiita.com/nakanokensetsu/items/ecc183fae033565af7cb, "前提" (rotation
// on the input side), "4. 効いた高速化" (per-token int8 after the rotation).
// Both kernels produce exactly what the unfused pair produces: the rotation is the
// same wave routine (exact in binary64, rounded once to f32), the maximum is over
// those f32 values, and each element is then converted with the same f32 /
// binary64 expressions as the GEMV prep and the quantisation kernels
// (store_block_limbs, quant_code).
//
// GEMV limbs: one wavefront per (token, 1024-block); the limbs are scaled per
// block, so no wave waits for another, and the rotation hands each lane four runs
// of four consecutive elements, stored as 4-byte words.
// int8 activations (scaled per token): one workgroup per token of W waves; wave w
// rotates blocks w, w + W, ... into registers (at most BPW blocks,
// W = ceil(blocks / BPW) <= 16, BPW chosen by fuse_shape), the workgroup reduces
// |x|max, and every lane converts and stores its own elements (lane + 64 j of each
// block: 64 consecutive bytes per wave store).
#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>

#include "rotate_dev.h"

namespace tl {
namespace {

constexpr int kMaxWaves = 16;

template <int BPW>
__device__ __forceinline__ float rotate_token(const uint16_t *__restrict__ xrow,
                                              const int8_t *__restrict__ signs, int nblk,
                                              double *lds, int wave, int W, int lane,
                                              float (&r)[BPW][kRotEPT]) {
  float m = 0.0f;
  // every block's inputs are requested before the first rotation starts (up to
  // three blocks per wave; beyond that the raw inputs would not fit the registers)
  constexpr int kPre = BPW <= 3 ? BPW : 1;
  RotRaw raw[kPre];
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    const int blk = wave + i * W;
    if (blk < nblk)
      rotate_load(xrow + int64_t(blk) * kHBlock, signs ? signs + int64_t(blk) * kHBlock : nullptr, lane,
                  raw[i]);
  }
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int blk = wave + i * W;
    if (blk < nblk) {
      if (i >= kPre)
        rotate_load(xrow + int64_t(blk) * kHBlock, signs ? signs + int64_t(blk) * kHBlock : nullptr, lane,
                    raw[0]);
      rotate_block_raw(raw[i < kPre ? i : 0], signs != nullptr, lds, lane, r[i]);
#pragma unroll
      for (int j = 0; j < kRotEPT; ++j) m = fmaxf(m, fabsf(r[i][j]));
    }
  }
  return m;
}

// max over the workgroup's W waves; every thread gets it
__device__ __forceinline__ float token_max(float m, float *red, int wave, int W, int lane) {
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  float v = red[0];
  for (int w = 1; w < W; ++w) v = fmaxf(v, red[w]);
  return v;
}

__global__ __launch_bounds__(64) void gemv_prep_x_kernel(const uint16_t *__restrict__ x,
                                                         const int8_t *__restrict__ signs, int64_t K, int64_t Kp,
                                                         int b, int8_t *__restrict__ xhi,
                                                         float *__restrict__ sigma) {
  __shared__ double lds[kRotLds];
  const int lane = threadIdx.x;
  const int nblk = int(K / kHBlock);
  const int t = int(blockIdx.x / unsigned(nblk)), blk = int(blockIdx.x - unsigned(t * nblk));
  const int64_t k0 = int64_t(blk) * kHBlock;
  RotRaw raw;
  rotate_load(x + int64_t(t) * K + k0, signs ? signs + k0 : nullptr, lane, raw);
  float r[kRotEPT];
  rotate_block_raw<true>(raw, signs != nullptr, lds, lane, r);
  store_block_limbs(r, lane, t, b, K, Kp, k0, kHBlock, xhi, sigma + int64_t(t) * nblk + blk);
}

template <int BPW>
__global__ __launch_bounds__(64 * kMaxWaves) void quant_x_kernel(
    const uint16_t *__restrict__ x, const int8_t *__restrict__ signs, int64_t K,
    int8_t *__restrict__ xq, float *__restrict__ tok_scale) {
  extern __shared__ double lds[];  // W * kRotLds
  __shared__ float red[kMaxWaves];
  const int W = blockDim.x >> 6, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nblk = int(K / kHBlock);
  const int64_t t = blockIdx.x;
  float r[BPW][kRotEPT];
  const float m = rotate_token<BPW>(x + t * K, signs, nblk, lds + wave * kRotLds, wave, W, lane, r);
  const float amax = token_max(m, red, wave, W, lane);
  const float sx = (float)((double)amax / 127.0);
  if (threadIdx.x == 0) tok_scale[t] = sx;
  const bool live = sx > 0.0f;
  int8_t *orow = xq + t * K;
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int blk = wave + i * W;
    if (blk < nblk) {
#pragma unroll
      for (int j = 0; j < kRotEPT; ++j) {
        const int qi = live ? quant_code(r[i][j], sx) : 0;
        orow[int64_t(blk) * kHBlock + lane + 64 * j] = (int8_t)qi;
      }
    }
  }
}

struct FuseShape {
  int waves, bpw;
  size_t lds;
};

// workgroups of a rotation -> int8 variant resident per compute unit (0: unknown)
int fuse_resident(int bpw, int waves) {
  static std::mutex mu;
  static std::map<std::tuple<int, int>, int> cache;
  const auto key = std::make_tuple(bpw, waves);
  {
    std::lock_guard<std::mutex> lock(mu);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  const void *fn = bpw == 1 ? reinterpret_cast<const void *>(quant_x_kernel<1>)
                 : bpw == 2 ? reinterpret_cast<const void *>(quant_x_kernel<2>)
                 : bpw == 3 ? reinterpret_cast<const void *>(quant_x_kernel<3>)
                            : reinterpret_cast<const void *>(quant_x_kernel<4>);
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, 64 * waves,
                                                   size_t(waves) * kRotLds * sizeof(double)) != hipSuccess)
    n = 0;
  (void)hipGetLastError();
  std::lock_guard<std::mutex> lock(mu);
  cache[key] = n;
  return n;
}

// Blocks per wave (and so waves per workgroup, one workgroup per token): the
// fewest rounds x blocks per wave, where a round is as many tokens as the chip
// holds at once (residency from the runtime's occupancy figure, else by LDS).
// Few tokens (decode): one round whatever the shape, so one block per wave.
// 512 tokens of K = 17408 (17 blocks): 6 waves x 3 blocks, two workgroups per CU,
// rather than 16 waves x 2 blocks with one (LDS) and a wave left doing two blocks.
FuseShape fuse_shape(int64_t K, int64_t T) {
  const int nblk = int(K / kHBlock);
  FuseShape best{};
  int64_t best_cost = INT64_MAX;
  for (int bpw = 1; bpw <= 4; ++bpw) {
    const int waves = (nblk + bpw - 1) / bpw;
    if (waves > kMaxWaves) continue;
    if (bpw == 4 && nblk <= 3 * kMaxWaves) continue;  // four blocks per wave spill: only when needed
    const size_t lds = size_t(waves) * kRotLds * sizeof(double);
    int64_t per_cu = fuse_resident(bpw, waves);
    if (per_cu <= 0) per_cu = std::max<int64_t>(1, int64_t(160 * 1024 / lds));
    const int64_t rounds = (T + 256 * per_cu - 1) / (256 * per_cu);
    if (rounds * bpw < best_cost) {
      best_cost = rounds * bpw;
      best = FuseShape{waves, bpw, lds};
    }
  }
  return best;
}

}  // namespace

bool fused_input_supported(int64_t K) { return K > 0 && K % kHBlock == 0 && K <= 4 * kMaxWaves * kHBlock; }

hipError_t launch_gemv_prepare_x(const uint16_t *x, int64_t b, int64_t K, const int8_t *signs,
                                 int8_t *xhi, int64_t Kp, float *sigma, hipStream_t stream) {
  const int64_t grid = b * (K / kHBlock);
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  (void)hipGetLastError();  // drop errors left by earlier, unrelated runtime calls
  hipLaunchKernelGGL(gemv_prep_x_kernel, dim3(unsigned(grid)), dim3(64), 0, stream, x, signs, K, Kp, int(b), xhi,
                     sigma);
  set_last_kernel("gemv_prep_rotate_limbs");
  return hipGetLastError();
}

hipError_t launch_quant_x(const uint16_t *x, int64_t T, int64_t K, const int8_t *signs, int8_t *xq,
                          float *tok_scale, hipStream_t stream) {
  if (T > 0x7FFFFFFF) return hipErrorInvalidValue;
  const FuseShape s = fuse_shape(K, T);
  const dim3 grid{unsigned(T)}, blk{unsigned(64 * s.waves)};
  (void)hipGetLastError();  // drop errors left by earlier, unrelated runtime calls
  switch (s.bpw) {
    case 1: hipLaunchKernelGGL(quant_x_kernel<1>, grid, blk, s.lds, stream, x, signs, K, xq, tok_scale); break;
    case 2: hipLaunchKernelGGL(quant_x_kernel<2>, grid, blk, s.lds, stream, x, signs, K, xq, tok_scale); break;
    case 3: hipLaunchKernelGGL(quant_x_kernel<3>, grid, blk, s.lds, stream, x, signs, K, xq, tok_scale); break;
    default: hipLaunchKernelGGL(quant_x_kernel<4>, grid, blk, s.lds, stream, x, signs, K, xq, tok_scale); break;
  }
  set_last_kernel("quant_rotate_int8");
  return hipGetLastError();
}

}  // namespace tl
