// Decode GEMV of the ternary layer: y[t, n] = sum_g s[n,g] sum_{k in g} code[n,k] xr[t,k]
// for 1..16 tokens.
//
// Method: qiita.com/nakanokensetsu/items/ecc183fae033565af7cb, "前提" (y = W (H_blk x)
// with W = 2-bit code times a per-128 fp16 scale).  The page does not describe its
// decode kernel; this design is ours, for CDNA4.
//
// The weight stream (0.25 byte per weight + 1/64 byte of scale) is the only
// HBM-sized input, so each packed word is read once and serves all b tokens.
// Unpacking must be cheap: with the packed layout of include/tl.h,
// (w << (6 - 2r)) & 0xC0C0C0C0 yields codes 4r..4r+3 as int8 values 64*code, in
// k order -- one or two VALU ops per four weights.  The contraction runs on the
// int8 matrix cores (v_mfma_i32_16x16x64_i8): rows of D are the 16 token slots,
// columns are 16 weight rows, so one instruction covers 16 rows x 64 k for every
// token at once, and per-group results are exact integers.
//
// Activations must keep about 15 bits for a 1e-3 output error bar, so a prep
// kernel turns each token row into a fixed-point value v = RNE(x * 32639/amax)
// split into two int8 limbs, v = 256 hi + lo (hi in [-127,127], lo in
// [-128,127]).  Each group runs two MFMA chains (hi and lo) on the same unpacked
// weights; 256 D_hi + D_lo is the exact group sum, converted to f32 and
// multiplied by the group scale.  At the end the token scale amax/32639 and the
// weights' factor 1/64 are applied.
//
// Weights come in the wavefront-shaped tiles of the packed layout: for a pair of
// groups and 16 rows, lane l's 16 contiguous bytes are exactly its fragment words
// for both groups, so every weight load instruction reads 1 KB contiguously.
// Work split: a workgroup owns 16*RB consecutive rows and all of K; its waves take
// contiguous runs of group pairs, and the partial sums are reduced through LDS.
// Two kernels:
//  * gemv_lds: for small b*K.  The workgroup copies the limbs of all b tokens
//    into LDS once (global_load_lds); each wave issues every weight load it
//    needs at once (at most PMAX pairs), so a wave holds only weights in
//    registers and many workgroups stay resident.
//  * gemv_reg: for large b*K.  Limb fragments are loaded into registers with the
//    weights, two pairs in flight, and are shared by RB row blocks.
// Rows past N and token slots past b read clamped, valid addresses (no divergent
// branches around loads) and their results are never stored.
#include "tl_device.h"

namespace tl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr float kLimbRange = 32639.0f;  // 127 * 257: hi, lo of 256*hi + lo stay in int8
constexpr int kRowPad = 16;             // bytes after each limb row: spreads LDS banks

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// workspace: hi limbs [b][Kp] then lo limbs [b][Kp] (contiguous), then sigma[16]
struct GemvWs {
  int8_t *xhi;
  float *sigma;
  int64_t Kp;
};
GemvWs carve(void *workspace, int64_t b, int64_t K) {
  char *ws = static_cast<char *>(workspace);
  const int64_t Kp = K + kRowPad;
  return {reinterpret_cast<int8_t *>(ws), reinterpret_cast<float *>(ws + align256(2 * size_t(b) * Kp)),
          Kp};
}

// --------------------------------------------------------------------------
// prep: xr f32 [b, K] -> limb rows hi, lo and sigma[t] = amax_t / 32639
// --------------------------------------------------------------------------
constexpr int kPrepThreads = 256;

__global__ __launch_bounds__(kPrepThreads) void gemv_prep_kernel(const float *__restrict__ xr,
                                                                 int64_t K, int64_t Kp, int b,
                                                                 int8_t *__restrict__ xhi,
                                                                 float *__restrict__ sigma) {
  __shared__ float red[kPrepThreads / 64];
  const int64_t t = blockIdx.x;
  const float *row = xr + t * K;
  float m = 0.0f;
  for (int64_t i = 4 * threadIdx.x; i < K; i += 4 * kPrepThreads) {
    const float4 v = *reinterpret_cast<const float4 *>(row + i);
    m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  const float amax = block_max<kPrepThreads>(m, red);
  const float inv = amax > 0.0f ? kLimbRange / amax : 0.0f;
  if (threadIdx.x == 0) sigma[t] = amax / kLimbRange;
  int8_t *hrow = xhi + t * Kp;
  int8_t *lrow = xhi + (int64_t(b) + t) * Kp;
  for (int64_t i = 16 * threadIdx.x; i < K; i += 16 * kPrepThreads) {
    const float4 *src = reinterpret_cast<const float4 *>(row + i);
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float4 v = src[c];
      const float f[4] = {v.x, v.y, v.z, v.w};
      uint32_t h = 0, l = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int q = (int)rintf(f[e] * inv);
        q = q > 32639 ? 32639 : (q < -32639 ? -32639 : q);
        const int hi = (q + 128) >> 8;  // floor division: lo lands in [-128, 127]
        const int lo = q - hi * 256;
        h |= (uint32_t)(hi & 0xFF) << (8 * e);
        l |= (uint32_t)(lo & 0xFF) << (8 * e);
      }
      hw[c] = h;
      lw[c] = l;
    }
    *reinterpret_cast<uint4 *>(hrow + i) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    *reinterpret_cast<uint4 *>(lrow + i) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
}

// --------------------------------------------------------------------------
// shared pieces of the weight-streaming kernels
// --------------------------------------------------------------------------
// codes 4r..4r+3 of word w as int8 values 64*code (byte order = k order)
__device__ __forceinline__ v4i unpack_x64(uint32_t w) {
  v4i r;
  r[0] = (int)((w << 6) & 0xC0C0C0C0u);
  r[1] = (int)((w << 4) & 0xC0C0C0C0u);
  r[2] = (int)((w << 2) & 0xC0C0C0C0u);
  r[3] = (int)(w & 0xC0C0C0C0u);
  return r;
}

// A operand row r holds token 4*(r%4) + r/4, so D row 4q+i (lane quarter q,
// accumulator i) holds token 4i + q: for b <= 4 every token sits in i = 0 and the
// epilogue only touches the first ceil(b/4) accumulators.
__device__ __forceinline__ int token_of_arow(int r) { return 4 * (r & 3) + (r >> 2); }

// one group for RB row blocks: two 64-k halves x two limbs, then f32 accumulation.
// w0/w1 are the lane's packed words for the group's two 64-k halves.
template <int RB, int NT>
__device__ __forceinline__ void group_mfma(const v4i (&ah)[2], const v4i (&al)[2],
                                           const uint32_t (&w0)[RB], const uint32_t (&w1)[RB],
                                           const float (&s)[RB], float (&acc)[RB][4]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const v4i z = {0, 0, 0, 0};
    const v4i b0 = unpack_x64(w0[rb]);
    const v4i b1 = unpack_x64(w1[rb]);
    v4i dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah[0], b0, z, 0, 0, 0);
    v4i dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(al[0], b0, z, 0, 0, 0);
    dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah[1], b1, dh, 0, 0, 0);
    dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(al[1], b1, dl, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[rb][i] = fmaf(s[rb], (float)(dh[i] * 256 + dl[i]), acc[rb][i]);
  }
}

// both groups of a pair: tile words .x/.y feed group 2p, .z/.w group 2p+1
template <int RB, int NT>
__device__ __forceinline__ void pair_mfma(const v4i (&ah)[2][2], const v4i (&al)[2][2],
                                          const uint4 (&w)[RB], const float (&s)[2][RB],
                                          float (&acc)[RB][4]) {
  uint32_t a0[RB], a1[RB], b0[RB], b1[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    a0[rb] = w[rb].x;
    a1[rb] = w[rb].y;
    b0[rb] = w[rb].z;
    b1[rb] = w[rb].w;
  }
  group_mfma<RB, NT>(ah[0], al[0], a0, a1, s[0], acc);
  group_mfma<RB, NT>(ah[1], al[1], b0, b1, s[1], acc);
}

// the lane's 16 bytes of tile (row block rbg, pair p): one coalesced kilobyte per wave
__device__ __forceinline__ uint4 load_tile(const uint32_t *__restrict__ packed, int64_t rbg, int GP,
                                           int p, int lane) {
  return *reinterpret_cast<const uint4 *>(packed + 256 * (rbg * GP + p) + 4 * lane);
}

// group scales of the lane's row for groups 2p and 2p+1 (0 past the last group)
__device__ __forceinline__ void load_pair_scales(const uint16_t *__restrict__ srow, int G, int p,
                                                 float &s0, float &s1) {
  const int g0 = 2 * p, g1 = 2 * p + 1;
  s0 = half_bits_to_float(srow[g0]);
  s1 = g1 < G ? half_bits_to_float(srow[g1]) : 0.0f;
}

// partial sums of the W waves -> LDS -> wave 0 scales by sigma/64 and stores
template <int RB, int NT>
__device__ __forceinline__ void reduce_and_store(float (&acc)[RB][4], float *red, int W, int wave,
                                                 int lane, int b, int64_t n0, int64_t N,
                                                 const float *__restrict__ sigma, void *y,
                                                 int y_dtype) {
  const int col = lane & 15, qd = lane >> 4;
  if (W > 1) {
    if (wave > 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < NT; ++i) red[(((wave - 1) * RB + rb) * NT + i) * 64 + lane] = acc[rb][i];
    }
    __syncthreads();
    if (wave > 0) return;
    for (int w = 1; w < W; ++w)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < NT; ++i) acc[rb][i] += red[(((w - 1) * RB + rb) * NT + i) * 64 + lane];
  }
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int t = 4 * i + qd;  // token held by D row 4*qd + i
    if (t >= b) continue;
    const float sc = sigma[t] * (1.0f / 64.0f);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int64_t n = n0 + 16 * rb + col;
      if (n >= N) continue;
      const float v = acc[rb][i] * sc;
      if (y_dtype == TL_F32)
        reinterpret_cast<float *>(y)[int64_t(t) * N + n] = v;
      else
        reinterpret_cast<uint16_t *>(y)[int64_t(t) * N + n] = float_to_bf16_bits(v);
    }
  }
}

// --------------------------------------------------------------------------
// gemv_lds: limbs staged in LDS, every weight load of a wave issued up front
// --------------------------------------------------------------------------
template <int RB, int NT, int PMAX>
__global__ __launch_bounds__(1024) void gemv_lds_kernel(
    const int8_t *__restrict__ limbs, const float *__restrict__ sigma, int b, int64_t K,
    int64_t Kp, int64_t N, const uint32_t *__restrict__ packed, const uint16_t *__restrict__ scales,
    void *__restrict__ y, int y_dtype, int lds_limb_bytes) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int8_t *lx = reinterpret_cast<int8_t *>(smem);
  float *red = reinterpret_cast<float *>(smem + lds_limb_bytes);
  const int W = blockDim.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15, qd = lane >> 4;
  const int G = int(K / kGroup);
  const int GP = (G + 1) >> 1;
  const int64_t NB = (N + 15) >> 4;
  const int p_begin = (GP * wave) / W;
  const int p_end = (GP * (wave + 1)) / W;
  const int64_t n0 = int64_t(blockIdx.x) * (16 * RB);

  // 1. every weight tile and scale pair this wave needs (at most PMAX pairs)
  uint4 wv[PMAX][RB];
  float sv[PMAX][2][RB];
#pragma unroll
  for (int pi = 0; pi < PMAX; ++pi) {
    if (p_begin + pi < p_end) {
      const int p = p_begin + pi;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int64_t rbg = min(int64_t(blockIdx.x) * RB + rb, NB - 1);
        const int64_t n = n0 + 16 * rb + col;
        const int64_t nn = n < N ? n : N - 1;
        wv[pi][rb] = load_tile(packed, rbg, GP, p, lane);
        load_pair_scales(scales + nn * G, G, p, sv[pi][0][rb], sv[pi][1][rb]);
      }
    }
  }
  // 2. limbs of all b tokens -> LDS, 1 KB per wave per step, straight from global
  for (int blk = wave; blk * 1024 < lds_limb_bytes; blk += W) {
    const int64_t off = int64_t(blk) * 1024 + 16 * lane;
    const int64_t src = off < 2 * int64_t(b) * Kp ? off : 0;
    __builtin_amdgcn_global_load_lds(limbs + src,
                                     (__attribute__((address_space(3))) void *)(lx + blk * 1024), 16,
                                     0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // 3. compute
  float acc[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[rb][i] = 0.0f;
  const int tok = token_of_arow(col);
  const int tok_ld = tok < b ? tok : b - 1;
  const int8_t *lah = lx + int64_t(tok_ld) * Kp + 32 * qd;
  const int8_t *lal = lah + int64_t(b) * Kp;
#pragma unroll
  for (int pi = 0; pi < PMAX; ++pi) {
    if (p_begin + pi < p_end) {
      const int p = p_begin + pi;
      v4i ah[2][2], al[2][2];
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const int gl = min(2 * p + gi, G - 1);  // a padded last group reads a valid row part
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          ah[gi][h] = *reinterpret_cast<const v4i *>(lah + 128 * gl + 16 * h);
          al[gi][h] = *reinterpret_cast<const v4i *>(lal + 128 * gl + 16 * h);
        }
      }
      pair_mfma<RB, NT>(ah, al, wv[pi], sv[pi], acc);
    }
  }
  __syncthreads();  // every wave is done with the limbs before `red` is written
  reduce_and_store<RB, NT>(acc, red, W, wave, lane, b, n0, N, sigma, y, y_dtype);
}

// --------------------------------------------------------------------------
// gemv_reg: limb fragments in registers, two pairs of groups in flight per wave
// --------------------------------------------------------------------------
template <int RB>
struct PairSlot {
  v4i ah[2][2], al[2][2];  // limbs: [group of the pair][64-k half]
  uint4 w[RB];             // tile words, per row block
  float s[2][RB];          // group scales
};

template <int RB>
__device__ __forceinline__ void load_pair(PairSlot<RB> &f, int p, int G, int GP, const int8_t *ah,
                                          const int8_t *al, const uint32_t *__restrict__ packed,
                                          const int64_t (&rbg)[RB], const uint16_t *const (&srow)[RB],
                                          int lane) {
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const int gl = min(2 * p + gi, G - 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f.ah[gi][h] = *reinterpret_cast<const v4i *>(ah + 128 * int64_t(gl) + 16 * h);
      f.al[gi][h] = *reinterpret_cast<const v4i *>(al + 128 * int64_t(gl) + 16 * h);
    }
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    f.w[rb] = load_tile(packed, rbg[rb], GP, p, lane);
    load_pair_scales(srow[rb], G, p, f.s[0][rb], f.s[1][rb]);
  }
}

// wave cap per workgroup: larger row tiles need more registers per wave
template <int RB>
struct GemvWaveCap {
  static constexpr int value = RB == 1 ? 12 : RB == 2 ? 8 : 4;
};

template <int RB, int NT>
__global__ __launch_bounds__(64 * GemvWaveCap<RB>::value) void gemv_reg_kernel(
    const int8_t *__restrict__ limbs, const float *__restrict__ sigma, int b, int64_t K,
    int64_t Kp, int64_t N, const uint32_t *__restrict__ packed, const uint16_t *__restrict__ scales,
    void *__restrict__ y, int y_dtype) {
  extern __shared__ float red[];  // (W - 1) * RB * NT * 64 floats
  const int W = blockDim.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15, qd = lane >> 4;
  const int G = int(K / kGroup);
  const int GP = (G + 1) >> 1;
  const int64_t NB = (N + 15) >> 4;
  const int p_begin = (GP * wave) / W;
  const int p_end = (GP * (wave + 1)) / W;
  const int64_t n0 = int64_t(blockIdx.x) * (16 * RB);

  const int tok = token_of_arow(col);
  const int tok_ld = tok < b ? tok : b - 1;
  const int8_t *ah = limbs + int64_t(tok_ld) * Kp + 32 * qd;
  const int8_t *al = ah + int64_t(b) * Kp;
  int64_t rbg[RB];
  const uint16_t *srow[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    rbg[rb] = min(int64_t(blockIdx.x) * RB + rb, NB - 1);
    const int64_t n = n0 + 16 * rb + col;
    srow[rb] = scales + (n < N ? n : N - 1) * G;
  }

  float acc[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[rb][i] = 0.0f;

  // two pair slots: slot (p - p_begin) % 2; the next pair is in flight while one is used
  PairSlot<RB> sl[2];
  if (p_begin < p_end) load_pair<RB>(sl[0], p_begin, G, GP, ah, al, packed, rbg, srow, lane);
  if (p_begin + 1 < p_end) load_pair<RB>(sl[1], p_begin + 1, G, GP, ah, al, packed, rbg, srow, lane);
  for (int p = p_begin; p < p_end; p += 2) {
    pair_mfma<RB, NT>(sl[0].ah, sl[0].al, sl[0].w, sl[0].s, acc);
    if (p + 2 < p_end) load_pair<RB>(sl[0], p + 2, G, GP, ah, al, packed, rbg, srow, lane);
    if (p + 1 < p_end) {
      pair_mfma<RB, NT>(sl[1].ah, sl[1].al, sl[1].w, sl[1].s, acc);
      if (p + 3 < p_end) load_pair<RB>(sl[1], p + 3, G, GP, ah, al, packed, rbg, srow, lane);
    }
  }
  reduce_and_store<RB, NT>(acc, red, W, wave, lane, b, n0, N, sigma, y, y_dtype);
}

// --------------------------------------------------------------------------
// variant choice and launch
// --------------------------------------------------------------------------
struct GemvPlan {
  bool lds;
  int rb, waves, pmax;
  int lds_limb_bytes;
  size_t lds_bytes;
  const char *name;
};

constexpr int kLdsLimbBudget = 96 * 1024;
constexpr int kPmax = 5;  // pairs per wave in the LDS kernel

GemvPlan plan_gemv(int64_t b, int64_t K, int64_t N) {
  const int64_t G = K / kGroup, GP = (G + 1) / 2;
  const int64_t Kp = K + kRowPad;
  const int nt = int((b + 3) / 4);
  GemvPlan p{};
  const int64_t limb_bytes = (2 * b * Kp + 1023) / 1024 * 1024;
  if (limb_bytes <= kLdsLimbBudget && GP <= 16 * kPmax) {
    p.lds = true;
    p.waves = int(GP < 10 ? GP : (GP + 1) / 2 < 16 ? (GP + 1) / 2 : 16);
    p.pmax = int((GP + p.waves - 1) / p.waves);
    p.rb = N >= 16 * 2 * 512 ? 2 : 1;
    p.lds_limb_bytes = int(limb_bytes);
    p.lds_bytes = size_t(limb_bytes) + size_t(p.waves - 1) * p.rb * nt * 64 * sizeof(float);
    static const char *names[2] = {"gemv_lds_rb1", "gemv_lds_rb2"};
    p.name = names[p.rb - 1];
    return p;
  }
  p.lds = false;
  p.rb = N >= 16 * 2 * 128 ? 2 : 1;
  const int cap = p.rb == 1 ? GemvWaveCap<1>::value : GemvWaveCap<2>::value;
  p.waves = int(GP < cap ? GP : cap);
  p.lds_bytes = size_t(p.waves > 1 ? p.waves - 1 : 1) * p.rb * nt * 64 * sizeof(float);
  static const char *names[2] = {"gemv_reg_rb1", "gemv_reg_rb2"};
  p.name = names[p.rb - 1];
  return p;
}

template <int RB, int NT, int PMAX>
void launch_lds_t(const GemvPlan &p, dim3 grid, const GemvWs &w, int64_t b, int64_t K, int64_t N,
                  const uint32_t *packed, const uint16_t *scales, void *y, int y_dtype,
                  hipStream_t stream) {
  hipLaunchKernelGGL((gemv_lds_kernel<RB, NT, PMAX>), grid, dim3(64 * p.waves), p.lds_bytes, stream,
                     w.xhi, w.sigma, int(b), K, w.Kp, N, packed, scales, y, y_dtype,
                     p.lds_limb_bytes);
}

template <int RB, int NT>
void launch_lds_rn(const GemvPlan &p, dim3 grid, const GemvWs &w, int64_t b, int64_t K, int64_t N,
                   const uint32_t *packed, const uint16_t *scales, void *y, int y_dtype,
                   hipStream_t stream) {
  switch (p.pmax) {
    case 1: launch_lds_t<RB, NT, 1>(p, grid, w, b, K, N, packed, scales, y, y_dtype, stream); break;
    case 2: launch_lds_t<RB, NT, 2>(p, grid, w, b, K, N, packed, scales, y, y_dtype, stream); break;
    case 3: launch_lds_t<RB, NT, 3>(p, grid, w, b, K, N, packed, scales, y, y_dtype, stream); break;
    case 4: launch_lds_t<RB, NT, 4>(p, grid, w, b, K, N, packed, scales, y, y_dtype, stream); break;
    default: launch_lds_t<RB, NT, 5>(p, grid, w, b, K, N, packed, scales, y, y_dtype, stream); break;
  }
}

template <int RB>
void launch_lds_r(const GemvPlan &p, dim3 grid, const GemvWs &w, int64_t b, int64_t K, int64_t N,
                  const uint32_t *packed, const uint16_t *scales, void *y, int y_dtype,
                  hipStream_t stream) {
  switch ((b + 3) / 4) {
    case 1: launch_lds_rn<RB, 1>(p, grid, w, b, K, N, packed, scales, y, y_dtype, stream); break;
    case 2: launch_lds_rn<RB, 2>(p, grid, w, b, K, N, packed, scales, y, y_dtype, stream); break;
    case 3: launch_lds_rn<RB, 3>(p, grid, w, b, K, N, packed, scales, y, y_dtype, stream); break;
    default: launch_lds_rn<RB, 4>(p, grid, w, b, K, N, packed, scales, y, y_dtype, stream); break;
  }
}

template <int RB>
void launch_reg_r(const GemvPlan &p, dim3 grid, const GemvWs &w, int64_t b, int64_t K, int64_t N,
                  const uint32_t *packed, const uint16_t *scales, void *y, int y_dtype,
                  hipStream_t stream) {
  const dim3 blk(64 * p.waves);
  switch ((b + 3) / 4) {
    case 1: hipLaunchKernelGGL((gemv_reg_kernel<RB, 1>), grid, blk, p.lds_bytes, stream, w.xhi, w.sigma, int(b), K, w.Kp, N, packed, scales, y, y_dtype); break;
    case 2: hipLaunchKernelGGL((gemv_reg_kernel<RB, 2>), grid, blk, p.lds_bytes, stream, w.xhi, w.sigma, int(b), K, w.Kp, N, packed, scales, y, y_dtype); break;
    case 3: hipLaunchKernelGGL((gemv_reg_kernel<RB, 3>), grid, blk, p.lds_bytes, stream, w.xhi, w.sigma, int(b), K, w.Kp, N, packed, scales, y, y_dtype); break;
    default: hipLaunchKernelGGL((gemv_reg_kernel<RB, 4>), grid, blk, p.lds_bytes, stream, w.xhi, w.sigma, int(b), K, w.Kp, N, packed, scales, y, y_dtype); break;
  }
}

}  // namespace

size_t gemv_workspace_bytes(int64_t b, int64_t K, int64_t /*N*/) {
  // two int8 limb planes [b, K + 16] and the per-token scales
  return align256(2 * size_t(b) * size_t(K + kRowPad)) + align256(16 * sizeof(float));
}

hipError_t launch_gemv_prepare(const float *xr, int64_t b, int64_t K, void *workspace,
                               hipStream_t stream) {
  const GemvWs w = carve(workspace, b, K);
  (void)hipGetLastError();  // drop errors left by earlier, unrelated runtime calls
  hipLaunchKernelGGL(gemv_prep_kernel, dim3(unsigned(b)), dim3(kPrepThreads), 0, stream, xr, K, w.Kp,
                     int(b), w.xhi, w.sigma);
  set_last_kernel("gemv_prep_limbs");
  return hipGetLastError();
}

hipError_t launch_gemv_main(const void *workspace, int64_t b, int64_t K, int64_t N,
                            const uint32_t *packed, const uint16_t *scales, void *y, int y_dtype,
                            hipStream_t stream) {
  const GemvWs w = carve(const_cast<void *>(workspace), b, K);
  const GemvPlan p = plan_gemv(b, K, N);
  const dim3 grid(unsigned((N + 16 * p.rb - 1) / (16 * p.rb)));
  (void)hipGetLastError();  // drop errors left by earlier, unrelated runtime calls
  if (p.lds) {
    if (p.rb == 2) launch_lds_r<2>(p, grid, w, b, K, N, packed, scales, y, y_dtype, stream);
    else launch_lds_r<1>(p, grid, w, b, K, N, packed, scales, y, y_dtype, stream);
  } else {
    if (p.rb == 2) launch_reg_r<2>(p, grid, w, b, K, N, packed, scales, y, y_dtype, stream);
    else launch_reg_r<1>(p, grid, w, b, K, N, packed, scales, y, y_dtype, stream);
  }
  set_last_kernel(p.name);
  return hipGetLastError();
}

}  // namespace tl
