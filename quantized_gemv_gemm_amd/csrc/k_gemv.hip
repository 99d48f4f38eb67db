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
// Work split: a workgroup owns 16*RB consecutive rows and all of K; its W waves
// split the K groups and reduce through LDS.  Rows past N and token slots past
// b are masked at load time (no memory traffic for them).
#include "tl_device.h"

namespace tl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr float kLimbRange = 32639.0f;  // 127 * 257: hi, lo of 256*hi + lo stay in int8

// --------------------------------------------------------------------------
// prep: xr f32 [b, K] -> limbs hi, lo int8 [b, K] and sigma[b] = amax / 32639
// --------------------------------------------------------------------------
constexpr int kPrepThreads = 256;

__global__ __launch_bounds__(kPrepThreads) void gemv_prep_kernel(const float *__restrict__ xr,
                                                                 int64_t K,
                                                                 int8_t *__restrict__ xhi,
                                                                 int8_t *__restrict__ xlo,
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
    *reinterpret_cast<uint4 *>(xhi + t * K + i) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    *reinterpret_cast<uint4 *>(xlo + t * K + i) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
  }
}

// --------------------------------------------------------------------------
// main kernel
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

template <int RB>
struct GemvSlot {
  v4i ah[2], al[2];  // activation limbs of the group's two 64-k halves
  uint2 w[RB];       // packed words 2q, 2q+1 of the group, per row block
  uint32_t s[RB];    // fp16 scale bits
};

// Loads are unconditional: lanes whose token slot or row is out of range read a
// valid clamped address instead, and their results are never stored.  Keeping
// the loop free of divergent branches lets the compiler count outstanding loads
// exactly, so four groups stay in flight.
template <int RB>
__device__ __forceinline__ void gemv_load(GemvSlot<RB> &f, int g, const int8_t *ah,
                                          const int8_t *al, const char *const (&wrow)[RB],
                                          const uint16_t *const (&srow)[RB]) {
  const v4i *ph = reinterpret_cast<const v4i *>(ah + 128 * int64_t(g));
  const v4i *pl = reinterpret_cast<const v4i *>(al + 128 * int64_t(g));
  f.ah[0] = ph[0];
  f.ah[1] = ph[1];
  f.al[0] = pl[0];
  f.al[1] = pl[1];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    f.w[rb] = *reinterpret_cast<const uint2 *>(wrow[rb] + 32 * int64_t(g));
    f.s[rb] = srow[rb][g];
  }
}

template <int RB, int NT>
__device__ __forceinline__ void gemv_compute(const GemvSlot<RB> &f, bool live, float (&acc)[RB][4]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const v4i z = {0, 0, 0, 0};
    const v4i b0 = unpack_x64(f.w[rb].x);
    const v4i b1 = unpack_x64(f.w[rb].y);
    v4i dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.ah[0], b0, z, 0, 0, 0);
    v4i dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.al[0], b0, z, 0, 0, 0);
    dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.ah[1], b1, dh, 0, 0, 0);
    dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(f.al[1], b1, dl, 0, 0, 0);
    const float s = live ? half_bits_to_float((uint16_t)f.s[rb]) : 0.0f;
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[rb][i] = fmaf(s, (float)(dh[i] * 256 + dl[i]), acc[rb][i]);
  }
}

// wave cap per workgroup: larger row tiles need more registers per wave
template <int RB>
struct GemvWaveCap {
  static constexpr int value = RB == 1 ? 16 : RB == 2 ? 12 : 8;
};

// One workgroup: 16*RB rows, all of K.  Its waves (blockDim.x / 64 of them) take
// contiguous runs of 4-group chunks (one 128-byte line per row), keep the four
// groups of a chunk in flight while the previous chunk is consumed, and reduce
// through LDS at the end.  NT = ceil(b / 4).
template <int RB, int NT>
__global__ __launch_bounds__(64 * GemvWaveCap<RB>::value) void gemv_i8x2_kernel(
    const int8_t *__restrict__ xhi, const int8_t *__restrict__ xlo,
    const float *__restrict__ sigma, int b, int64_t K, int64_t N,
    const uint32_t *__restrict__ packed, const uint16_t *__restrict__ scales, void *__restrict__ y,
    int y_dtype) {
  extern __shared__ float red[];  // (W - 1) * RB * NT * 64 floats
  const int W = blockDim.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;  // B/D column = weight row in the block; A row = token slot
  const int qd = lane >> 4;   // lane quarter: k quarter for A/B, token for D
  const int G = int(K / kGroup);
  const int nchunk = (G + 3) >> 2;
  const int c_begin = (nchunk * wave) / W;
  const int c_end = (nchunk * (wave + 1)) / W;
  const int64_t n0 = int64_t(blockIdx.x) * (16 * RB);

  const int tok = token_of_arow(col);
  const int tok_ld = tok < b ? tok : b - 1;
  const int8_t *ah = xhi + int64_t(tok_ld) * K + 32 * qd;
  const int8_t *al = xlo + int64_t(tok_ld) * K + 32 * qd;
  const char *wrow[RB];
  const uint16_t *srow[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int64_t n = n0 + 16 * rb + col;
    const int64_t nn = n < N ? n : N - 1;
    wrow[rb] = reinterpret_cast<const char *>(packed) + nn * (K / 4) + 8 * qd;
    srow[rb] = scales + nn * G;
  }

  float acc[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[rb][i] = 0.0f;

  if (c_begin < c_end) {
    // slot j holds group 4c + j of the chunk c in flight; groups past G (only in a
    // last, partial chunk) re-read group G-1 and are given scale 0
    GemvSlot<RB> sl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) gemv_load<RB>(sl[j], min(4 * c_begin + j, G - 1), ah, al, wrow, srow);
    for (int c = c_begin; c < c_end - 1; ++c) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        gemv_compute<RB, NT>(sl[j], true, acc);
        gemv_load<RB>(sl[j], min(4 * (c + 1) + j, G - 1), ah, al, wrow, srow);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) gemv_compute<RB, NT>(sl[j], 4 * (c_end - 1) + j < G, acc);
  }

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

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

template <int RB, int NT>
hipError_t launch_main_rb_nt(const int8_t *xhi, const int8_t *xlo, const float *sigma, int64_t b,
                             int64_t K, int64_t N, const uint32_t *packed, const uint16_t *scales,
                             void *y, int y_dtype, int waves, hipStream_t stream) {
  const int64_t grid = (N + 16 * RB - 1) / (16 * RB);
  const size_t lds = size_t(waves > 1 ? waves - 1 : 1) * RB * NT * 64 * sizeof(float);
  hipLaunchKernelGGL((gemv_i8x2_kernel<RB, NT>), dim3(unsigned(grid)), dim3(64 * waves), lds,
                     stream, xhi, xlo, sigma, int(b), K, N, packed, scales, y, y_dtype);
  return hipGetLastError();
}

template <int RB>
hipError_t launch_main_rb(const int8_t *xhi, const int8_t *xlo, const float *sigma, int64_t b,
                          int64_t K, int64_t N, const uint32_t *packed, const uint16_t *scales,
                          void *y, int y_dtype, int waves, hipStream_t stream) {
  switch ((b + 3) / 4) {
    case 1: return launch_main_rb_nt<RB, 1>(xhi, xlo, sigma, b, K, N, packed, scales, y, y_dtype, waves, stream);
    case 2: return launch_main_rb_nt<RB, 2>(xhi, xlo, sigma, b, K, N, packed, scales, y, y_dtype, waves, stream);
    case 3: return launch_main_rb_nt<RB, 3>(xhi, xlo, sigma, b, K, N, packed, scales, y, y_dtype, waves, stream);
    default: return launch_main_rb_nt<RB, 4>(xhi, xlo, sigma, b, K, N, packed, scales, y, y_dtype, waves, stream);
  }
}

struct GemvVariant {
  int rb, waves;
  const char *name;
};

// Rows per workgroup (16*rb) and waves per workgroup for a problem size.  Each
// wave should own at least one 4-group chunk; row blocks per workgroup trade
// CU coverage (more, smaller workgroups) against activation re-reads (each
// workgroup reads all of the b x K activations).
GemvVariant choose_gemv(int64_t b, int64_t K, int64_t N) {
  const int64_t G = K / kGroup, nchunk = (G + 3) / 4;
  int rb = 1;
  if (b > 4 && N >= 64 * 256) rb = 4;
  else if (b > 4 && N >= 32 * 256) rb = 2;
  const int cap = rb == 1 ? GemvWaveCap<1>::value : rb == 2 ? GemvWaveCap<2>::value : GemvWaveCap<4>::value;
  const int waves = int(nchunk < cap ? nchunk : cap);
  static const char *names[3] = {"gemv_i8x2_rb1", "gemv_i8x2_rb2", "gemv_i8x2_rb4"};
  return {rb, waves, names[rb == 1 ? 0 : rb == 2 ? 1 : 2]};
}

}  // namespace

size_t gemv_workspace_bytes(int64_t b, int64_t K, int64_t /*N*/) {
  // two int8 limb planes [b, K] and the per-token scales
  return 2 * align256(size_t(b) * size_t(K)) + align256(16 * sizeof(float));
}

namespace {
struct GemvWs {
  int8_t *xhi, *xlo;
  float *sigma;
};
GemvWs carve(void *workspace, int64_t b, int64_t K) {
  char *ws = static_cast<char *>(workspace);
  const size_t plane = align256(size_t(b) * size_t(K));
  return {reinterpret_cast<int8_t *>(ws), reinterpret_cast<int8_t *>(ws + plane),
          reinterpret_cast<float *>(ws + 2 * plane)};
}
}  // namespace

hipError_t launch_gemv_prepare(const float *xr, int64_t b, int64_t K, void *workspace,
                               hipStream_t stream) {
  const GemvWs w = carve(workspace, b, K);
  (void)hipGetLastError();  // drop errors left by earlier, unrelated runtime calls
  hipLaunchKernelGGL(gemv_prep_kernel, dim3(unsigned(b)), dim3(kPrepThreads), 0, stream, xr, K,
                     w.xhi, w.xlo, w.sigma);
  set_last_kernel("gemv_prep_limbs");
  return hipGetLastError();
}

hipError_t launch_gemv_main(const void *workspace, int64_t b, int64_t K, int64_t N,
                            const uint32_t *packed, const uint16_t *scales, void *y, int y_dtype,
                            hipStream_t stream) {
  const GemvWs w = carve(const_cast<void *>(workspace), b, K);
  const GemvVariant v = choose_gemv(b, K, N);
  (void)hipGetLastError();  // drop errors left by earlier, unrelated runtime calls
  hipError_t e;
  if (v.rb == 4)
    e = launch_main_rb<4>(w.xhi, w.xlo, w.sigma, b, K, N, packed, scales, y, y_dtype, v.waves, stream);
  else if (v.rb == 2)
    e = launch_main_rb<2>(w.xhi, w.xlo, w.sigma, b, K, N, packed, scales, y, y_dtype, v.waves, stream);
  else
    e = launch_main_rb<1>(w.xhi, w.xlo, w.sigma, b, K, N, packed, scales, y, y_dtype, v.waves, stream);
  set_last_kernel(v.name);
  return e;
}

}  // namespace tl
