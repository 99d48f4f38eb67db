// Prefill int8 GEMM with in-kernel weight expansion and rescale.
//
// Method: qiita.com/nakanokensetsu/items/ecc183fae033565af7cb, "4. 効いた高速化":
// W_int8[n,k] = code[n,k] * q[n, k/128] is exact in int8, the rotated activations
// are int8 per token, one int8 x int8 -> int32 GEMM covers the matmul, and a
// per-row (row_scale) and per-token (tok_scale) rescale follows.  The page
// expands the weights to int8 every step (31 of 83 ms in its 256-token step);
// here the 2-bit codes are expanded in registers as the tiles are consumed, so
// the int8 weight matrix never exists in memory.
//
// Tiling (CDNA4, v_mfma_i32_32x32x32_i8): a 256-thread workgroup computes a
// 128 x 256 tile of y; each of its 4 waves owns 128 x 64 (4 x 2 MFMA tiles,
// 128 int32 accumulators per lane).  The K loop steps one 128-wide scale group
// at a time (4 MFMA k-steps).  The activation tile (128 rows x 128 bytes) is
// staged in LDS, double buffered, and shared by the 4 waves.  Each wave loads
// its own weight columns straight from global memory: one 16-byte load per
// column per group gives the 4 words that feed the group's 4 k-steps.  The
// expansion code -> code*q is one v_perm_b32 per 4 weights: the selector bytes
// are the 2-bit fields ((w >> 2r) & 0x03030303) and the table holds
// {0, q, -, -q}.  The packed layout puts codes 4r..4r+3 in bytes 0..3 of that
// selector, in k order, so the weight fragment lines up with 16 consecutive
// activation bytes read from LDS.
#include "tl_device.h"

namespace tl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;
constexpr int kBN = 256;
constexpr int kThreads = 256;
constexpr int kAStride = kGroup + 16;  // LDS row pitch in bytes (padding spreads banks)

static_assert(kBM * kGroup == kThreads * 4 * 16, "A stage = 4 x 16 bytes per thread");
static_assert(kBN == 4 * 64, "4 waves x 64 columns");

__device__ __forceinline__ uint32_t perm_table(int qv) {
  // bytes: [0] = 0, [1] = q, [2] = unused, [3] = -q
  return ((uint32_t)(uint8_t)(int8_t)(-qv) << 24) | ((uint32_t)(uint8_t)(int8_t)qv << 8);
}

// 16 int8 weights code*q from one packed word, k order
__device__ __forceinline__ v4i expand_word(uint32_t w, uint32_t table) {
  v4i r;
  r[0] = (int)__builtin_amdgcn_perm(0u, table, w & 0x03030303u);
  r[1] = (int)__builtin_amdgcn_perm(0u, table, (w >> 2) & 0x03030303u);
  r[2] = (int)__builtin_amdgcn_perm(0u, table, (w >> 4) & 0x03030303u);
  r[3] = (int)__builtin_amdgcn_perm(0u, table, (w >> 6) & 0x03030303u);
  return r;
}

__global__ __launch_bounds__(kThreads) void gemm_i8_kernel(
    const int8_t *__restrict__ xq, const float *__restrict__ tok_scale, int64_t M, int64_t K,
    int64_t N, const uint32_t *__restrict__ packed, const int8_t *__restrict__ q,
    const float *__restrict__ row_scale, void *__restrict__ y, int y_dtype,
    int32_t *__restrict__ acc_out) {
  __shared__ __attribute__((aligned(16))) int8_t sA[2][kBM * kAStride];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int64_t m0 = int64_t(blockIdx.y) * kBM;
  const int64_t n0 = int64_t(blockIdx.x) * kBN;
  const int G = int(K / kGroup);

  // activation staging: chunk c = tid + 256 i -> row c/8, 16-byte column c%8
  const int8_t *asrc[4];
  bool arow_ok[4];
  int adst[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + kThreads * i;
    const int row = c >> 3, c16 = c & 7;
    arow_ok[i] = m0 + row < M;
    asrc[i] = xq + (arow_ok[i] ? (m0 + row) : 0) * K + 16 * c16;
    adst[i] = row * kAStride + 16 * c16;
  }
  // weight columns of this lane: one per 32-wide N tile
  const char *bsrc[2];
  const int8_t *qsrc[2];
  bool bcol_ok[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = n0 + 64 * wave + 32 * j + l32;
    bcol_ok[j] = n < N;
    const int64_t nn = bcol_ok[j] ? n : 0;
    bsrc[j] = reinterpret_cast<const char *>(packed) + nn * (K / 4) + 16 * h;
    qsrc[j] = q + nn * G;
  }

  v16i acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][j][r] = 0;

  uint4 areg[4];
  uint4 breg[2];
  int qreg[2];
  const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int i = 0; i < 4; ++i) areg[i] = arow_ok[i] ? *reinterpret_cast<const uint4 *>(asrc[i]) : z4;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    breg[j] = bcol_ok[j] ? *reinterpret_cast<const uint4 *>(bsrc[j]) : z4;
    qreg[j] = bcol_ok[j] ? (int)qsrc[j][0] : 0;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4 *>(&sA[0][adst[i]]) = areg[i];
  __syncthreads();

  for (int g = 0; g < G; ++g) {
    const int cur = g & 1;
    const bool more = g + 1 < G;
    // prefetch the next group (the last iteration re-reads the current one)
    const int gn = more ? g + 1 : g;
    uint4 anx[4], bnx[2];
    int qnx[2];
    {
      const int64_t koff = int64_t(gn) * kGroup;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        anx[i] = arow_ok[i] ? *reinterpret_cast<const uint4 *>(asrc[i] + koff) : z4;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bnx[j] = bcol_ok[j] ? *reinterpret_cast<const uint4 *>(bsrc[j] + 32 * int64_t(gn)) : z4;
        qnx[j] = bcol_ok[j] ? (int)qsrc[j][gn] : 0;
      }
    }

    const uint32_t tab0 = perm_table(qreg[0]), tab1 = perm_table(qreg[1]);
    const int8_t *abase = &sA[cur][l32 * kAStride + 64 * h];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint32_t w0 = s == 0 ? breg[0].x : s == 1 ? breg[0].y : s == 2 ? breg[0].z : breg[0].w;
      const uint32_t w1 = s == 0 ? breg[1].x : s == 1 ? breg[1].y : s == 2 ? breg[1].z : breg[1].w;
      const v4i bf0 = expand_word(w0, tab0);
      const v4i bf1 = expand_word(w1, tab1);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const v4i af = *reinterpret_cast<const v4i *>(abase + 32 * mt * kAStride + 16 * s);
        acc[mt][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, bf0, acc[mt][0], 0, 0, 0);
        acc[mt][1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, bf1, acc[mt][1], 0, 0, 0);
      }
    }

    if (more) {
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4 *>(&sA[cur ^ 1][adst[i]]) = anx[i];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        breg[j] = bnx[j];
        qreg[j] = qnx[j];
      }
    }
    __syncthreads();
  }

  // epilogue: lane holds column l32 of each 32x32 tile, rows 8*(r/4) + 4*h + r%4
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = n0 + 64 * wave + 32 * j + l32;
    if (n >= N) continue;
    const float rs = row_scale[n];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + 32 * mt + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m >= M) continue;
        const int a = acc[mt][j][r];
        const float v = ((float)a * rs) * tok_scale[m];
        if (acc_out) acc_out[m * N + n] = a;
        if (y_dtype == TL_F32)
          reinterpret_cast<float *>(y)[m * N + n] = v;
        else
          reinterpret_cast<uint16_t *>(y)[m * N + n] = float_to_bf16_bits(v);
      }
    }
  }
}

}  // namespace

size_t gemm_workspace_bytes(int64_t /*M*/, int64_t /*K*/, int64_t /*N*/) { return 0; }

hipError_t launch_gemm(const int8_t *xq, const float *tok_scale, int64_t M, int64_t K, int64_t N,
                       const uint32_t *packed, const int8_t *q, const float *row_scale, void *y,
                       int y_dtype, int32_t *acc_out, void * /*workspace*/, hipStream_t stream) {
  const int64_t gx = (N + kBN - 1) / kBN, gy = (M + kBM - 1) / kBM;
  if (gx > 0x7FFFFFFF || gy > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemm_i8_kernel, dim3(unsigned(gx), unsigned(gy)), dim3(kThreads), 0, stream,
                     xq, tok_scale, M, K, N, packed, q, row_scale, y, y_dtype, acc_out);
  set_last_kernel("gemm_i8_mfma32_128x256");
  return hipGetLastError();
}

}  // namespace tl
