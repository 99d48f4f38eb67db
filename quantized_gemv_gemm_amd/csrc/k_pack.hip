// Load-time packing of one ternary layer and its scale decomposition.
//
// Method: qiita.com/nakanokensetsu/items/ecc183fae033565af7cb, "前提" (2-bit codes
// in {-1,0,+1}, one fp16 scale per row and 128-group) and "4. 効いた高速化"
// (q[n,g] = round(127 s[n,g] / smax[n]) so that code * q is exact in int8).
//
// The packed word encoding (include/tl.h) puts code 4r + b in byte b, bit pair
// r, so packing 16 int8 codes is four masks and shifts:
// word = sum_r ((c_r & 0x03030303) << 2r), where c_r is the 32-bit word holding
// codes 4r..4r+3.  Fields are the codes' two's-complement low bits.  Words go to
// the wavefront-shaped 1 KB tiles of the layout.
// The scale decomposition takes the row maximum of |s|, then
// q = RNE(fl32(fl32(127 s) / smax)): the quotient is formed in binary64 and
// rounded to binary32 once, which equals the correctly rounded binary32 division
// because binary64 carries more than 2*24+2 bits.
#include "tl_device.h"

namespace tl {
namespace {

constexpr int kThreads = 256;

// number of bytes of w that are not 0x00, 0x01 or 0xFF
__device__ __forceinline__ int bad_bytes(uint32_t w) {
  int n = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t v = ((w >> (8 * i)) + 1u) & 0xFFu;  // 0x00->1, 0x01->2, 0xFF->0
    n += v > 2u;
  }
  return n;
}

// One workgroup per 1024-byte tile (rb, p): thread t builds word t of the tile,
// which holds the 16 codes k = 128*(2p + gi) + 16*(2*(l/16) + m) + j of row
// 16*rb + l%16, with l = t/4, gi = (t/2)%2, m = t%2.  Codes past N or K are the
// zero padding of the layout.  Writes are one contiguous kilobyte per tile.
__global__ __launch_bounds__(kThreads) void pack_tiles_kernel(const int8_t *__restrict__ codes,
                                                              int64_t N, int64_t K, int GP,
                                                              uint32_t *__restrict__ packed,
                                                              int32_t *__restrict__ invalid_count) {
  const int64_t tile = blockIdx.x;
  const int64_t rb = tile / GP;
  const int p = int(tile - rb * GP);
  const int t = threadIdx.x;
  const int l = t >> 2, gi = (t >> 1) & 1, m = t & 1;
  const int64_t n = rb * 16 + (l & 15);
  const int64_t k0 = 128 * (2 * int64_t(p) + gi) + 16 * (2 * (l >> 4) + m);
  uint32_t word = 0;
  int bad = 0;
  if (n < N && k0 < K) {
    const uint4 c = *reinterpret_cast<const uint4 *>(codes + n * K + k0);
    word = (c.x & 0x03030303u) | ((c.y & 0x03030303u) << 2) | ((c.z & 0x03030303u) << 4) |
           ((c.w & 0x03030303u) << 6);
    if (invalid_count) bad = bad_bytes(c.x) + bad_bytes(c.y) + bad_bytes(c.z) + bad_bytes(c.w);
  }
  packed[tile * 256 + t] = word;
  if (bad) atomicAdd(invalid_count, bad);
}

// One workgroup per row: smax = max_g |s|, q = RNE(fl32(127 s) / smax), row_scale.
__global__ __launch_bounds__(kThreads) void scale_rows_kernel(const uint16_t *__restrict__ scales,
                                                              int G, int8_t *__restrict__ q,
                                                              float *__restrict__ row_scale) {
  __shared__ float red[kThreads / 64];
  const int64_t n = blockIdx.x;
  const uint16_t *srow = scales + n * G;
  float mx = 0.0f;
  for (int g = threadIdx.x; g < G; g += kThreads) mx = fmaxf(mx, half_bits_to_float(srow[g] & 0x7FFFu));
  const float smax = block_max<kThreads>(mx, red);
  int8_t *qrow = q + n * G;
  for (int g = threadIdx.x; g < G; g += kThreads) {
    int8_t qv = 0;
    if (smax > 0.0f) {
      const float num = 127.0f * half_bits_to_float(srow[g]);  // exact in binary32
      const float quo = (float)((double)num / (double)smax);
      qv = (int8_t)(int)rintf(quo);
    }
    qrow[g] = qv;
  }
  if (threadIdx.x == 0) row_scale[n] = (float)((double)smax / 127.0);
}

}  // namespace

int64_t packed_words(int64_t N, int64_t K) { return ((N + 15) / 16) * ((K + 255) / 256) * 256; }

hipError_t launch_pack(const int8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                       uint32_t *packed, int8_t *q, float *row_scale, int32_t *invalid_count,
                       hipStream_t stream) {
  const int64_t NB = (N + 15) / 16, GP = (K + 255) / 256;
  if (NB * GP > 0x7FFFFFFF || N > 0x7FFFFFFF) return hipErrorInvalidValue;
  (void)hipGetLastError();  // drop errors left by earlier, unrelated runtime calls
  hipLaunchKernelGGL(pack_tiles_kernel, dim3(unsigned(NB * GP)), dim3(kThreads), 0, stream, codes, N,
                     K, int(GP), packed, invalid_count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scale_rows_kernel, dim3(unsigned(N)), dim3(kThreads), 0, stream, scales,
                     int(K / kGroup), q, row_scale);
  set_last_kernel("pack_tiles+scale_rows");
  return hipGetLastError();
}

}  // namespace tl
