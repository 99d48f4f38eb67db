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
#include <algorithm>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "rotate_dev.h"
#include "tl_device.h"

namespace tl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kRowPad = kLimbRowPad;
constexpr int kSigLds = 1024;  // stream kernels' LDS for a chunk's limb scales (16 tokens x 16 blocks)
// LDS of the ring kernel for one chunk's limb scales: 16 tokens x the blocks of K
__host__ __device__ constexpr int ring_sig_bytes(int64_t K) {
  return int((16 * ((K + 1023) / 1024) * 4 + 255) / 256 * 256);
}    // bytes after each limb row: spreads LDS banks

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// workspace: the limb region (limb_region_bytes: rows for b <= 8, operand order
// for b > 8), then sigma[b][limb_blocks(K)]
struct GemvWs {
  int8_t *xhi;
  float *sigma;
  int64_t Kp;
};
GemvWs carve(void *workspace, int64_t b, int64_t K) {
  char *ws = static_cast<char *>(workspace);
  const int64_t Kp = K + kRowPad;
  return {reinterpret_cast<int8_t *>(ws), reinterpret_cast<float *>(ws + align256(size_t(limb_region_bytes(b, K)))),
          Kp};
}

// --------------------------------------------------------------------------
// prep: xr f32 [b, K] -> limbs and sigma[t][j] = |x|max / 32639 of each 1024-block,
// one wavefront per (token, block): no step waits for another block
// --------------------------------------------------------------------------
__global__ __launch_bounds__(64) void gemv_prep_kernel(const float *__restrict__ xr, int64_t K, int64_t Kp,
                                                       int b, int8_t *__restrict__ xhi,
                                                       float *__restrict__ sigma) {
  const int nbk = limb_blocks(K);
  const int t = int(blockIdx.x / unsigned(nbk)), blk = int(blockIdx.x - unsigned(t * nbk));
  const int lane = threadIdx.x;
  const int64_t k0 = int64_t(blk) * kHBlock;
  const int len = int(K - k0 < kHBlock ? K - k0 : kHBlock);
  const float *row = xr + int64_t(t) * K + k0;
  float v[16];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int e = 256 * s + 4 * lane;
    const float4 f = e < len ? *reinterpret_cast<const float4 *>(row + e) : make_float4(0.f, 0.f, 0.f, 0.f);
    v[4 * s] = f.x;
    v[4 * s + 1] = f.y;
    v[4 * s + 2] = f.z;
    v[4 * s + 3] = f.w;
  }
  store_block_limbs(v, lane, t, b, K, Kp, k0, len, xhi, sigma + int64_t(t) * nbk + blk);
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

// Paired-limb mode (LP, for b <= 8): A row r holds limb r%2 (0 = hi, 1 = lo) of
// token 2*(r/4) + (r/2)%2, so a single MFMA chain yields both limb sums of a token
// in one lane -- D rows 4q, 4q+1 are hi, lo of token 2q and 4q+2, 4q+3 those of
// token 2q+1 -- which halves the MFMAs and activation reads of the two-limb form.
__device__ __forceinline__ int lp_token(int r) { return 2 * (r >> 2) + ((r >> 1) & 1); }

// More than 16 tokens: grid row blockIdx.y takes token chunk c = 16 c .. 16 c + 15
// (operand-order limbs at 32 K c, sigma and y rows from 16 c); b becomes the
// chunk's token count.
template <class PL, class PS, class PY>  // the kernels' (restrict-qualified) parameter types
__device__ __forceinline__ void select_chunk(PL &limbs, PS &sigma, PY &y, int &b, int64_t K, int64_t N,
                                             int y_dtype) {
  const int c = blockIdx.y;
  if (c == 0) return;
  limbs += 32 * K * c;
  sigma += int64_t(kTokChunk) * c * limb_blocks(K);
  y = static_cast<char *>(y) + int64_t(kTokChunk) * c * N * (y_dtype == TL_F32 ? 4 : 2);
  b = min(kTokChunk, b - kTokChunk * c);
}

// both groups of a pair: tile words .x/.y feed group 2p, .z/.w group 2p+1.  With
// paired limbs each group is a single chain, so the two groups' chains are issued
// interleaved (first halves, then second halves): one chain's matrix instruction
// runs while the other's result is pending.
template <int RB, int NT, bool LP>
__device__ __forceinline__ void pair_mfma(const v4i (&ah)[2][2], const v4i (&al)[2][2],
                                          const uint4 (&w)[RB], const float (&s)[2][RB],
                                          float (&acc)[RB][4]) {
  const v4i z = {0, 0, 0, 0};
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const v4i a0 = unpack_x64(w[rb].x), a1 = unpack_x64(w[rb].y);  // group 2p
    const v4i b0 = unpack_x64(w[rb].z), b1 = unpack_x64(w[rb].w);  // group 2p + 1
    if (LP) {  // one chain per group: interleaved
      v4i d0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah[0][0], a0, z, 0, 0, 0);
      v4i d1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah[1][0], b0, z, 0, 0, 0);
      d0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah[0][1], a1, d0, 0, 0, 0);
      d1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah[1][1], b1, d1, 0, 0, 0);
      acc[rb][0] = fmaf(s[0][rb], (float)(d0[0] * 256 + d0[1]), acc[rb][0]);
      acc[rb][1] = fmaf(s[0][rb], (float)(d0[2] * 256 + d0[3]), acc[rb][1]);
      acc[rb][0] = fmaf(s[1][rb], (float)(d1[0] * 256 + d1[1]), acc[rb][0]);
      acc[rb][1] = fmaf(s[1][rb], (float)(d1[2] * 256 + d1[3]), acc[rb][1]);
      continue;
    }
    // two limbs: each group already has two independent chains (hi, lo)
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const v4i c0 = gi ? b0 : a0, c1 = gi ? b1 : a1;
      v4i dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah[gi][0], c0, z, 0, 0, 0);
      v4i dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(al[gi][0], c0, z, 0, 0, 0);
      dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah[gi][1], c1, dh, 0, 0, 0);
      dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(al[gi][1], c1, dl, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < NT; ++i) acc[rb][i] = fmaf(s[gi][rb], (float)(dh[i] * 256 + dl[i]), acc[rb][i]);
    }
  }
}

// the lane's 16 bytes of tile (row block rbg, pair p): one coalesced kilobyte per wave
__device__ __forceinline__ uint4 load_tile(const uint32_t *__restrict__ packed, int64_t rbg, int GP,
                                           int p, int lane) {
  return *reinterpret_cast<const uint4 *>(packed + 256 * (rbg * GP + p) + 4 * lane);
}

// The fp16 scales of the workgroup's 16*RB rows are one contiguous run of the
// row-major [N, G] array: it is copied into LDS with 1 KB direct loads (chunk c
// by wave c mod W) in the same memory round as the weights, instead of two scattered
// 2-byte loads per lane and pair.  Pieces past the end of the array read a
// clamped, valid address; those LDS bytes lie beyond the run and are never read.
__device__ __forceinline__ void stage_scales(const uint16_t *__restrict__ scales, int64_t N, int G,
                                             int64_t n0, int rows, char *ls, int wave, int W,
                                             int lane) {
  if (n0 + rows > N) {
    // the last workgroup holds fewer rows: its run may end inside a 16-byte piece
    const int64_t valid = (N - n0) * G;
    for (int64_t e = 64 * wave + lane; e < valid; e += 64 * W)
      reinterpret_cast<uint16_t *>(ls)[e] = scales[n0 * G + e];
    return;
  }
  // a whole run ends on a 32-byte boundary: every piece it needs lies inside the array
  const int64_t begin = n0 * G * 2, total = N * G * 2;
  const int chunks = (rows * G * 2 + 1023) / 1024;
  for (int c = wave; c < chunks; c += W) {
    const int64_t off = begin + int64_t(c) * 1024 + 16 * lane;
    const int64_t src = off + 16 <= total ? off : 0;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const char *>(scales) + src,
                                     (__attribute__((address_space(3))) void *)(ls + c * 1024), 16, 0,
                                     0);
  }
}

// group scales of local row r for groups 2p and 2p+1 (0 past the last group), from LDS
__device__ __forceinline__ void pair_scales_lds(const char *ls, int r, int G, int p, float &s0,
                                                float &s1) {
  const uint16_t *row = reinterpret_cast<const uint16_t *>(ls) + r * G;
  s0 = half_bits_to_float(row[2 * p]);
  s1 = 2 * p + 1 < G ? half_bits_to_float(row[2 * p + 1]) : 0.0f;
}

// s_waitcnt immediate (gfx9 encoding): vmcnt(n), lgkmcnt(0), expcnt left free
template <int n>
constexpr int waitcnt_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  return (n & 15) | ((n >> 4) << 14) | (7 << 4);
}

// LDS reads the compiler does not track; lds_wait() waits for them and ties the
// values to that wait, so nothing uses them earlier
__device__ __forceinline__ v4i lds_read16(const int8_t *p) {
  v4i r;
  asm volatile("ds_read_b128 %0, %1"
               : "=v"(r)
               : "v"((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) int8_t *)p));
  return r;
}
__device__ __forceinline__ uint32_t lds_read_u16(const char *p) {
  uint32_t r;
  asm volatile("ds_read_u16 %0, %1"
               : "=v"(r)
               : "v"((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p));
  return r;
}
template <int RB>
__device__ __forceinline__ void lds_wait(v4i (&ah)[2][2], v4i (&al)[2][2], uint32_t (&sb)[2][RB],
                                         bool lp) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(ah[0][0]), "+v"(ah[0][1]), "+v"(ah[1][0]), "+v"(ah[1][1]));
  if (!lp) asm volatile("" : "+v"(al[0][0]), "+v"(al[0][1]), "+v"(al[1][0]), "+v"(al[1][1]));
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) asm volatile("" : "+v"(sb[0][rb]), "+v"(sb[1][rb]));
}

// as lds_wait, leaving the last N LDS reads (those of the next pair) in flight
template <int N, int RB>
__device__ __forceinline__ void lds_wait_n(v4i (&ah)[2][2], v4i (&al)[2][2], uint32_t (&sb)[2][RB], bool lp) {
  asm volatile("s_waitcnt lgkmcnt(%4)"
               : "+v"(ah[0][0]), "+v"(ah[0][1]), "+v"(ah[1][0]), "+v"(ah[1][1])
               : "n"(N));
  if (!lp) asm volatile("" : "+v"(al[0][0]), "+v"(al[0][1]), "+v"(al[1][0]), "+v"(al[1][1]));
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) asm volatile("" : "+v"(sb[0][rb]), "+v"(sb[1][rb]));
}

// the LDS operands of one pair: A fragments (limbs staged in LDS) and the two
// groups' scales of the RB row blocks
template <int RB, bool LP, bool ALDS>
__device__ __forceinline__ void pair_lds_issue(int p, int G, const int8_t *lah, const int8_t *lal, const char *ls,
                                               int col, v4i (&ah)[2][2], v4i (&al)[2][2], uint32_t (&sb)[2][RB]) {
  constexpr int kGS = LP ? 128 : 4096, kHS = LP ? 16 : 2048;  // group and half strides
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const int gl = min(2 * p + gi, G - 1);
    if (ALDS) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        ah[gi][h] = lds_read16(lah + kGS * gl + kHS * h);
        if (!LP) al[gi][h] = lds_read16(lal + kGS * gl + kHS * h);
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) sb[gi][rb] = lds_read_u16(ls + 2 * ((16 * rb + col) * G + gl));
  }
}

__host__ __device__ constexpr int scale_lds_bytes(int rows, int G) {
  return (rows * G * 2 + 1023) / 1024 * 1024;
}

// base[t * stride] for the token t of each accumulator of the lane (token b - 1
// past b: those accumulators are never stored).  base and stride are the same for
// the whole wave, so the addresses are a scalar base plus a 32-bit lane offset.
// The values are used as loaded, with nothing computed from them here, so that
// no instruction right after the loads has to wait for them.
template <int NT, bool LP>
__device__ __forceinline__ void token_scales(const float *__restrict__ base, int stride, int b, int lane,
                                             float (&u)[4]) {
  const int qd = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = LP ? 2 * qd + i : 4 * i + qd;
    u[i] = i < NT ? base[(t < b ? t : b - 1) * stride] : 0.0f;
  }
}

// The sums of accumulator i, so far in units of limb scale ua, move to units ub
// (the limb scale of the block that starts): acc *= ua / ub, with the hardware
// reciprocal (within an ulp or so: far inside the layer's error).  A block of
// zeros (ub = 0) adds nothing and keeps the units; ua = 0 means nothing has been
// added yet.  ua becomes the new units.
template <int RB>
__device__ __forceinline__ void change_unit(float (&acc)[RB][4], int i, float &ua, float ub) {
  const float r = ub > 0.0f ? ua * __builtin_amdgcn_rcpf(ub) : 1.0f;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) acc[rb][i] *= r;
  ua = ub > 0.0f ? ub : ua;
}
template <int RB, int NT>
__device__ __forceinline__ void change_units(float (&acc)[RB][4], float (&ua)[4], const float (&ub)[4]) {
#pragma unroll
  for (int i = 0; i < NT; ++i) change_unit<RB>(acc, i, ua[i], ub[i]);
}

// output element of accumulator (rb, i) of the lane: token 2 qd + i (LP) or 4 i + qd, row 16 rb + col
template <bool LP>
__device__ __forceinline__ void store_out(float v, int rb, int i, int lane, int b, int64_t n0, int64_t N,
                                          void *y, int y_dtype) {
  const int col = lane & 15, qd = lane >> 4;
  const int t = LP ? 2 * qd + i : 4 * i + qd;
  const int64_t n = n0 + 16 * rb + col;
  if (t >= b || n >= N) return;
  if (y_dtype == TL_F32)
    reinterpret_cast<float *>(y)[int64_t(t) * N + n] = v;
  else
    reinterpret_cast<uint16_t *>(y)[int64_t(t) * N + n] = float_to_bf16_bits(v);
}

// Each wave's partial sums times its own token scales tsc (the limb or token
// scale and the 1/64 of the unpacked codes) go to LDS (W x RB x NT x 64 floats);
// then accumulator c = rb NT + i of every lane is added over the waves, in wave
// order, and stored by wave c mod W, so that the adds and stores are spread over
// the waves instead of falling on one.
template <int RB, int NT, bool LP>
__device__ __forceinline__ void reduce_and_store(float (&acc)[RB][4], float *red, int W, int wave,
                                                 int lane, int b, int64_t n0, int64_t N,
                                                 const float (&tsc)[4], void *y, int y_dtype) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[rb][i] *= tsc[i];
  if (W == 1) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < NT; ++i) store_out<LP>(acc[rb][i], rb, i, lane, b, n0, N, y, y_dtype);
    return;
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < NT; ++i) red[((wave * RB + rb) * NT + i) * 64 + lane] = acc[rb][i];
  __syncthreads();
  for (int c = wave; c < RB * NT; c += W) {
    const int rb = c / NT, i = c - rb * NT;
    float v = red[(rb * NT + i) * 64 + lane];
    for (int w = 1; w < W; ++w) v += red[((w * RB + rb) * NT + i) * 64 + lane];
    store_out<LP>(v, rb, i, lane, b, n0, N, y, y_dtype);
  }
}

// --------------------------------------------------------------------------
// phase timestamps of gemv_stream (instrumented builds only: TL_PHASE_STAMPS=1)
// --------------------------------------------------------------------------
// Each wave keeps the constant-rate clock (100 MHz) at its phase boundaries in
// registers -- entry, every load issued, direct loads waited for, barrier
// passed, first pair computed, last pair computed -- and stores them, with its
// hardware id, before the cross-wave reduction; wave 0 adds the time its
// outputs were stored.  Record w = (blockIdx.y * gridDim.x + blockIdx.x) * 16 +
// wave, eight 64-bit words.  No store happens before the reduction, so the
// kernel's own memory waits are unchanged.  Off in the product build, where the
// calls are empty.
#ifndef TL_PHASE_STAMPS
#define TL_PHASE_STAMPS 0
#endif
#if TL_PHASE_STAMPS
__device__ unsigned long long *g_phase_stamps;
struct PhaseStamps {
  unsigned long long t[6];
  __device__ __forceinline__ void mark(int k) { t[k] = wall_clock64(); }
  __device__ __forceinline__ unsigned long long *record() const {
    unsigned long long *base = g_phase_stamps;
    return base ? base + ((int64_t(blockIdx.y) * gridDim.x + blockIdx.x) * 16 + (threadIdx.x >> 6)) * 8 : nullptr;
  }
  __device__ __forceinline__ void flush() const {
    unsigned long long *r = record();
    if (!r || (threadIdx.x & 63) != 0) return;
    unsigned hw, xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
#pragma unroll
    for (int k = 0; k < 6; ++k) r[k] = t[k];
    r[7] = (unsigned long long)hw | ((unsigned long long)xcc << 32);
  }
  __device__ __forceinline__ void done() const {
    unsigned long long *r = record();
    if (r && (threadIdx.x & 63) == 0) r[6] = wall_clock64();
  }
};
#else
struct PhaseStamps {
  __device__ __forceinline__ void mark(int) {}
  __device__ __forceinline__ void flush() const {}
  __device__ __forceinline__ void done() const {}
};
#endif

// --------------------------------------------------------------------------
// gemv_stream: every load of the wave issued at once, pairs consumed as they land
// --------------------------------------------------------------------------
// ALDS: the limbs of all b tokens are staged in LDS (one copy per workgroup);
// otherwise each wave loads its A fragments from L2 into registers with its tiles.
// Issue order per wave: direct loads into LDS (scale block, limbs), then for each
// of the PMAX pairs its A fragments (if not ALDS) and its RB tiles.  The fences
// keep that order, the wave waits only for the direct loads before the barrier,
// and the compiler then waits for each pair's own loads right before its MFMAs,
// so a pair is computed while later pairs are still arriving.  A wave with fewer
// than PMAX pairs repeats its last pair with scale 0 (no branch around loads).
// Variants that hold many tiles (and A fragments) in registers get 512-thread
// workgroups, hence up to 256 VGPRs, instead of 1024 threads and 128 VGPRs.
constexpr bool stream_heavy(bool alds, int rb, int pmax, bool lp) {
  // two-limb register variants with up to two pairs of up to three row blocks fit
  // 128 VGPRs (119 at three row blocks): 1024-thread workgroups, so ten waves
  // can split K = 5120 (b = 16 qkv 9.9 -> 9.2 us, gate_up 27.0 -> 21.4 us)
  if (alds) return pmax * rb > 10;
  if (lp) return pmax * (rb + 4) > 16;
  return pmax * (rb + 8) > (rb <= 3 ? 24 : 16);
}
constexpr int stream_threads(bool alds, int rb, int pmax, bool lp) {
  return stream_heavy(alds, rb, pmax, lp) ? 512 : 1024;
}

template <int RB, int NT, int PMAX, bool LP, bool ALDS>
__global__ __launch_bounds__(stream_threads(ALDS, RB, PMAX, LP)) void gemv_stream_kernel(
    const int8_t *__restrict__ limbs, const float *__restrict__ sigma, int b, int64_t K,
    int64_t Kp, int64_t N, const uint32_t *__restrict__ packed, const uint16_t *__restrict__ scales,
    void *__restrict__ y, int y_dtype, int lds_limb_bytes, uint32_t wmagic) {
  constexpr int NA = LP ? 4 : 8;  // A fragment loads per pair when not ALDS
  extern __shared__ __attribute__((aligned(16))) char smem[];
  static_assert(PMAX <= 5, "a wave's pairs span at most two 1024-blocks");
  PhaseStamps ps;
  ps.mark(0);
  select_chunk(limbs, sigma, y, b, K, N, y_dtype);
  const int64_t region = LP ? limb_region_bytes(b, K) : 32 * K;  // this chunk's limbs
  int8_t *lx = reinterpret_cast<int8_t *>(smem);
  char *ls = smem + (ALDS ? lds_limb_bytes : 0);
  const int G = int(K / kGroup);
  float *lsig = reinterpret_cast<float *>(ls + scale_lds_bytes(16 * RB, G));  // limb scales [b][nbk]
  float *red = lsig + kSigLds / 4;
  const int W = blockDim.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar arithmetic
  const int col = lane & 15, qd = lane >> 4;
  const int GP = (G + 1) >> 1;
  const int64_t NB = (N + 15) >> 4;
  // the wave's pairs GP w / W .. GP (w + 1) / W - 1, divided by multiplying with
  // wmagic = ceil(2^16 / W) (exact: GP (w + 1) < 4096 <= 2^16 / W)
  const int p_begin = int((uint32_t(GP * wave) * wmagic) >> 16);
  const int np = int((uint32_t(GP * (wave + 1)) * wmagic) >> 16) - p_begin;
  const int64_t n0 = int64_t(blockIdx.x) * (16 * RB);
  // The wave's pairs lie in 1024-block fb and, from pair 4 lb on, in block lb
  // (four pairs a block, at most five pairs a wave, so at most two blocks).  The
  // sums of each block are kept apart and scaled by that block's limb scales at
  // the end; the scales come into LDS with the other direct loads, so no load
  // of the weight stream waits for them.  Only the variants with limbs in LDS
  // have the registers for a second set of sums; the plan gives the others only
  // shapes whose waves' pairs stay in one block.
  const int nbk = limb_blocks(K);
  const int fb = min(p_begin >> 2, nbk - 1), lb = min((p_begin + np - 1) >> 2, nbk - 1);

  // A operand row of this lane: (token, limb) per the LP or two-limb mapping
  const int tok = LP ? lp_token(col) : token_of_arow(col);
  const int tok_ld = tok < b ? tok : b - 1;
  const int64_t arow = LP ? int64_t(col & 1) * b + tok_ld : tok_ld;
  // LP: row-major limb rows; otherwise operand order (1 KB per group, half, limb)
  const int8_t *gah = LP ? limbs + arow * Kp + 32 * qd : limbs + 16 * lane;  // global limbs
  const int8_t *gal = LP ? gah + int64_t(b) * Kp : gah + 1024;
  const int8_t *lah = LP ? lx + arow * Kp + 32 * qd : lx + 16 * lane;        // the same in LDS
  const int8_t *lal = LP ? lah + int64_t(b) * Kp : lah + 1024;
  constexpr int kGS = LP ? 128 : 4096, kHS = LP ? 16 : 2048;  // group and half strides

  // 1. direct loads into LDS
  stage_scales(scales, N, G, n0, 16 * RB, ls, wave, W, lane);
  if (wave == W - 1) {
    // the chunk's b x nbk limb scales in 16-byte pieces (the workspace holds those
    // of 64 tokens, so a rounded-up last piece stays inside it)
    const int pieces = (b * nbk * 4 + 15) >> 4;
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const char *>(sigma) + 16 * min(lane, pieces - 1),
                                     (__attribute__((address_space(3))) void *)lsig, 16, 0, 0);
  }
  if (ALDS) {
    for (int blk = wave; blk * 1024 < lds_limb_bytes; blk += W) {
      const int64_t off = int64_t(blk) * 1024 + 16 * lane;
      const int64_t src = off < region ? off : 0;
      __builtin_amdgcn_global_load_lds(limbs + src,
                                       (__attribute__((address_space(3))) void *)(lx + blk * 1024),
                                       16, 0, 0);
    }
  }
  asm volatile("" ::: "memory");
  // 2. register loads of every pair
  v4i ga[ALDS ? 1 : PMAX][2][2][LP ? 1 : 2];  // [pair][group][64-k half][limb]
  uint4 wv[PMAX][RB];
#pragma unroll
  for (int pi = 0; pi < PMAX; ++pi) {
    const int p = p_begin + (pi < np ? pi : np - 1);
    if (!ALDS) {
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const int64_t gl = min(2 * p + gi, G - 1);  // a padded last group reads a valid row part
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          ga[ALDS ? 0 : pi][gi][h][0] = *reinterpret_cast<const v4i *>(gah + kGS * gl + kHS * h);
          if (!LP) ga[ALDS ? 0 : pi][gi][h][LP ? 0 : 1] = *reinterpret_cast<const v4i *>(gal + kGS * gl + kHS * h);
        }
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      wv[pi][rb] = load_tile(packed, min(int64_t(blockIdx.x) * RB + rb, NB - 1), GP, p, lane);
  }
  asm volatile("" ::: "memory");
  ps.mark(1);
  // 3. wait for the direct loads only; the register loads may stay in
  //    flight.  With limbs in LDS nothing may be scheduled above this point: work
  //    on a tile moved up here would make the wait cover every load (the counter
  //    is in order).  With limbs in registers the compiler's own interleaving of
  //    the first pairs' matrix instructions with the loads is the faster one.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm<PMAX * (RB + (ALDS ? 0 : NA))>());
  ps.mark(2);
  __builtin_amdgcn_s_barrier();
  if constexpr (ALDS) __builtin_amdgcn_sched_barrier(0);
  ps.mark(3);

  // 4. pairs in arrival order.  LDS is read through lds_read* so that the
  //    compiler, which cannot tell these reads from the destinations of the
  //    direct loads, does not make each of them wait for every register load.
  //    The next pair's LDS reads are issued before this pair's matrix
  //    instructions (two register slots), so their latency overlaps the work.
  float acc[RB][4], acc1[ALDS ? RB : 1][4];  // acc1: block fb's sums once block lb starts
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[rb][i] = 0.0f;
  constexpr int kLdsPerPair = (ALDS ? (LP ? 4 : 8) : 0) + 2 * RB;
  // the second slot costs registers: only where the estimate (tiles, both slots,
  // accumulators, addressing) stays inside the variant's budget; and the wait
  // count field holds up to 15
  constexpr int kRegs = PMAX * RB * 4 + (ALDS ? 2 * (LP ? 16 : 32) : 0) + 8 * RB + 48;
  constexpr bool kPipe =
      kLdsPerPair <= 15 && (!ALDS || kRegs <= (stream_heavy(ALDS, RB, PMAX, LP) ? 256 : 128));
  v4i ahs[2][2][2], als[2][2][2];             // [slot][group][64-k half]
  uint32_t sbs[2][2][RB];
  if (kPipe) pair_lds_issue<RB, LP, ALDS>(p_begin, G, lah, lal, ls, col, ahs[0], als[0], sbs[0]);
#pragma unroll
  for (int pi = 0; pi < PMAX; ++pi) {
    const bool live = pi < np;
    const int p = p_begin + (live ? pi : np - 1);
    const int sl = kPipe ? (pi & 1) : 0;
    if (kPipe && pi + 1 < PMAX) {
      const int pn = p_begin + (pi + 1 < np ? pi + 1 : np - 1);
      pair_lds_issue<RB, LP, ALDS>(pn, G, lah, lal, ls, col, ahs[sl ^ 1], als[sl ^ 1], sbs[sl ^ 1]);
      lds_wait_n<kPipe ? kLdsPerPair : 0, RB>(ahs[sl], als[sl], sbs[sl], LP || !ALDS);
    } else {
      if (!kPipe) pair_lds_issue<RB, LP, ALDS>(p, G, lah, lal, ls, col, ahs[sl], als[sl], sbs[sl]);
      lds_wait_n<0, RB>(ahs[sl], als[sl], sbs[sl], LP || !ALDS);
    }
    v4i ah[2][2], al[2][2];
    if (!ALDS) {
#pragma unroll
      for (int gi = 0; gi < 2; ++gi)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          ah[gi][h] = ga[ALDS ? 0 : pi][gi][h][0];
          al[gi][h] = ga[ALDS ? 0 : pi][gi][h][LP ? 0 : 1];
        }
    } else {
#pragma unroll
      for (int gi = 0; gi < 2; ++gi)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          ah[gi][h] = ahs[sl][gi][h];
          al[gi][h] = LP ? ahs[sl][gi][h] : als[sl][gi][h];
        }
    }
    float sv[2][RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      sv[0][rb] = live ? half_bits_to_float(uint16_t(sbs[sl][0][rb])) : 0.0f;
      sv[1][rb] = live && 2 * p + 1 < G ? half_bits_to_float(uint16_t(sbs[sl][1][rb])) : 0.0f;
    }
    if constexpr (ALDS) {
      if (lb != fb && live && p == 4 * lb) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc1[rb][i] = acc[rb][i], acc[rb][i] = 0.0f;
      }
    }
    pair_mfma<RB, NT, LP>(ah, al, wv[pi], sv, acc);
    if (pi == 0) ps.mark(4);
  }
  ps.mark(5);
  // each block's sums times its limb scales (and the 1/64 of the unpacked codes);
  // every LDS read of the loop has been waited for
  float ua[4], ub[ALDS ? 4 : 1];
  token_scales<NT, LP>(lsig + fb, nbk, b, lane, ua);
  if constexpr (ALDS) token_scales<NT, LP>(lsig + lb, nbk, b, lane, ub);
  float tsc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) tsc[i] = 1.0f / 64.0f;
  if (ALDS && lb != fb) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < NT; ++i) acc[rb][i] = acc1[ALDS ? rb : 0][i] * ua[i] + acc[rb][i] * ub[ALDS ? i : 0];
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < NT; ++i) acc[rb][i] *= ua[i];
  }
  ps.flush();
  // `red` lies past every region the loop reads (limbs, scales, limb scales), and
  // every direct load into LDS was waited for before the first barrier: the
  // partials can go to LDS at once, the barrier inside the reduction orders them
  reduce_and_store<RB, NT, LP>(acc, red, W, wave, lane, b, n0, N, tsc, y, y_dtype);
  ps.done();
}

// --------------------------------------------------------------------------
// gemv_q8: the same weight stream against int8 activations (one limb)
// --------------------------------------------------------------------------
// y[t, n] = sx_t * sum_g s[n,g] sum_{k in g} code[n,k] xq[t,k] with xq, sx the
// per-token int8 activations of the prefill path (tl_quant_act_int8).  One MFMA
// chain per group instead of the two limb chains, and b*K activation bytes
// instead of 2*b*K; the price is the activation rounding (~8e-3 relative on the
// generator's data, against ~3e-5 for the two-limb GEMV).  A operand row r holds
// token 4 (r % 4) + r / 4 (clamped to b - 1), read from the caller's row-major
// xq: staged in LDS with rows K + 16 bytes apart when b (K + 16) fits, else
// loaded from L2 into registers with the tiles.
template <int RB, int NT>
__device__ __forceinline__ void group_mfma_q8(const v4i (&a)[2], const uint32_t (&w0)[RB],
                                              const uint32_t (&w1)[RB], const float (&s)[RB],
                                              float (&acc)[RB][4]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const v4i z = {0, 0, 0, 0};
    v4i d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[0], unpack_x64(w0[rb]), z, 0, 0, 0);
    d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[1], unpack_x64(w1[rb]), d, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[rb][i] = fmaf(s[rb], (float)d[i], acc[rb][i]);
  }
}

// register budget: ALDS holds RB tiles per pair, otherwise also 4 activation fragments
// (more than 20 registers' worth of 16-byte loads: 512 threads, 256 VGPRs; the
// register variant then takes up to 9 pairs per wave, which covers K <= 18432)
constexpr bool q8_heavy(bool alds, int rb, int pmax) { return alds ? pmax * rb > 10 : pmax * (rb + 4) > 20; }
constexpr int kQ8PmaxReg = 9;

template <int RB, int NT, int PMAX, bool ALDS>
__global__ __launch_bounds__(q8_heavy(ALDS, RB, PMAX) ? 512 : 1024) void gemv_q8_kernel(
    const int8_t *__restrict__ xq, const float *__restrict__ tok_scale, int b, int64_t K, int64_t N,
    const uint32_t *__restrict__ packed, const uint16_t *__restrict__ scales, void *__restrict__ y,
    int y_dtype, int lds_a_bytes) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int8_t *lx = reinterpret_cast<int8_t *>(smem);
  char *ls = smem + (ALDS ? lds_a_bytes : 0);
  const int G = int(K / kGroup);
  float *red = reinterpret_cast<float *>(ls + scale_lds_bytes(16 * RB, G));
  const int W = blockDim.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar arithmetic
  const int col = lane & 15, qd = lane >> 4;
  const int GP = (G + 1) >> 1;
  const int64_t NB = (N + 15) >> 4;
  const int p_begin = (GP * wave) / W;
  const int np = (GP * (wave + 1)) / W - p_begin;
  const int64_t n0 = int64_t(blockIdx.x) * (16 * RB);
  const int64_t Ks = K + kRowPad;  // LDS row pitch
  const int tok = token_of_arow(col);
  const int tok_ld = tok < b ? tok : b - 1;
  const int8_t *ga = xq + int64_t(tok_ld) * K + 32 * qd;
  const int8_t *la = lx + int64_t(tok_ld) * Ks + 32 * qd;

  // 1. direct loads: the scale block, and (ALDS) the b activation rows, byte P of
  //    the LDS image holding row P / Ks, column P % Ks (the 16 pad bytes of a row
  //    load any valid address)
  stage_scales(scales, N, G, n0, 16 * RB, ls, wave, W, lane);
  if (ALDS) {
    for (int c = wave; c * 1024 < lds_a_bytes; c += W) {
      const int64_t P = int64_t(c) * 1024 + 16 * lane;
      const int64_t r = P / Ks, off = P - r * Ks;
      const int8_t *src = r < b && off < K ? xq + r * K + off : xq;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(lx + c * 1024), 16,
                                       0, 0);
    }
  }
  asm volatile("" ::: "memory");
  // 2. register loads of every pair
  v4i ga_r[ALDS ? 1 : PMAX][2][2];  // [pair][group][64-k half]
  uint4 wv[PMAX][RB];
#pragma unroll
  for (int pi = 0; pi < PMAX; ++pi) {
    const int p = p_begin + (pi < np ? pi : np - 1);
    if (!ALDS) {
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        const int64_t gl = min(2 * p + gi, G - 1);
#pragma unroll
        for (int h = 0; h < 2; ++h) ga_r[ALDS ? 0 : pi][gi][h] = *reinterpret_cast<const v4i *>(ga + 128 * gl + 16 * h);
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      wv[pi][rb] = load_tile(packed, min(int64_t(blockIdx.x) * RB + rb, NB - 1), GP, p, lane);
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm<PMAX * (RB + (ALDS ? 0 : 4))>());
  __builtin_amdgcn_s_barrier();

  // 3. pairs in arrival order
  float acc[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[rb][i] = 0.0f;
#pragma unroll
  for (int pi = 0; pi < PMAX; ++pi) {
    const bool live = pi < np;
    const int p = p_begin + (live ? pi : np - 1);
    v4i a[2][2], unused[2][2];
    uint32_t sb[2][RB];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const int gl = min(2 * p + gi, G - 1);
      if (ALDS) {
#pragma unroll
        for (int h = 0; h < 2; ++h) a[gi][h] = lds_read16(la + 128 * gl + 16 * h);
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sb[gi][rb] = lds_read_u16(ls + 2 * ((16 * rb + col) * G + gl));
    }
    lds_wait<RB>(a, unused, sb, true);
    if (!ALDS) {
#pragma unroll
      for (int gi = 0; gi < 2; ++gi)
#pragma unroll
        for (int h = 0; h < 2; ++h) a[gi][h] = ga_r[ALDS ? 0 : pi][gi][h];
    }
    float s0[RB], s1[RB];
    uint32_t w00[RB], w01[RB], w10[RB], w11[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      s0[rb] = live ? half_bits_to_float(uint16_t(sb[0][rb])) : 0.0f;
      s1[rb] = live && 2 * p + 1 < G ? half_bits_to_float(uint16_t(sb[1][rb])) : 0.0f;
      w00[rb] = wv[pi][rb].x;
      w01[rb] = wv[pi][rb].y;
      w10[rb] = wv[pi][rb].z;
      w11[rb] = wv[pi][rb].w;
    }
    group_mfma_q8<RB, NT>(a[0], w00, w01, s0, acc);
    group_mfma_q8<RB, NT>(a[1], w10, w11, s1, acc);
  }
  __syncthreads();  // every wave is done with LDS before `red` is written
  float tsc[4];
  token_scales<NT, false>(tok_scale, 1, b, lane, tsc);
#pragma unroll
  for (int i = 0; i < 4; ++i) tsc[i] *= 1.0f / 64.0f;
  reduce_and_store<RB, NT, false>(acc, red, W, wave, lane, b, n0, N, tsc, y, y_dtype);
}

// --------------------------------------------------------------------------
// gemv_ring: limb fragments in registers, two pairs of groups in flight per wave
// (for long K, where a wave's pairs do not all fit in registers at once)
// --------------------------------------------------------------------------
template <int RB>
struct PairSlot {
  v4i ah[2][2], al[2][2];  // limbs: [group of the pair][64-k half]
  uint4 w[RB];             // tile words, per row block
};

template <int RB, bool LP>
__device__ __forceinline__ void load_pair(PairSlot<RB> &f, int p, int G, int GP, const int8_t *ah,
                                          const int8_t *al, const uint32_t *__restrict__ packed,
                                          const int64_t (&rbg)[RB], int lane) {
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const int gl = min(2 * p + gi, G - 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      constexpr int64_t kGS = LP ? 128 : 4096, kHS = LP ? 16 : 2048;  // row-major / operand order
      f.ah[gi][h] = *reinterpret_cast<const v4i *>(ah + kGS * gl + kHS * h);
      if (!LP) f.al[gi][h] = *reinterpret_cast<const v4i *>(al + kGS * gl + kHS * h);
    }
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) f.w[rb] = load_tile(packed, rbg[rb], GP, p, lane);
}

// scales of pair p for the lane's rows, from the staged block
template <int RB>
__device__ __forceinline__ void pair_scales(float (&s)[2][RB], const char *ls, int col, int G, int p) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) pair_scales_lds(ls, 16 * rb + col, G, p, s[0][rb], s[1][rb]);
}

// wave cap per workgroup: larger row tiles need more registers per wave
template <int RB>
struct GemvWaveCap {
  static constexpr int value = RB == 1 ? 12 : RB == 2 ? 8 : 4;
};

// before pair q: where a 1024-block starts, the sums change to its units (the
// chunk's limb scales lsig [b][nbk] are in LDS)
template <int RB, int NT, bool LP>
__device__ __forceinline__ void ring_block(int q, int &cb, float (&acc)[RB][4], float (&ua)[4],
                                           const float *lsig, int nbk, int b, int lane) {
  if ((q >> 2) == cb) return;
  cb = q >> 2;
  float un[4];
  token_scales<NT, LP>(lsig + cb, nbk, b, lane, un);
  change_units<RB, NT>(acc, ua, un);
}

template <int RB, int NT, bool LP>
__global__ __launch_bounds__(64 * GemvWaveCap<RB>::value) void gemv_ring_kernel(
    const int8_t *__restrict__ limbs, const float *__restrict__ sigma, int b, int64_t K,
    int64_t Kp, int64_t N, const uint32_t *__restrict__ packed, const uint16_t *__restrict__ scales,
    void *__restrict__ y, int y_dtype) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  select_chunk(limbs, sigma, y, b, K, N, y_dtype);
  // scale block of the workgroup's rows, the chunk's limb scales [b][nbk], then
  // W * RB * NT * 64 floats
  char *ls = smem;
  float *lsig = reinterpret_cast<float *>(smem + scale_lds_bytes(16 * RB, int(K / kGroup)));
  float *red = reinterpret_cast<float *>(reinterpret_cast<char *>(lsig) + ring_sig_bytes(K));
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
  // the sums hold units of the limb scale of block cb and change units as each
  // next 1024-block starts (four pairs a block), with the scales from LDS
  const int nbk = limb_blocks(K);
  int cb = min(p_begin >> 2, nbk - 1);
  for (int e = threadIdx.x; e < b * nbk; e += blockDim.x) lsig[e] = sigma[e];

  const int tok = LP ? lp_token(col) : token_of_arow(col);
  const int tok_ld = tok < b ? tok : b - 1;
  const int8_t *ah = LP ? limbs + int64_t((col & 1) * b + tok_ld) * Kp + 32 * qd : limbs + 16 * lane;
  const int8_t *al = LP ? ah + int64_t(b) * Kp : ah + 1024;
  int64_t rbg[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) rbg[rb] = min(int64_t(blockIdx.x) * RB + rb, NB - 1);

  float acc[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[rb][i] = 0.0f;

  // two pair slots: slot (p - p_begin) % 2; the next pair is in flight while one is used
  PairSlot<RB> sl[2];
  if (p_begin < p_end) load_pair<RB, LP>(sl[0], p_begin, G, GP, ah, al, packed, rbg, lane);
  if (p_begin + 1 < p_end) load_pair<RB, LP>(sl[1], p_begin + 1, G, GP, ah, al, packed, rbg, lane);
  stage_scales(scales, N, G, n0, 16 * RB, ls, wave, W, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  float ua[4];
  token_scales<NT, LP>(lsig + cb, nbk, b, lane, ua);
  for (int p = p_begin; p < p_end; p += 2) {
    float s[2][RB];
    pair_scales<RB>(s, ls, col, G, p);
    ring_block<RB, NT, LP>(p, cb, acc, ua, lsig, nbk, b, lane);
    pair_mfma<RB, NT, LP>(sl[0].ah, LP ? sl[0].ah : sl[0].al, sl[0].w, s, acc);
    if (p + 2 < p_end) load_pair<RB, LP>(sl[0], p + 2, G, GP, ah, al, packed, rbg, lane);
    if (p + 1 < p_end) {
      pair_scales<RB>(s, ls, col, G, p + 1);
      ring_block<RB, NT, LP>(p + 1, cb, acc, ua, lsig, nbk, b, lane);
      pair_mfma<RB, NT, LP>(sl[1].ah, LP ? sl[1].ah : sl[1].al, sl[1].w, s, acc);
      if (p + 3 < p_end) load_pair<RB, LP>(sl[1], p + 3, G, GP, ah, al, packed, rbg, lane);
    }
  }
  float tsc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) tsc[i] = ua[i] * (1.0f / 64.0f);
  reduce_and_store<RB, NT, LP>(acc, red, W, wave, lane, b, n0, N, tsc, y, y_dtype);
}

// --------------------------------------------------------------------------
// variant choice and launch
// --------------------------------------------------------------------------
struct GemvPlan {
  int kind;  // 0: stream with limbs in LDS, 1: stream with limbs from L2, 2: ring
  int rb, waves, pmax;
  int chunks;  // grid rows: token chunks of 16
  int lds_limb_bytes;
  size_t lds_bytes;
  const char *name;
  bool ok;     // the variant fits the compute unit (LDS, workgroup size)
};

constexpr int kLdsLimbBudget = 96 * 1024;
constexpr int kPmaxLds = 5;   // pairs per wave, limbs in LDS
constexpr int kPmaxReg = 3;   // pairs per wave, A fragments in registers
constexpr int kMaxWaves = 16;

// Row blocks per workgroup of the int8-activation variant: the smallest of 1, 2, 4
// whose workgroups all fit on the chip at once (one round), given how many fit per
// compute unit by LDS and by waves; 4 when none does.
constexpr int kCUs = 256;
constexpr int kLdsPerCU = 160 * 1024;
constexpr int kWavesPerCU = 32;

int fit_rb(int64_t N, int64_t chunks, size_t lds_fixed, size_t lds_per_rb, int waves) {
  for (int rb = 1; rb <= 4; rb *= 2) {
    const size_t lds = lds_fixed + lds_per_rb * rb;
    const int64_t per_cu = std::min<int64_t>(int64_t(kLdsPerCU / lds), kWavesPerCU / waves);
    if ((N + 16 * rb - 1) / (16 * rb) * chunks <= per_cu * kCUs) return rb;
  }
  return 4;
}

// workgroups of a stream-kernel variant resident per compute unit (defined after
// the launch helpers); 0 when the runtime cannot tell
int stream_resident(bool alds, int rb, int64_t b, int pmax, int waves, size_t lds);

// "gemv_stream_lds_rb1_w4p5": kind, row blocks per workgroup, waves and pairs per
// wave (the ring keeps two pairs per wave in flight: "gemv_ring_rb2_w8").  Static
// strings, built once.
const char *variant_name(int kind, int rb, int waves, int pmax) {
  static const std::vector<std::string> table = [] {
    std::vector<std::string> t;
    static const char *kinds[3] = {"gemv_stream_lds", "gemv_stream_reg", "gemv_ring"};
    for (int k = 0; k < 3; ++k)
      for (int r = 1; r <= 4; ++r)
        for (int w = 0; w <= 16; ++w)
          for (int m = 0; m <= kPmaxLds; ++m)
            t.push_back(std::string(kinds[k]) + "_rb" + std::to_string(r) + "_w" + std::to_string(w) +
                        (k == 2 ? "" : "p" + std::to_string(m)));
    return t;
  }();
  if (kind < 0 || kind > 2 || rb < 1 || rb > 4 || waves < 0 || waves > 16 || pmax < 0 || pmax > kPmaxLds)
    return "gemv_unnamed";
  return table[((size_t(kind) * 4 + (rb - 1)) * 17 + waves) * (kPmaxLds + 1) + pmax].c_str();
}

// true when some wave's share of the GP pairs (GP w / W .. GP (w + 1) / W - 1)
// reaches across a 1024-block boundary (four pairs)
bool straddles(int64_t GP, int W) {
  for (int w = 0; w < W; ++w) {
    const int64_t pb = GP * w / W, pe = GP * (w + 1) / W - 1;
    if (pe >= pb && (pb >> 2) != (pe >> 2)) return true;
  }
  return false;
}

GemvPlan plan_gemv(int64_t b, int64_t K, int64_t N) {
  // more than 16 tokens: one grid row per chunk of 16, each shaped like b = 16
  const int64_t chunks = b > kTokChunk ? limb_chunks(b) : 1;
  b = std::min<int64_t>(b, kTokChunk);
  const int64_t G = K / kGroup, GP = (G + 1) / 2;
  const int nt = b <= 8 ? 2 : int((b + 3) / 4);  // accumulators per row block and lane
  const int64_t limb_bytes = (limb_region_bytes(b, K) + 1023) / 1024 * 1024;
  GemvPlan p{};
  const bool lp = b <= 8;
  // waves for PMAX pairs each, within the wave cap of the resulting variant; false
  // when even the largest pair count leaves more waves than the cap allows
  auto shape = [&](bool alds, int rb, int pmax) {
    for (;; ++pmax) {
      const int cap = stream_heavy(alds, rb, pmax, lp) ? 8 : kMaxWaves;
      const int waves = int((GP + pmax - 1) / pmax);
      if (waves <= cap) {
        p.waves = waves;
        p.pmax = int((GP + waves - 1) / waves);
        return true;
      }
      if (pmax >= (alds ? kPmaxLds : kPmaxReg)) return false;
    }
  };
  // Row blocks per workgroup, 1..4 (limbs in LDS: the measured rule below first):
  // the smallest whose workgroups are all resident
  // at once (one round), else the one with the lowest rounds x (3 + RB).  A
  // workgroup costs about 3 row blocks' worth of weight streaming for its fixed
  // part (limbs, scales, reduction) plus one per row block: the fit to measured qkv
  // and gate_up launches at b = 1..16 (RB = 3 beat 4 by 7-14 % at b = 8 and 16).
  // Residency: the runtime's occupancy figure for the variant (its registers and
  // LDS), cached per variant.
  // Row blocks that cannot be shaped, or whose LDS exceeds the compute unit's, are
  // skipped; 0 when none is left.
  auto choose_rb = [&](bool alds, int pmax0, size_t lds_limbs) {
    if (alds) {
      // limbs in LDS: the row-block count measured best (qkv 5120 -> 10240, o
      // 5120 -> 5120, gate_up 5120 -> 34816 and a 1024 -> 300 layer at
      // b = 1, 2, 4, 8; each workgroup stages 2 b K bytes of limbs): one row block
      // while b <= 2, while b <= 4 and the grid of single row blocks is at most
      // three per CU, or when it does not even fill the CUs; else three, or two
      // where three would leave a quarter of the CUs idle.  (gate_up b = 1:
      // 11.2 us at one against 13.0 at two; qkv b = 8: 6.9 us at three against
      // 9.0 at two and 9.8 at one; o b = 8: 5.3 us at two against 6.4 at three.)
      const int64_t rows16 = (N + 15) / 16 * chunks, rows48 = (N + 47) / 48 * chunks;
      const int pref = rows16 <= kCUs || b <= 2 || (b <= 4 && rows16 <= 3 * kCUs) ? 1
                       : rows48 >= 3 * kCUs / 4 ? 3 : 2;
      const size_t lds = lds_limbs + scale_lds_bytes(16 * pref, int(G)) + kSigLds;
      if (shape(true, pref, pmax0) &&
          lds + size_t(p.waves) * pref * nt * 256 <= size_t(kLdsPerCU))
        return pref;
    }
    int best = 0;
    int64_t best_cost = INT64_MAX;
    for (int rb = 1; rb <= 4; ++rb) {
      if (!shape(alds, rb, pmax0) || (!alds && straddles(GP, p.waves))) continue;
      const size_t lds = lds_limbs + scale_lds_bytes(16 * rb, int(G)) + kSigLds +
                         size_t(p.waves) * rb * nt * 256;
      if (lds > size_t(kLdsPerCU)) continue;
      int64_t per_cu = stream_resident(alds, rb, b, p.pmax, p.waves, lds);
      if (per_cu <= 0) {  // no answer from the runtime: bound by LDS and the register budget
        const int wave_cap = stream_heavy(alds, rb, p.pmax, lp) ? 8 : 16;
        per_cu = std::max<int64_t>(1, std::min<int64_t>(int64_t(kLdsPerCU / lds), wave_cap / p.waves));
      }
      // limbs from L2: every workgroup reads all b tokens' limbs itself (2 b K
      // bytes, against 4 K of weights per row block), so a second workgroup on a
      // compute unit adds that traffic rather than hiding latency: count one
      // (b = 16 qkv: 3 row blocks in 213 workgroups 7.7 us, 2 in 320 resident
      // two per CU 9.7 us)
      if (!alds) per_cu = 1;
      const int64_t wgs = (N + 16 * rb - 1) / (16 * rb) * chunks;
      const int64_t rounds = (wgs + per_cu * kCUs - 1) / (per_cu * kCUs);
      if (rounds == 1) return rb;
      if (rounds * (3 + rb) < best_cost) best_cost = rounds * (3 + rb), best = rb;
    }
    return best;
  };
  int rb = 0;
  if (limb_bytes <= kLdsLimbBudget && GP <= 8 * kPmaxLds &&
      (rb = choose_rb(true, b <= 4 ? 5 : 3, size_t(limb_bytes))) > 0) {
    // limbs in LDS.  Small batches: few waves with several pairs each, so that
    // pairs are computed while later ones arrive; b > 4: up to four row blocks
    // share one copy of the limbs.
    p.kind = 0;
    p.lds_limb_bytes = int(limb_bytes);
    p.rb = rb;
    shape(true, p.rb, b <= 4 ? 5 : 3);
  } else if (GP <= 8 * kPmaxReg && (rb = choose_rb(false, 2, 0)) > 0) {
    // limbs from L2 into registers, all pairs at once (shapes whose waves' pairs
    // each stay inside one 1024-block)
    p.kind = 1;
    p.lds_limb_bytes = 0;
    p.rb = rb;
    shape(false, p.rb, 2);
  } else {
    p.kind = 2;
    p.rb = N >= 16 * 2 * 128 ? 2 : 1;
    const int cap = p.rb == 1 ? GemvWaveCap<1>::value : GemvWaveCap<2>::value;
    p.waves = int(GP < cap ? GP : cap);
    p.pmax = 0;
    p.lds_limb_bytes = 0;
  }
  p.lds_bytes = size_t(p.lds_limb_bytes) + scale_lds_bytes(16 * p.rb, int(G)) + (p.kind == 2 ? ring_sig_bytes(K) : kSigLds) +
                size_t(p.waves) * p.rb * nt * 64 * sizeof(float);
  p.name = variant_name(p.kind, p.rb, p.waves, p.pmax);
  p.chunks = int(chunks);
  p.ok = p.lds_bytes <= size_t(kLdsPerCU) && p.waves >= 1 && 64 * p.waves <= 1024 &&
         (p.kind == 2 || GP * p.waves < 4096);  // the stream kernels' reciprocal division
  return p;
}

struct GemvArgs {
  const GemvWs *w;
  int64_t b, K, N;
  const uint32_t *packed;
  const uint16_t *scales;
  void *y;
  int y_dtype;
  hipStream_t stream;
  int *resident = nullptr;  // set: report workgroups per CU for the variant instead of launching
};

template <int RB, int NT, int PMAX, bool LP, bool ALDS>
void launch_stream_t(const GemvPlan &p, dim3 grid, const GemvArgs &a) {
  if (a.resident) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(a.resident, gemv_stream_kernel<RB, NT, PMAX, LP, ALDS>,
                                                     64 * p.waves, p.lds_bytes) != hipSuccess)
      *a.resident = 0;
    return;
  }
  hipLaunchKernelGGL((gemv_stream_kernel<RB, NT, PMAX, LP, ALDS>), grid, dim3(64 * p.waves), p.lds_bytes,
                     a.stream, a.w->xhi, a.w->sigma, int(a.b), a.K, a.w->Kp, a.N, a.packed, a.scales, a.y,
                     a.y_dtype, p.lds_limb_bytes, (65536u + p.waves - 1) / p.waves);
}

template <int RB, int NT, bool LP, bool ALDS>
void launch_stream_p(const GemvPlan &p, dim3 grid, const GemvArgs &a) {
  if constexpr (ALDS) {
    switch (p.pmax) {
      case 1: launch_stream_t<RB, NT, 1, LP, ALDS>(p, grid, a); break;
      case 2: launch_stream_t<RB, NT, 2, LP, ALDS>(p, grid, a); break;
      case 3: launch_stream_t<RB, NT, 3, LP, ALDS>(p, grid, a); break;
      case 4: launch_stream_t<RB, NT, 4, LP, ALDS>(p, grid, a); break;
      default: launch_stream_t<RB, NT, 5, LP, ALDS>(p, grid, a); break;
    }
  } else {
    switch (p.pmax) {
      case 1: launch_stream_t<RB, NT, 1, LP, ALDS>(p, grid, a); break;
      case 2: launch_stream_t<RB, NT, 2, LP, ALDS>(p, grid, a); break;
      default: launch_stream_t<RB, NT, 3, LP, ALDS>(p, grid, a); break;
    }
  }
}

template <int RB, bool ALDS>
void launch_stream_n(const GemvPlan &p, dim3 grid, const GemvArgs &a) {
  switch ((std::min<int64_t>(a.b, kTokChunk) + 3) / 4) {
    case 1:
    case 2: launch_stream_p<RB, 2, true, ALDS>(p, grid, a); break;
    case 3: launch_stream_p<RB, 3, false, ALDS>(p, grid, a); break;
    default: launch_stream_p<RB, 4, false, ALDS>(p, grid, a); break;
  }
}

template <bool ALDS>
void launch_stream(const GemvPlan &p, dim3 grid, const GemvArgs &a) {
  if (p.rb == 3) launch_stream_n<3, ALDS>(p, grid, a);
  else if (p.rb == 4) launch_stream_n<4, ALDS>(p, grid, a);
  else if (p.rb == 2) launch_stream_n<2, ALDS>(p, grid, a);
  else launch_stream_n<1, ALDS>(p, grid, a);
}

template <int RB>
void launch_ring_r(const GemvPlan &p, dim3 grid, const GemvArgs &a) {
  const dim3 blk(64 * p.waves);
  const GemvWs &w = *a.w;
  switch ((std::min<int64_t>(a.b, kTokChunk) + 3) / 4) {
    case 1:
    case 2: hipLaunchKernelGGL((gemv_ring_kernel<RB, 2, true>), grid, blk, p.lds_bytes, a.stream, w.xhi, w.sigma, int(a.b), a.K, w.Kp, a.N, a.packed, a.scales, a.y, a.y_dtype); break;
    case 3: hipLaunchKernelGGL((gemv_ring_kernel<RB, 3, false>), grid, blk, p.lds_bytes, a.stream, w.xhi, w.sigma, int(a.b), a.K, w.Kp, a.N, a.packed, a.scales, a.y, a.y_dtype); break;
    default: hipLaunchKernelGGL((gemv_ring_kernel<RB, 4, false>), grid, blk, p.lds_bytes, a.stream, w.xhi, w.sigma, int(a.b), a.K, w.Kp, a.N, a.packed, a.scales, a.y, a.y_dtype); break;
  }
}

// int8-activation variant: limbs replaced by the caller's xq rows (see gemv_q8)
struct Q8Plan {
  bool ok, alds;
  int rb, nt, waves, pmax, lds_a;
  size_t lds;
  const char *name;
};

Q8Plan plan_q8(int64_t b, int64_t K, int64_t N) {
  Q8Plan p{};
  const int64_t G = K / kGroup, GP = (G + 1) / 2;
  p.nt = b <= 4 ? 1 : b <= 8 ? 2 : 4;
  const int64_t lds_a = (b * (K + kRowPad) + 1023) / 1024 * 1024;
  p.alds = lds_a <= kLdsLimbBudget;
  p.lds_a = p.alds ? int(lds_a) : 0;
  p.rb = GP > 40 ? 1 : fit_rb(N, 1, size_t(p.lds_a), scale_lds_bytes(16, int(G)) + 8 * size_t(p.nt) * 256, 8);
  p.rb = std::min(p.rb, 2);
  for (int pmax = b <= 4 ? 5 : 3;; ++pmax) {
    if (pmax > (p.alds ? kPmaxLds : (p.rb == 1 ? kQ8PmaxReg : kPmaxLds))) return p;  // not supported
    const int cap = q8_heavy(p.alds, p.rb, pmax) ? 8 : kMaxWaves;
    const int64_t waves = (GP + pmax - 1) / pmax;
    if (waves <= cap) {
      p.waves = int(waves);
      p.pmax = int((GP + waves - 1) / waves);
      break;
    }
  }
  p.lds = size_t(p.lds_a) + scale_lds_bytes(16 * p.rb, int(G)) +
          size_t(p.waves) * p.rb * p.nt * 64 * sizeof(float);
  p.ok = p.lds <= size_t(kLdsPerCU);
  static const char *names[2][2] = {{"gemv_q8_reg_rb1", "gemv_q8_reg_rb2"}, {"gemv_q8_lds_rb1", "gemv_q8_lds_rb2"}};
  p.name = names[p.alds ? 1 : 0][p.rb - 1];
  return p;
}

struct Q8Args {
  const int8_t *xq;
  const float *tok_scale;
  int64_t b, K, N;
  const uint32_t *packed;
  const uint16_t *scales;
  void *y;
  int y_dtype;
  hipStream_t stream;
};

template <int RB, int NT, int PMAX, bool ALDS>
void launch_q8_t(const Q8Plan &p, const Q8Args &a) {
  const dim3 grid(unsigned((a.N + 16 * RB - 1) / (16 * RB)));
  hipLaunchKernelGGL((gemv_q8_kernel<RB, NT, PMAX, ALDS>), grid, dim3(64 * p.waves), p.lds, a.stream, a.xq,
                     a.tok_scale, int(a.b), a.K, a.N, a.packed, a.scales, a.y, a.y_dtype, p.lds_a);
}

template <int RB, int NT, bool ALDS>
void launch_q8_p(const Q8Plan &p, const Q8Args &a) {
  switch (p.pmax) {
    case 1: launch_q8_t<RB, NT, 1, ALDS>(p, a); break;
    case 2: launch_q8_t<RB, NT, 2, ALDS>(p, a); break;
    case 3: launch_q8_t<RB, NT, 3, ALDS>(p, a); break;
    case 4: launch_q8_t<RB, NT, 4, ALDS>(p, a); break;
    case 5: launch_q8_t<RB, NT, 5, ALDS>(p, a); break;
    default:
      if constexpr (!ALDS && RB == 1) {  // long K: the register variant with up to 9 pairs
        switch (p.pmax) {
          case 6: launch_q8_t<RB, NT, 6, ALDS>(p, a); break;
          case 7: launch_q8_t<RB, NT, 7, ALDS>(p, a); break;
          case 8: launch_q8_t<RB, NT, 8, ALDS>(p, a); break;
          default: launch_q8_t<RB, NT, 9, ALDS>(p, a); break;
        }
      }
      break;
  }
}

template <int RB, bool ALDS>
void launch_q8_n(const Q8Plan &p, const Q8Args &a) {
  if (p.nt == 1) launch_q8_p<RB, 1, ALDS>(p, a);
  else if (p.nt == 2) launch_q8_p<RB, 2, ALDS>(p, a);
  else launch_q8_p<RB, 4, ALDS>(p, a);
}

// --------------------------------------------------------------------------
// gemv_rot: rotation, limbs and GEMV in one launch, for one or two tokens
// --------------------------------------------------------------------------
// Wave w of a workgroup owns Hadamard block w (1024 k, four group pairs) for the
// workgroup's 16 RB rows.  It requests its block of x, the block's 8 group
// scales of those rows (one 16-byte piece per row, straight into LDS) and its
// four pairs of weight tiles, all at once; rotates the block for each token as
// soon as x lands (binary64, exact, rounded once to f32 -- the same arithmetic
// as tl_hadamard_blk); splits each token's block into two int8 limbs against the
// block's own |x|max (sigma per token and block instead of per token); stages
// the limbs in its own LDS (paired-limb rows, reusing the rotation scratch) and
// runs its pairs as the tiles land.  Its partial sums, times the block's sigma,
// are added across the waves.  Every workgroup rotates the blocks it needs
// itself: no limbs in memory, no second launch, no barrier before the MFMAs.
constexpr int kRotScratchBytes = kRotLds * 8;              // rotate_block_raw's LDS, per wave
constexpr int kRotWaveBytes = kRotScratchBytes + 1024;     // + the wave's scale pieces
constexpr int kRotLimbPitch = kHBlock + 16;                // limb row pitch in LDS
constexpr int kRotMaxBlocks = 6;                           // waves per workgroup (LDS <= 64 KB)
static_assert(4 * kRotLimbPitch <= kRotScratchBytes, "two tokens' limb rows fit the scratch");

__host__ __device__ constexpr int rot_lds_bytes(int nblk, int rb) {
  return nblk * kRotWaveBytes + (nblk > 1 ? nblk - 1 : 1) * rb * 2 * 64 * 4;
}

template <int RB, int B>
__global__ __launch_bounds__(64 * kRotMaxBlocks) void gemv_rot_kernel(
    const uint16_t *__restrict__ x, const int8_t *__restrict__ signs, int64_t K, int64_t N,
    const uint32_t *__restrict__ packed, const uint16_t *__restrict__ scales, void *__restrict__ y,
    int y_dtype) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int W = blockDim.x >> 6;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, qd = lane >> 4;
  const int G = int(K / kGroup), GP = G >> 1;
  const int64_t NB = (N + 15) >> 4;
  const int64_t n0 = int64_t(blockIdx.x) * (16 * RB);
  char *wl = smem + wave * kRotWaveBytes;
  double *scratch = reinterpret_cast<double *>(wl);
  int8_t *lx = reinterpret_cast<int8_t *>(wl);  // limb rows, once the rotations are done
  char *ls = wl + kRotScratchBytes;
  float *red = reinterpret_cast<float *>(smem + W * kRotWaveBytes);
  const int blk = wave;

  // 1. loads, in this order: x (waited for first), scale pieces, weight tiles
  RotRaw raw[B];
#pragma unroll
  for (int t = 0; t < B; ++t)
    rotate_load(x + t * K + int64_t(kHBlock) * blk, signs ? signs + int64_t(kHBlock) * blk : nullptr,
                lane, raw[t]);
  asm volatile("" ::: "memory");
  {
    // lane r < 16 RB: the 8 scales of row n0 + r in this block (rows past N and
    // lanes past 16 RB read a clamped, valid row; those bytes are never used)
    const int64_t r = min(n0 + min(lane, 16 * RB - 1), N - 1);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const char *>(scales) + (r * G + 8 * blk) * 2,
                                     (__attribute__((address_space(3))) void *)ls, 16, 0, 0);
  }
  asm volatile("" ::: "memory");
  uint4 wv[4][RB];
#pragma unroll
  for (int pi = 0; pi < 4; ++pi)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      wv[pi][rb] = load_tile(packed, min(int64_t(blockIdx.x) * RB + rb, NB - 1), GP, 4 * blk + pi, lane);
  asm volatile("" ::: "memory");

  // 2. rotation and limbs (rotate_block_raw waits for its own x loads)
  float out[B][kRotEPT];
  float sig[B];
#pragma unroll
  for (int t = 0; t < B; ++t) {
    rotate_block_raw(raw[t], signs != nullptr, scratch, lane, out[t]);
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < kRotEPT; ++j) m = fmaxf(m, fabsf(out[t][j]));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    sig[t] = m / kLimbRange;
    const float inv = m > 0.0f ? kLimbRange / m : 0.0f;
#pragma unroll
    for (int j = 0; j < kRotEPT; ++j) out[t][j] *= inv;
  }
  // limb rows (hi of every token, then lo) over the scratch, element lane + 64 j
#pragma unroll
  for (int t = 0; t < B; ++t)
#pragma unroll
    for (int j = 0; j < kRotEPT; ++j) {
      int q = (int)rintf(out[t][j]);
      q = q > 32639 ? 32639 : (q < -32639 ? -32639 : q);
      const int hi = (q + 128) >> 8;  // floor division: lo lands in [-128, 127]
      lx[t * kRotLimbPitch + lane + 64 * j] = int8_t(hi);
      lx[(B + t) * kRotLimbPitch + lane + 64 * j] = int8_t(q - 256 * hi);
    }
  rot_wave_sync();
  // the scale pieces have landed once only the weight loads are outstanding
  __builtin_amdgcn_s_waitcnt(waitcnt_vm<4 * RB>());

  // 3. the block's four pairs (paired-limb A rows: hi/lo of tokens 0, 1)
  const int tok = lp_token(col);
  const int arow = (col & 1) * B + (tok < B ? tok : B - 1);
  const int8_t *lah = lx + arow * kRotLimbPitch + 32 * qd;
  float acc[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[rb][i] = 0.0f;
#pragma unroll
  for (int pi = 0; pi < 4; ++pi) {
    v4i ah[2][2], al[2][2];
    uint32_t sb[2][RB];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const int gl = 2 * pi + gi;  // group inside the block
#pragma unroll
      for (int h = 0; h < 2; ++h) ah[gi][h] = lds_read16(lah + 128 * gl + 16 * h);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sb[gi][rb] = lds_read_u16(ls + 16 * (16 * rb + col) + 2 * gl);
    }
    lds_wait<RB>(ah, al, sb, true);
#pragma unroll
    for (int gi = 0; gi < 2; ++gi)
#pragma unroll
      for (int h = 0; h < 2; ++h) al[gi][h] = ah[gi][h];
    float sv[2][RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      sv[0][rb] = half_bits_to_float(uint16_t(sb[0][rb]));
      sv[1][rb] = half_bits_to_float(uint16_t(sb[1][rb]));
    }
    pair_mfma<RB, 2, true>(ah, al, wv[pi], sv, acc);
  }

  // 4. the block's sigma (accumulator i holds token 2 qd + i), the 1/64 of the
  //    unpacked codes, then the sum over the waves
  const float c0 = sig[min(2 * qd, B - 1)] * (1.0f / 64.0f);
  const float c1 = sig[min(2 * qd + 1, B - 1)] * (1.0f / 64.0f);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    acc[rb][0] *= c0;
    acc[rb][1] *= c1;
  }
  if (wave > 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 2; ++i) red[(((wave - 1) * RB + rb) * 2 + i) * 64 + lane] = acc[rb][i];
  }
  __syncthreads();
  if (wave > 0) return;
  for (int w = 1; w < W; ++w)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 2; ++i) acc[rb][i] += red[(((w - 1) * RB + rb) * 2 + i) * 64 + lane];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = 2 * qd + i;
    if (t >= B) continue;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int64_t n = n0 + 16 * rb + col;
      if (n >= N) continue;
      if (y_dtype == TL_F32)
        reinterpret_cast<float *>(y)[int64_t(t) * N + n] = acc[rb][i];
      else
        reinterpret_cast<uint16_t *>(y)[int64_t(t) * N + n] = float_to_bf16_bits(acc[rb][i]);
    }
  }
}

template <int RB, int B>
void launch_rot_t(int nblk, const uint16_t *x, const int8_t *signs, int64_t K, int64_t N,
                  const uint32_t *packed, const uint16_t *scales, void *y, int y_dtype,
                  hipStream_t stream) {
  const dim3 grid(unsigned((N + 16 * RB - 1) / (16 * RB)));
  hipLaunchKernelGGL((gemv_rot_kernel<RB, B>), grid, dim3(64 * nblk), rot_lds_bytes(nblk, RB), stream, x,
                     signs, K, N, packed, scales, y, y_dtype);
}

}  // namespace

#if TL_PHASE_STAMPS
// where gemv_stream writes its phase timestamps (NULL: nowhere); instrumented builds only
extern "C" int tl_phase_stamps_set(void *device_buffer) {
  return hipMemcpyToSymbol(HIP_SYMBOL(g_phase_stamps), &device_buffer, sizeof(device_buffer)) == hipSuccess ? 0 : 1;
}
#endif

bool gemv_supported(int64_t b, int64_t K, int64_t N) {
  return b <= 0 || N <= 0 || plan_gemv(b, K, N).ok;
}

size_t gemv_workspace_bytes(int64_t b, int64_t K, int64_t /*N*/) {
  // the two int8 limbs of b tokens, then the limb scales of up to 64 tokens
  return align256(size_t(limb_region_bytes(b, K))) +
         align256(size_t(kGemvMaxTokens) * limb_blocks(K) * sizeof(float));
}

namespace {
int stream_resident(bool alds, int rb, int64_t b, int pmax, int waves, size_t lds) {
  static std::mutex mu;
  static std::map<std::tuple<bool, int, int64_t, int, int, size_t>, int> cache;
  const auto key = std::make_tuple(alds, rb, std::min<int64_t>(b, kTokChunk), pmax, waves, lds);
  {
    std::lock_guard<std::mutex> lock(mu);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  GemvPlan p{};
  p.rb = rb;
  p.pmax = pmax;
  p.waves = waves;
  p.lds_bytes = lds;
  int n = 0;
  GemvArgs a{};
  a.b = b;
  a.resident = &n;
  if (alds) launch_stream<true>(p, dim3(1), a);
  else launch_stream<false>(p, dim3(1), a);
  (void)hipGetLastError();  // a failed query leaves no error behind
  std::lock_guard<std::mutex> lock(mu);
  cache[key] = n;
  return n;
}
}  // namespace

hipError_t launch_gemv_prepare(const float *xr, int64_t b, int64_t K, void *workspace,
                               hipStream_t stream) {
  const GemvWs w = carve(workspace, b, K);
  (void)hipGetLastError();  // drop errors left by earlier, unrelated runtime calls
  hipLaunchKernelGGL(gemv_prep_kernel, dim3(unsigned(b * limb_blocks(K))), dim3(64), 0, stream, xr, K,
                     w.Kp, int(b), w.xhi, w.sigma);
  set_last_kernel("gemv_prep_limbs");
  return hipGetLastError();
}

hipError_t launch_gemv_prepare_rotated(const uint16_t *x, int64_t b, int64_t K, const int8_t *signs,
                                       void *workspace, hipStream_t stream) {
  const GemvWs w = carve(workspace, b, K);
  return launch_gemv_prepare_x(x, b, K, signs, w.xhi, w.Kp, w.sigma, stream);
}

hipError_t launch_gemv_main(const void *workspace, int64_t b, int64_t K, int64_t N,
                            const uint32_t *packed, const uint16_t *scales, void *y, int y_dtype,
                            hipStream_t stream) {
  const GemvWs w = carve(const_cast<void *>(workspace), b, K);
  const GemvPlan p = plan_gemv(b, K, N);
  if (!p.ok) return hipErrorInvalidValue;
  const dim3 grid(unsigned((N + 16 * p.rb - 1) / (16 * p.rb)), unsigned(p.chunks));
  const GemvArgs a{&w, b, K, N, packed, scales, y, y_dtype, stream};
  (void)hipGetLastError();  // drop errors left by earlier, unrelated runtime calls
  if (p.kind == 0) launch_stream<true>(p, grid, a);
  else if (p.kind == 1) launch_stream<false>(p, grid, a);
  else if (p.rb == 2) launch_ring_r<2>(p, grid, a);
  else launch_ring_r<1>(p, grid, a);
  set_last_kernel(p.name);
  return hipGetLastError();
}

// The one-launch path trades redundant rotations (every workgroup rotates every
// block of every token) for one launch fewer and no limb round trip, so it is
// ahead while the workgroups and the rotations per wave are few.  Measured
// against the fused prep + GEMV pair (back-to-back launches over rotating weight
// copies, us, one launch vs two):
//  * one token: ahead at every K <= 6144 and N <= 12288 but one (K = 5120:
//    5.8 vs 6.9 at N = 1024, 9.1 vs 9.4 at 10240, 9.3 vs 9.4 at 12288; K = 6144:
//    7.6 vs 9.3 at N = 8192, behind at 12288, 10.8 vs 10.4), and behind at
//    N = 34816;
//  * two tokens: ahead while K <= 4096 (K = 2048: 5.5 vs 6.5 at N = 1024, 6.7 vs
//    7.3 at 6144; K = 4096: 6.4 vs 6.8 at 1024, 7.8 vs 7.9 at 6144), behind from
//    K = 5120 on (7.9 vs 7.1 at N = 1024, 9.4 vs 8.3 at 5120).
bool gemv_rot_supported(int64_t b, int64_t K, int64_t N) {
  if (K <= 0 || K % kHBlock || K / kHBlock > kRotMaxBlocks) return false;
  if (b == 1) return N <= 12288 && (K <= 5120 || N <= 8192);
  return b == 2 && N <= 6144 && K <= 4096;
}

hipError_t launch_gemv_rot(const uint16_t *x, int64_t b, int64_t K, int64_t N, const int8_t *signs,
                           const uint32_t *packed, const uint16_t *scales, void *y, int y_dtype,
                           hipStream_t stream) {
  if (!gemv_rot_supported(b, K, N)) return hipErrorInvalidValue;
  const int nblk = int(K / kHBlock);
  const bool two_rb = N > 4096;  // 16 or 32 rows per workgroup: at most 256 or 384 workgroups
  (void)hipGetLastError();  // drop errors left by earlier, unrelated runtime calls
  if (b == 1) {
    if (two_rb) launch_rot_t<2, 1>(nblk, x, signs, K, N, packed, scales, y, y_dtype, stream);
    else launch_rot_t<1, 1>(nblk, x, signs, K, N, packed, scales, y, y_dtype, stream);
  } else {
    if (two_rb) launch_rot_t<2, 2>(nblk, x, signs, K, N, packed, scales, y, y_dtype, stream);
    else launch_rot_t<1, 2>(nblk, x, signs, K, N, packed, scales, y, y_dtype, stream);
  }
  static const char *names[2][2] = {{"gemv_rot_rb1_b1", "gemv_rot_rb1_b2"}, {"gemv_rot_rb2_b1", "gemv_rot_rb2_b2"}};
  set_last_kernel(names[two_rb][b - 1]);
  return hipGetLastError();
}

bool gemv_q8_supported(int64_t b, int64_t K, int64_t N) { return plan_q8(b, K, N).ok; }

hipError_t launch_gemv_q8(const int8_t *xq, const float *tok_scale, int64_t b, int64_t K, int64_t N,
                          const uint32_t *packed, const uint16_t *scales, void *y, int y_dtype,
                          hipStream_t stream) {
  const Q8Plan p = plan_q8(b, K, N);
  if (!p.ok) return hipErrorInvalidValue;
  const Q8Args a{xq, tok_scale, b, K, N, packed, scales, y, y_dtype, stream};
  (void)hipGetLastError();  // drop errors left by earlier, unrelated runtime calls
  if (p.alds) {
    if (p.rb == 2) launch_q8_n<2, true>(p, a); else launch_q8_n<1, true>(p, a);
  } else {
    if (p.rb == 2) launch_q8_n<2, false>(p, a); else launch_q8_n<1, false>(p, a);
  }
  set_last_kernel(p.name);
  return hipGetLastError();
}

}  // namespace tl
