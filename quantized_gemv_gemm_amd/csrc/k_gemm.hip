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
// 128 int32 accumulators per lane), so every expanded weight fragment feeds four
// MFMAs.  The K loop steps one pair of 128-wide scale groups (8 MFMA k-steps).
//
// Pipeline: two workgroups share each compute unit (256 registers per lane
// each), so that one's stalls are covered by the other's MFMAs:
//  * the activation tile of pair p+1 is loaded straight into the second of two
//    LDS buffers (buffer loads with the LDS destination, 1 KB per instruction)
//    while pair p is computed from the first; rows are unpadded and each 16-byte
//    chunk c of row r sits at c ^ (r % 16), so the fragment reads of 16 rows
//    hit 16 different bank groups; the reads are issued by hand with their own
//    waits (the compiler would otherwise wait for every load before them);
//  * packed weight words arrive in a two-deep register ring, loaded straight
//    from the 1 KB packed tiles (two 16-byte loads per column per pair);
//  * the LDS reads of k-step s+1 are issued between the MFMAs of k-step s, and
//    the codes are expanded column by column: while the MFMAs of weight column j
//    run, column j+1 (or column 0 of the next k-step) is expanded into registers
//    whose readers have all been issued; there is one barrier per pair;
//  * the tile's row scales wait in LDS for the epilogue, so that no register is
//    held for them through the K loop.
// The expansion code -> code*q is one v_perm_b32 per 4 weights: the selector
// bytes are the 2-bit fields ((w >> 2r) & 0x03030303) and the table holds
// {0, q, -, -q}.
//
// Work distribution: the tiles are dealt out in whole rounds of workgroups (two
// per compute unit), each round XCD-aware so that the M-blocks of a
// weight strip run on one XCD and share its L2.  The tiles left over for a last,
// partial round are either
//  * cut into eight 32 x 128 sub-tiles (when at most 256 / 8 are left), each a
//    workgroup of its own over the whole K: the same pipeline with one 32 x 32
//    MFMA tile per wave; nothing to add up afterwards; or
//  * split along K into S pieces; every piece stores its int32 partial tile to
//    the workspace and bumps the tile's counter, and the piece that arrives last
//    adds the others and runs the epilogue (integer sums: exact and order
//    independent).
// The left-over work is dealt out XCD by XCD (workgroup i runs on XCD i % 8), so
// that the pieces or sub-tiles of one weight strip share an L2.
// With fewer than 512 tiles of 128 x 256 (fewer than two per compute unit), the
// problem takes 128 x 128 tiles (each wave 128 x 32) on the two-per-CU pipeline
// instead: whole rounds of 512, the rest split along K into at most 6 pieces.
// No workgroup ever waits for another.
//
// Issue priority: when the whole grid is resident at once, the waves raise
// their priority (s_setprio) for the middle k-steps of each pair, so that the
// two workgroups of a compute unit progress evenly; the left-over work at the
// end of a longer grid does the same (see gemm_i8_kernel).  Whole tiles store
// their output non-temporally.
#include <algorithm>

#include "tl_device.h"

namespace tl {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kPairK = 2 * kGroup;        // k per pipeline stage: one pair of groups
constexpr int kSlots = 256;               // the compute units of gfx950
constexpr int kXcds = 8;                  // workgroup i runs on XCD i % 8
constexpr int kMaxSplit = 6;

// A workgroup tile of 32 MT x 128 J: each of the 4 waves owns all 32 MT rows and
// 32 J columns (MT x J MFMA tiles of 32 x 32).
template <int MT, int J>
struct Tile {
  static constexpr int BM = 32 * MT, BN = 4 * 32 * J;
  static constexpr int Ints = BM * BN;
};
typedef Tile<4, 2> Big;     // 128 x 256: the tile of the whole rounds
typedef Tile<1, 1> Narrow;  // 32 x 128: an eighth of a big tile, for a short last round
typedef Tile<4, 1> Mid;     // 128 x 128: the tile of problems with fewer big tiles than CUs
constexpr int kBM = Big::BM;
constexpr int kBN = Big::BN;
constexpr int kTileInts = Big::Ints;
constexpr int kNarrowPerTile = (Big::BM / Narrow::BM) * (Big::BN / Narrow::BN);
// Two workgroups per compute unit (256 registers per lane each): two activation
// stages of 128 rows x 256 bytes loaded straight into LDS, weights in a two-deep
// register ring, the K loop in turns of two pairs.  The LDS block also serves as
// the epilogue's staging room (128 rows of 256 bf16 values and a 16-byte pad per
// row, written in one pass).
constexpr int kStageLds = 2 * kBM * (kPairK + 16);
constexpr int kWgPerCu = 2;
constexpr int kTurn = 2;  // pairs per ring turn (the K loop pads to it)

static_assert(kTileInts == kThreads * 128, "128 accumulators per thread");

template <int J>
struct BStage {
  v4u w[J][2];  // [N tile][lane quarter 2h, 2h+1]: tile words for both groups of the pair
  int q[J][2];  // [N tile][group of the pair], as loaded
  uint32_t keep[2];  // per group of the pair: all ones, or 0 for a padding pair / missing group
};

struct Schedule {
  int mb;         // M-blocks
  int tiles;      // MB * N-strips
  int round;      // workgroups per whole round: two per compute unit
  int full;       // tiles computed whole, in whole rounds (the rest are split or cut)
  int split;      // pieces per left-over tile along K (1: nothing is split)
  int narrow;     // 1: the left-over tiles are cut into kNarrowPerTile sub-tiles
  int mid;        // 1: every tile is a Mid tile (mb, tiles count Mid tiles), split `split` ways
  __host__ __device__ int64_t left() const { return split > 1 || narrow || mid ? tiles - full : 0; }
  __host__ __device__ int64_t grid() const { return full + left() * (narrow ? kNarrowPerTile : split); }
};

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

// Per-thread addressing, fixed for the whole tile.  All global reads go through
// buffer resources that cover exactly the tile's rows of xq, its packed row
// blocks and its q rows: a read past M, past N or past the last group returns
// zeros, which only ever meets zero weights or results that are not stored.
template <int J>
struct Frame {
  __amdgpu_buffer_rsrc_t ra, rb, rq;
  int boff[J];    // this lane's 16 bytes of the first tile of its weight column, per N tile
  int qoff[J];    // q row of that column
  int G;
};

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9)
constexpr int kCoherent = 16;           // cache policy sc1: coherent across the XCDs' L2s

template <int J>
__device__ __forceinline__ void load_b(BStage<J> &b, const Frame<J> &f, int p, bool live) {
#pragma unroll
  for (int j = 0; j < J; ++j) {
    b.w[j][0] = __builtin_amdgcn_raw_buffer_load_b128(f.rb, f.boff[j], p * 1024, 0);
    b.w[j][1] = __builtin_amdgcn_raw_buffer_load_b128(f.rb, f.boff[j] + 256, p * 1024, 0);
    b.q[j][0] = (int8_t)__builtin_amdgcn_raw_buffer_load_b8(f.rq, f.qoff[j], 2 * p, 0);
    b.q[j][1] = (int8_t)__builtin_amdgcn_raw_buffer_load_b8(f.rq, f.qoff[j] + 1, 2 * p, 0);
  }
  // a padding pair (live == false) and the missing half of a last odd pair expand
  // to zero weights; the mask is applied at expansion so that no instruction here
  // waits for the loads
  b.keep[0] = live ? ~0u : 0u;
  b.keep[1] = live && 2 * p + 1 < f.G ? ~0u : 0u;
}

// k-step s (0..7) of a pair: group gi = s / 4, sub-step ss = s % 4.  Word 4h + ss
// of the lane's column in group gi: words 4h, 4h+1 sit in the lane-quarter 2h slot
// of the tile, 4h+2, 4h+3 in the 2h+1 slot.
template <int J>
__device__ __forceinline__ void fetch_b(v4i (&bf)[J], const BStage<J> &b, int s) {
  const int gi = s >> 2, ss = s & 3;
#pragma unroll
  for (int j = 0; j < J; ++j)
    bf[j] = expand_word(b.w[j][ss >> 1][2 * gi + (ss & 1)], perm_table(b.q[j][gi]) & b.keep[gi]);
}

// column j only: the fragment of k-step s for the lane's j-th weight column
template <int J>
__device__ __forceinline__ v4i fetch_col(const BStage<J> &b, int s, int j) {
  const int gi = s >> 2, ss = s & 3;
  return expand_word(b.w[j][ss >> 1][2 * gi + (ss & 1)], perm_table(b.q[j][gi]) & b.keep[gi]);
}

template <int MT, int J>
__device__ __forceinline__ void mfma_step(const v4i (&af)[MT], const v4i (&bf)[J], v16i (&acc)[MT][J]) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < J; ++j)
      acc[mt][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[mt], bf[j], acc[mt][j], 0, 0, 0);
}

typedef float v4f __attribute__((ext_vector_type(4)));

// y = fl32(fl32(acc) * row_scale[n]) * tok_scale[m].  The lane holds column l32 of
// each 32x32 tile, rows 8*(r/4) + 4*h + r%4: four consecutive rows per r/4, whose
// token scales come from LDS in one 16-byte read.  A tile that lies inside
// [M, N] takes the variant without per-element bounds tests.
template <bool kCheck, bool kF32, bool kAcc, int MT, int J>
__device__ __forceinline__ void epilogue(const v16i (&acc)[MT][J], const float *s_tok,
                                         const float (&rsv)[J], int64_t m0, int64_t n0, int64_t M,
                                         int64_t N, int wave, int l32, int h, void *y,
                                         int32_t *acc_out) {
  // the lane's first row (4 h) and column; element (r, 32 j) away sits r N + 32 j
  // further, a uniform offset, so that only the two base pointers are per lane
  const int64_t mb = m0 + 4 * h, nb = n0 + 32 * J * wave + l32;
  char *yb = static_cast<char *>(y) + (mb * N + nb) * (kF32 ? 4 : 2);
  int32_t *ab = kAcc ? acc_out + (mb * N + nb) : nullptr;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (kCheck && nb + 32 * j >= N) continue;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const v4f ts = *reinterpret_cast<const v4f *>(s_tok + 32 * mt + 8 * rq + 4 * h);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 32 * mt + 8 * rq + i;
          if (kCheck && mb + r >= M) continue;
          const int a = acc[mt][j][4 * rq + i];
          const float v = ((float)a * rsv[j]) * ts[i];
          const int64_t off = int64_t(r) * N + 32 * j;
          if (kAcc) ab[off] = a;
          if (kF32)
            reinterpret_cast<float *>(yb)[off] = v;
          else
            reinterpret_cast<uint16_t *>(yb)[off] = float_to_bf16_bits(v);
        }
        // one group of four rows at a time: keeps the live values within the
        // register budget of the two-per-CU pipeline
        __builtin_amdgcn_sched_barrier(0);
      }
  }
}

// The same values for a tile that lies inside [M, N], staged through LDS (the
// activation buffers, free once the K loop is done) so that every lane stores 16
// contiguous bytes of a row -- a wave writes whole rows -- instead of 2- or
// 4-byte pieces down a column.  f32 output goes in two passes of 64 rows.
template <bool kF32, int MT, int J, int kStageCap>
__device__ __forceinline__ void epilogue_lds(const v16i (&acc)[MT][J], const float *s_tok,
                                             const float (&rsv)[J], int64_t m0, int64_t n0, int64_t N,
                                             int wave, int l32, int h, int tid, void *y, int8_t *stage) {
  constexpr int BM = Tile<MT, J>::BM, BN = Tile<MT, J>::BN;
  constexpr int ES = kF32 ? 4 : 2;         // bytes per output
  constexpr int PITCH = BN * ES + 16;      // LDS row pitch (the pad spreads the 4-row steps over banks)
  constexpr int ROWS = BM * PITCH <= kStageCap ? BM : BM / 2;  // rows per pass
  constexpr int CPR = BN * ES / 16;        // 16-byte chunks per row
  static_assert(ROWS * PITCH <= kStageCap, "staging fits the activation buffers");
  __syncthreads();  // every wave is done with the activation buffers
#pragma unroll
  for (int pass = 0; pass < BM / ROWS; ++pass) {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int c = 32 * J * wave + 32 * j + l32;
#pragma unroll
      for (int mt = pass * (ROWS / 32); mt < (pass + 1) * (ROWS / 32); ++mt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int row = 32 * mt + 8 * rq + 4 * h;
          const v4f ts = *reinterpret_cast<const v4f *>(s_tok + row);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = ((float)acc[mt][j][4 * rq + i] * rsv[j]) * ts[i];
            int8_t *dst = stage + (row + i - pass * ROWS) * PITCH + c * ES;
            if (kF32)
              *reinterpret_cast<float *>(dst) = v;
            else
              *reinterpret_cast<uint16_t *>(dst) = float_to_bf16_bits(v);
          }
        }
    }
    __syncthreads();
    char *ybase = static_cast<char *>(y) + ((m0 + pass * ROWS) * N + n0) * ES;
#pragma unroll
    for (int k = tid; k < ROWS * CPR; k += kThreads) {
      const int r = k / CPR, cc = k - r * CPR;
      // non-temporal: the output is not read again by this launch
      __builtin_nontemporal_store(*reinterpret_cast<const v4u *>(stage + r * PITCH + 16 * cc),
                                  reinterpret_cast<v4u *>(ybase + (int64_t(r) * N) * ES + 16 * cc));
    }
    if (pass + 1 < BM / ROWS) __syncthreads();  // the next pass overwrites the staging rows
  }
}

// With at least 512 tiles of 128 x 256 (two per compute unit) the big tiles run
// in whole rounds of 512 and the left-over tiles are cut or split so that the
// last round is at most one workgroup per CU.  With fewer, the problem takes
// 128 x 128 tiles instead, also two per CU: twice the workgroups, and, when the
// left-over ones are split along K, S partial tiles of half the size.
inline Schedule make_schedule(int64_t M, int64_t N, int64_t GP) {
  Schedule sc;
  sc.mb = int((M + kBM - 1) / kBM);
  sc.tiles = sc.mb * int((N + kBN - 1) / kBN);
  sc.mid = 0;
  if (sc.tiles < 2 * kSlots) {
    // Mid tiles: whole rounds of 512 workgroups (two per CU), the rest split
    // along K into S pieces (S x rest <= 512).  S by a cost in pair-steps fitted
    // to measurements: the longest piece (padded to an even pair count) at 0.9
    // per pair when every workgroup has a CU to itself, 2.0 when some CUs hold
    // two, plus one per extra piece (its partial tile read back by the last
    // piece); ties go to fewer pieces.
    const int mmb = int((M + Mid::BM - 1) / Mid::BM);
    const int mtiles = mmb * int((N + Mid::BN - 1) / Mid::BN);
    const int full = mtiles / (2 * kSlots) * (2 * kSlots);
    const int left = mtiles - full;
    int S = 1;
    double best = 1e30;
    for (int s = 1; left && s <= kMaxSplit && s * left <= 2 * kSlots && s <= GP; ++s) {
      const int64_t piece = (GP + s - 1) / s;
      const double cost = double(piece + (piece & 1)) * (s * left > kSlots ? 2.0 : 0.9) + (s - 1);
      if (cost < best - 1e-9) best = cost, S = s;
    }
    sc.mid = 1;
    sc.round = 2 * kSlots;
    sc.mb = mmb;
    sc.tiles = mtiles;
    sc.split = S;
    sc.full = S > 1 ? full : mtiles;
    sc.narrow = 0;
    return sc;
  }
  sc.round = 2 * kSlots;
  const int turn = kTurn;
  sc.narrow = 0;
  const int left = sc.tiles % sc.round;
  int best = 1;
  if (left && left * kNarrowPerTile <= kSlots) {
    // a short last round: every left-over tile becomes eight sub-tile workgroups
    sc.narrow = 1;
    sc.split = 1;
    sc.full = sc.tiles - left;
    return sc;
  }
  if (left) {
    int64_t best_cost = (GP + turn - 1) / turn * turn;
    for (int S = 2; S <= kMaxSplit && S * left <= kSlots && S <= GP; ++S) {
      const int64_t piece = (GP + S - 1) / S;
      const int64_t cost = (piece + turn - 1) / turn * turn + (S - 1);
      if (cost < best_cost) best_cost = cost, best = S;
    }
  }
  sc.split = best;
  sc.full = best > 1 ? sc.tiles - left : sc.tiles;
  return sc;
}

struct GemmArgs {
  const int8_t *xq;
  const float *tok_scale;
  int64_t M, K, N;
  const uint32_t *packed;
  const int8_t *q;
  const float *row_scale;
  void *y;
  int y_dtype;
  int32_t *acc_out, *part, *counters;
};

// ---------------------------------------------------------------------------
// two-stage pipeline with activation stages loaded straight into LDS
// ---------------------------------------------------------------------------
// Stage layout: rows of 256 bytes, no padding; 16-byte chunk c of row r sits at
// physical chunk c ^ (r & 15), so that 16 consecutive rows reading the same chunk
// hit 16 different bank groups.
__device__ __forceinline__ v4i lds_read16(uint32_t addr) {
  v4i r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}

template <int MT>
__device__ __forceinline__ void read_a2(v4i (&af)[MT], uint32_t rowaddr, int xsw, int h, int s) {
  const int c = 8 * (s >> 2) + (s & 3) + 4 * h;
  const uint32_t a = rowaddr + 16 * uint32_t(c ^ xsw);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) af[mt] = lds_read16(a + 32 * 256 * mt);
}

template <int MT, int N>
__device__ __forceinline__ void wait_a2(v4i (&af)[MT]) {
  if constexpr (MT == 4)
    asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(af[0]), "+v"(af[1]), "+v"(af[2]), "+v"(af[3]) : "n"(N));
  else if constexpr (MT == 2)
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(af[0]), "+v"(af[1]) : "n"(N));
  else
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(af[0]) : "n"(N));
}

// the activation stage of pair p into LDS buffer buf: instruction j = wave + 4 i
// covers rows 4 j .. 4 j + 3; lane l takes row 4 j + l / 16 and logical chunk
// (l % 16) ^ (row % 16), the row's bytes at physical chunk l % 16
template <int MT, int J>
__device__ __forceinline__ void dma_a2(const Frame<J> &f, int8_t *buf, int p, int wave, int dvoff,
                                       int64_t K) {
#if __HIP_DEVICE_COMPILE__
#pragma unroll
  for (int i = 0; i < 2 * MT; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        f.ra, (__attribute__((address_space(3))) void *)(buf + 1024 * (wave + 4 * i)), 16,
        dvoff + int(16 * K) * i, p * kPairK, 0, 0);
#endif
}

template <int S, int MT, int J, bool kPrio>
__device__ __forceinline__ void pair_body2(int p, int k0, int plast, const Frame<J> &f, int8_t *sA,
                                           uint32_t rowaddr, int xsw, int h, int wave, int dvoff, int64_t K,
                                           BStage<J> (&ring)[2], v4i (&af)[2][MT], v4i (&bf)[2][J],
                                           v16i (&acc)[MT][J]) {
  constexpr int AB = Tile<MT, J>::BM * 256;
  // the pair boundary (stage loads, first operand reads, the barrier) runs at the
  // normal issue priority, the middle k-steps at the raised one (kPrio)
  if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
  // the next pair's stage into the other buffer (every wave left it at the last barrier)
  dma_a2<MT, J>(f, sA + (S ^ 1) * AB, min(max(p + 1, k0), plast), wave, dvoff, K);
  const uint32_t cur = rowaddr + S * AB;
  read_a2<MT>(af[0], cur, xsw, h, 0);
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    if (s < 7) {
      read_a2<MT>(af[(s + 1) & 1], cur, xsw, h, s + 1);
      wait_a2<MT, MT>(af[s & 1]);
    } else {
      wait_a2<MT, 0>(af[s & 1]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (J >= 2) {
      // column by column: the MFMAs of column j read fragment j of this k-step
      // while the next fragment (column j + 1, or column 0 of the next k-step)
      // is expanded into the registers whose readers have all been issued
#pragma unroll
      for (int j = 0; j < J; ++j) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[s & 1][mt], bf[0][j], acc[mt][j], 0, 0, 0);
        if (j + 1 < J)
          bf[0][j + 1] = fetch_col(ring[S], s, j + 1);
        else if (s < 7)
          bf[0][0] = fetch_col(ring[S], s + 1, 0);
        else
          bf[0][0] = fetch_col(ring[S ^ 1], 0, 0);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // up to three VALU
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      mfma_step(af[s & 1], bf[s & 1], acc);
      if (s < 7)
        fetch_b(bf[(s + 1) & 1], ring[S], s + 1);
      else
        fetch_b(bf[0], ring[S ^ 1], 0);
#pragma unroll
      for (int i = 0; i < MT * J; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // up to four VALU
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kPrio && s == 0) __builtin_amdgcn_s_setprio(1);
    if (s == 7) {
      if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
      load_b(ring[S], f, min(max(p + 2, k0), plast), p + 2 >= k0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // this wave's stage loads are done (the weight loads just issued may stay in flight)
  __builtin_amdgcn_s_waitcnt(0x0F70 & ~0x0F | (4 * J));
  __syncthreads();
}

// One workgroup tile of 32 MT x 128 J at (m0, n0) over the pairs [k0, k1).  A
// piece of a K-split tile (piece >= 0) publishes its partial tile and only the
// last piece to arrive runs the epilogue.  kPrio: the middle k-steps of each pair
// run at a raised issue priority (see gemm_i8_kernel).
template <int MT, int J, bool kPrio>
__device__ __forceinline__ void run_tile(const GemmArgs &a, const Schedule &sc, int8_t *sA, float *s_tok,
                                         int *s_last, int64_t m0, int64_t n0, int k0, int k1, int tile,
                                         int piece, int slot) {
  typedef Tile<MT, J> T;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int64_t M = a.M, K = a.K, N = a.N;
  const int G = int(K / kGroup);
  const int GP = (G + 1) / 2;

  Frame<J> f;
  f.G = G;
  {
    const int64_t rows = M - m0 < T::BM ? M - m0 : T::BM;
    f.ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(a.xq + m0 * K), (short)0,
                                             int(rows * K), kRsrcWord3);
    const int64_t NB = (N + 15) / 16, rb0 = n0 / 16;
    const int64_t blocks = NB - rb0 < T::BN / 16 ? NB - rb0 : T::BN / 16;
    f.rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t *>(a.packed + 256 * rb0 * GP), (short)0,
                                             int(blocks * GP * 1024), kRsrcWord3);
    const int64_t cols = N - n0 < T::BN ? N - n0 : T::BN;
    f.rq = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(a.q + n0 * G), (short)0, int(cols * G),
                                             kRsrcWord3);
  }
  // token scales of the tile's rows (LDS, read in the epilogue) and this lane's row scales
  if (tid < T::BM) s_tok[tid] = a.tok_scale[m0 + tid < M ? m0 + tid : M - 1];
  // row scales of the tile's columns: LDS until the epilogue (no registers held
  // through the K loop)
  float *s_rsv = s_tok + kBM;
  if (tid < T::BN) s_rsv[tid] = a.row_scale[n0 + tid < N ? n0 + tid : N - 1];
  // weight columns of this lane: one per 32-wide N tile, read from the packed tiles
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = 32 * J * wave + 32 * j + l32;     // column inside the tile
    f.boff[j] = (c >> 4) * GP * 1024 + 16 * (32 * h + (c & 15));
    f.qoff[j] = c * G;
  }

  v16i acc[MT][J];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][j][r] = 0;

  // two LDS stages filled straight from memory, two weight slots; an even pair
  // count (a leading zero-weight pair when odd)
  const int p0 = k0 - ((k1 - k0) & 1);
  const int plast = k1 - 1;
  BStage<J> ring[2];
  load_b(ring[0], f, min(max(p0, k0), plast), p0 >= k0);
  load_b(ring[1], f, min(max(p0 + 1, k0), plast), p0 + 1 >= k0);
  // DMA source offset of this lane: row 4 wave + lane / 16 (+ 16 i), logical chunk
  const int rbase = 4 * wave + (lane >> 4);
  const int dvoff = int(rbase * K) + 16 * ((lane & 15) ^ (rbase & 15));
  dma_a2<MT, J>(f, sA, min(max(p0, k0), plast), wave, dvoff, K);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  const uint32_t rowaddr = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) int8_t *)sA + 256 * l32;
  const int xsw = l32 & 15;
  v4i af[2][MT], bf[2][J];
  if constexpr (J >= 2)
    bf[0][0] = fetch_col(ring[0], 0, 0);  // the other columns are expanded inside the loop
  else
    fetch_b(bf[0], ring[0], 0);
  for (int p = p0; p < k1; p += 2) {
    pair_body2<0, MT, J, kPrio>(p, k0, plast, f, sA, rowaddr, xsw, h, wave, dvoff, K, ring, af, bf, acc);
    pair_body2<1, MT, J, kPrio>(p + 1, k0, plast, f, sA, rowaddr, xsw, h, wave, dvoff, K, ring, af, bf, acc);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load outlives the loop
  if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);

  if (piece >= 0) {
    // Split tile: publish this piece, and only the last piece to arrive goes on.
    // Partials are written and read with device-scope atomic accesses (written
    // through to, and read from, the point where all XCDs are coherent), so no
    // whole-L2 fence is needed: the stores are waited for before the counter is
    // bumped, and the reads are issued after the counter has answered.
    // 16-byte pieces: piece (mt, j, r / 4) of thread tid at ((mt * J + j) * 4 + r / 4) * kThreads + tid,
    // written and read with the system-coherent cache policy (sc1), like the
    // device-scope atomic accesses, four elements per instruction
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        a.part + int64_t(slot - piece) * T::Ints, (short)0, int(sc.split * T::Ints * 4), kRsrcWord3);
    const int mine = piece * T::Ints * 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < J; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const v4i v = {acc[mt][j][4 * r4], acc[mt][j][4 * r4 + 1], acc[mt][j][4 * r4 + 2], acc[mt][j][4 * r4 + 3]};
          __builtin_amdgcn_raw_buffer_store_b128((v4u)v, rp, mine + 16 * (((mt * J + j) * 4 + r4) * kThreads + tid), 0,
                                                 kCoherent);
        }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): every partial store has completed
    __syncthreads();
    if (tid == 0) {
      const int old = __hip_atomic_fetch_add(&a.counters[tile - sc.full], 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
      *s_last = old == sc.split - 1;
    }
    __syncthreads();
    if (!*s_last) return;
    for (int o = 0; o < sc.split; ++o) {
      if (o == piece) continue;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const v4u v = __builtin_amdgcn_raw_buffer_load_b128(
                rp, o * T::Ints * 4 + 16 * (((mt * J + j) * 4 + r4) * kThreads + tid), 0, kCoherent);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[mt][j][4 * r4 + e] += (int)v[e];
          }
    }
    if (tid == 0)  // leave the workspace as it was found
      __hip_atomic_store(&a.counters[tile - sc.full], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  float rsv[J];
#pragma unroll
  for (int j = 0; j < J; ++j) rsv[j] = s_rsv[32 * J * wave + 32 * j + l32];
  const bool whole = m0 + T::BM <= M && n0 + T::BN <= N;
  if (whole && !a.acc_out && N % 8 == 0) {  // rows of y start on 16-byte boundaries
    if (a.y_dtype == TL_F32) epilogue_lds<true, MT, J, kStageLds>(acc, s_tok, rsv, m0, n0, N, wave, l32, h, tid, a.y, sA);
    else epilogue_lds<false, MT, J, kStageLds>(acc, s_tok, rsv, m0, n0, N, wave, l32, h, tid, a.y, sA);
    return;
  }
  // variants with and without the exact accumulators, so that no store sits
  // behind a per-element branch (edge tiles, and rows not 16-byte aligned, check bounds)
  const bool f32 = a.y_dtype == TL_F32;
  if (a.acc_out) {
    if (f32) {
      if (whole) epilogue<false, true, true>(acc, s_tok, rsv, m0, n0, M, N, wave, l32, h, a.y, a.acc_out);
      else epilogue<true, true, true>(acc, s_tok, rsv, m0, n0, M, N, wave, l32, h, a.y, a.acc_out);
    } else {
      if (whole) epilogue<false, false, true>(acc, s_tok, rsv, m0, n0, M, N, wave, l32, h, a.y, a.acc_out);
      else epilogue<true, false, true>(acc, s_tok, rsv, m0, n0, M, N, wave, l32, h, a.y, a.acc_out);
    }
  } else {
    if (f32) epilogue<true, true, false>(acc, s_tok, rsv, m0, n0, M, N, wave, l32, h, a.y, nullptr);
    else epilogue<true, false, false>(acc, s_tok, rsv, m0, n0, M, N, wave, l32, h, a.y, nullptr);
  }
}

// Work item of left-over workgroup e of `total`: workgroup e runs on XCD e % kXcds,
// so the items are dealt out XCD by XCD, each XCD taking a contiguous run (the
// pieces or sub-tiles of neighbouring tiles share weight strips and so its L2).
__device__ __forceinline__ int xcd_item(int e, int total) {
  if (total % kXcds) return e;
  return (total / kXcds) * (e % kXcds) + e / kXcds;
}

// kPrio (the host sets it when the whole grid is resident at once, two
// workgroups per CU): a wave raises its issue priority for the middle k-steps of
// each pair and drops it for the pair boundary, so a workgroup at its boundary
// yields the SIMDs to the other workgroup of its CU, and the two progress evenly
// instead of the older one finishing first.  When more workgroups follow, the
// whole tiles of the first rounds keep the uneven progress (the first to finish
// hands its slot on early); the left-over work that comes last in the grid (K
// pieces, sub-tiles) always raises it.
template <bool kPrio>
__global__ __launch_bounds__(kThreads, kWgPerCu) void gemm_i8_kernel(
    const int8_t *__restrict__ xq, const float *__restrict__ tok_scale, int64_t M, int64_t K,
    int64_t N, const uint32_t *__restrict__ packed, const int8_t *__restrict__ q,
    const float *__restrict__ row_scale, void *__restrict__ y, int y_dtype,
    int32_t *__restrict__ acc_out, int32_t *__restrict__ part, int32_t *__restrict__ counters,
    Schedule sc) {
  __shared__ __attribute__((aligned(16))) int8_t sA[kStageLds];
  __shared__ __attribute__((aligned(16))) float s_tok[kBM + kBN];  // token scales, then row scales
  __shared__ int s_last;
  const GemmArgs a{xq, tok_scale, M, K, N, packed, q, row_scale, y, y_dtype, acc_out, part, counters};
  const int GP = int((K / kGroup + 1) / 2);

  // which tile and which K range this workgroup computes
  const int g = blockIdx.x;
  if (sc.mid) {
    int tile, piece = -1, e = 0, k0 = 0, k1 = GP;
    if (g < sc.full) {
      // whole Mid tiles in rounds, the M-blocks of a strip on one XCD
      const int round = g / sc.round, u = g % sc.round;
      tile = (sc.round % kXcds == 0 && sc.full - round * sc.round >= sc.round)
                 ? round * sc.round + (sc.round / kXcds) * (u % kXcds) + u / kXcds
                 : g;
    } else {
      // left-over Mid tile full + e / S, K piece e % S (no piece when S = 1)
      e = xcd_item(g - sc.full, int(sc.grid() - sc.full));
      const int S = sc.split;
      tile = sc.full + e / S;
      piece = S > 1 ? e % S : -1;
      k0 = S > 1 ? int(int64_t(GP) * piece / S) : 0;
      k1 = S > 1 ? int(int64_t(GP) * (piece + 1) / S) : GP;
    }
    const int64_t m0 = int64_t(tile % sc.mb) * Mid::BM;
    const int64_t n0 = int64_t(tile / sc.mb) * Mid::BN;
    if (kPrio || g >= sc.full)
      run_tile<Mid::BM / 32, Mid::BN / 128, true>(a, sc, sA, s_tok, &s_last, m0, n0, k0, k1, tile, piece, e);
    else
      run_tile<Mid::BM / 32, Mid::BN / 128, false>(a, sc, sA, s_tok, &s_last, m0, n0, k0, k1, tile, piece, e);
    return;
  }
  if (g >= sc.full && sc.narrow) {
    // sub-tile u of a left-over tile: rows 32 (u % 4), columns 128 (u / 4) of it
    const int e = xcd_item(g - sc.full, int(sc.grid() - sc.full));
    const int tile = sc.full + e / kNarrowPerTile, u = e % kNarrowPerTile;
    constexpr int kRowCuts = Big::BM / Narrow::BM;
    const int64_t m0 = int64_t(tile % sc.mb) * kBM + Narrow::BM * (u % kRowCuts);
    const int64_t n0 = int64_t(tile / sc.mb) * kBN + Narrow::BN * (u / kRowCuts);
    if (m0 >= M || n0 >= N) return;  // the whole sub-tile lies past the output
    run_tile<Narrow::BM / 32, Narrow::BN / 128, true>(a, sc, sA, s_tok, &s_last, m0, n0, 0, GP, tile, -1, 0);
    return;
  }
  int tile, piece = -1, slot = 0, k0 = 0, k1 = GP;
  if (g < sc.full) {
    const int round = g / sc.round, u = g % sc.round;
    tile = (sc.round % kXcds == 0 && sc.full - round * sc.round >= sc.round)
               ? round * sc.round + (sc.round / kXcds) * (u % kXcds) + u / kXcds
               : g;
  } else {
    slot = xcd_item(g - sc.full, int(sc.grid() - sc.full));
    tile = sc.full + slot / sc.split;
    piece = slot % sc.split;
    k0 = int(int64_t(GP) * piece / sc.split);
    k1 = int(int64_t(GP) * (piece + 1) / sc.split);
  }
  const int64_t m0 = int64_t(tile % sc.mb) * kBM;
  const int64_t n0 = int64_t(tile / sc.mb) * kBN;
  if (kPrio || g >= sc.full)
    run_tile<Big::BM / 32, Big::BN / 128, true>(a, sc, sA, s_tok, &s_last, m0, n0, k0, k1, tile, piece, slot);
  else
    run_tile<Big::BM / 32, Big::BN / 128, false>(a, sc, sA, s_tok, &s_last, m0, n0, k0, k1, tile, piece, slot);
}

// Workspace layout, the same for every shape so that one workspace serves calls
// of different shapes: kSlots int32 counters (one per possible split tile; fewer
// than kSlots tiles are ever split: at most 256 / S left-over big tiles, or at
// most 512 / S Mid tiles), then the int32 partial tiles.
constexpr size_t kCounterBytes = kSlots * sizeof(int32_t);

}  // namespace

size_t gemm_workspace_bytes(int64_t M, int64_t K, int64_t N) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  const Schedule s = make_schedule(M, N, (K / kGroup + 1) / 2);
  if (s.split <= 1) return 0;
  return kCounterBytes + size_t(s.left() * s.split) * (s.mid ? Mid::Ints : kTileInts) * 4;
}

hipError_t launch_gemm(const int8_t *xq, const float *tok_scale, int64_t M, int64_t K, int64_t N,
                       const uint32_t *packed, const int8_t *q, const float *row_scale, void *y,
                       int y_dtype, int32_t *acc_out, void *workspace, hipStream_t stream) {
  if ((M + kBM - 1) / kBM * ((N + kBN - 1) / kBN) > 0x7FFFFFFF) return hipErrorInvalidValue;
  const Schedule s = make_schedule(M, N, (K / kGroup + 1) / 2);
  int32_t *counters = nullptr, *part = nullptr;
  if (s.split > 1) {
    counters = static_cast<int32_t *>(workspace);
    part = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + kCounterBytes);
  }
  (void)hipGetLastError();  // drop errors left by earlier, unrelated runtime calls
  if (s.grid() <= 2 * kSlots)
    hipLaunchKernelGGL(gemm_i8_kernel<true>, dim3(unsigned(s.grid())), dim3(kThreads), 0, stream, xq, tok_scale,
                       M, K, N, packed, q, row_scale, y, y_dtype, acc_out, part, counters, s);
  else
    hipLaunchKernelGGL(gemm_i8_kernel<false>, dim3(unsigned(s.grid())), dim3(kThreads), 0, stream, xq, tok_scale,
                       M, K, N, packed, q, row_scale, y, y_dtype, acc_out, part, counters, s);
  static const char *names[3] = {"gemm_i8_mfma32_128x256_lds2", "gemm_i8_mfma32_128x256_lds2_splitk",
                                  "gemm_i8_mfma32_128x256_lds2_narrowtail"};
  if (s.mid)
    set_last_kernel(s.split > 1 ? "gemm_i8_mfma32_128x128_lds2_splitk" : "gemm_i8_mfma32_128x128_lds2");
  else
    set_last_kernel(names[s.narrow ? 2 : s.split > 1 ? 1 : 0]);
  return hipGetLastError();
}

}  // namespace tl
