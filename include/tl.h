/*
 * tl.h -- C ABI of the ternary linear-layer library for AMD Instinct MI355X (gfx950).
 *
 * The layer is the quantized linear layer of the ternary 27B model described in
 * qiita.com/nakanokensetsu/items/ecc183fae033565af7cb (cited below as [P1] with
 * its section headings):
 *   - weights are 2-bit codes in {-1, 0, +1} with one fp16 scale per row and per
 *     128-element group along K ([P1] "前提");
 *   - the input is rotated by a block-wise Sylvester Hadamard transform with
 *     1024-wide blocks and an optional sign table ([P1] "前提", "1. TP=2 への移植");
 *   - decode computes y = W (H_blk x) for 1..64 tokens;
 *   - prefill decomposes each scale as q = round(127 s / smax) so that
 *     code * q is exact in int8, quantises the rotated activations to int8 per
 *     token, and runs one int8 x int8 -> int32 GEMM followed by a per-row and
 *     per-token rescale ([P1] "4. 効いた高速化").
 *
 * Conventions for every call
 *   - Every tensor argument is a DEVICE pointer owned by the caller, dense and
 *     row-major (C order).  The library allocates no device memory; scratch, when
 *     a call needs it, is a caller-provided workspace whose size a *_workspace_size
 *     query returns (tl_linear_apply_noalloc instead uses a static device array
 *     of tl_noalloc_scratch_bytes() per GPU, see there).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  All
 *     work is enqueued on it; no call synchronises.  A device fault surfaces at the
 *     caller's next synchronisation.
 *   - Arguments are checked on the host before anything is launched.  A failed
 *     check returns a non-zero TL_ERR_* code, launches nothing and leaves every
 *     output untouched.  Launch failures return TL_ERR_LAUNCH.
 *   - Counts of zero (T, b, M, N) are valid and do nothing; K must be positive.
 *   - Inputs and outputs must not overlap (TL_ERR_ALIAS).
 *   - Pointers must be 16-byte aligned (TL_ERR_ALIGN).
 *   - Value preconditions (codes in {-1,0,+1}, signs +-1, finite inputs) are not
 *     checked on the device, except that tl_pack_weights can count bad codes.
 *   - Calls are thread-safe; concurrent calls on different streams are
 *     independent (each uses only its own arguments and workspace).
 *
 * Packed weight layout (ABI version 2; the page gives no layout, this one is ours)
 *   Codes are stored two bits each in uint32 words.  Within a word, code j
 *   (j = 0..15, for 16 consecutive k) occupies bits 8*(j mod 4) + 2*(j div 4) and
 *   the bit above it, so ((w >> 2r) & 0x03030303) holds codes 4r..4r+3 in bytes
 *   0..3, in k order.  A field is the code's two's-complement low two bits:
 *   0 -> 00, +1 -> 01, -1 -> 11 (10 is never written).
 *   Words are grouped in 1024-byte tiles that match the lanes of a 64-wide
 *   wavefront: rows are taken in blocks of 16 and K in pairs of 128-groups,
 *   NB = ceil(N/16) row blocks, GP = ceil(K/256) group pairs (a last partial
 *   block or pair is padded with zero codes).  Tile (rb, p) starts at word
 *   256*(rb*GP + p).  Its word 4*l + 2*gi + m (l = 0..63, gi, m in {0, 1}) holds
 *   the codes k = 128*(2p + gi) + 16*(2*(l/16) + m) + j, j = 0..15, of row
 *   n = 16*rb + (l mod 16).  Lane l of a wavefront reading 16 bytes at
 *   4*l words thus gets, for both groups of the pair, the two words an
 *   int8 16x16x64 matrix instruction needs from it.  tl_packed_bytes(N, K)
 *   gives the size.
 */
#ifndef TL_H
#define TL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TL_ABI_VERSION 2

/* status codes returned by every call */
#define TL_OK 0
#define TL_ERR_NULLPTR 1     /* a required pointer is NULL */
#define TL_ERR_SHAPE 2       /* a size is negative, out of range or not a required multiple */
#define TL_ERR_ALIGN 3       /* a pointer is not 16-byte aligned */
#define TL_ERR_DTYPE 4       /* y_dtype is not TL_BF16 or TL_F32 */
#define TL_ERR_LAUNCH 5      /* the HIP runtime reported an error */
#define TL_ERR_UNSUPPORTED 6 /* no kernel variant for this request */
#define TL_ERR_WORKSPACE 7   /* workspace missing or smaller than the query says */
#define TL_ERR_ALIAS 8       /* an output overlaps an input or another output */
#define TL_ERR_SCRATCH 9     /* beyond the static scratch of tl_linear_apply_noalloc */

/* output element types */
#define TL_BF16 0 /* bfloat16, round to nearest even from fp32 */
#define TL_F32 1  /* IEEE binary32 */

/* Version of the packed layout and of the signatures below (TL_ABI_VERSION). */
int tl_abi_version(void);

/* Static text for a status code; never NULL. */
const char *tl_status_string(int status);

/* Name of the last kernel this host thread launched through the library
 * ("" before the first launch).  Used to check which variant ran. */
const char *tl_last_kernel_name(void);

/* Text of the HIP runtime error behind the last TL_ERR_LAUNCH returned on this
 * host thread ("" if none).  For diagnostics only. */
const char *tl_last_error_detail(void);

/*
 * tl_pack_weights -- load-time conversion of one ternary layer.
 *   [P1] "前提" (2-bit codes, one fp16 scale per row and 128-group) and
 *   [P1] "4. 効いた高速化" (q[n,g] = round(127 s[n,g] / smax[n])).
 * in  codes      int8   [N, K]     values in {-1, 0, +1}
 * in  scales     fp16   [N, K/128] (raw IEEE half bits), finite
 * out packed     uint32, tl_packed_bytes(N, K) bytes, layout above (padding
 *                included and written)
 * out q          int8   [N, K/128] q = RNE( fl32(fl32(127*s) / smax) ),
 *                                  smax[n] = max_g |s[n,g]|; |q| <= 127
 * out row_scale  f32    [N]        fl32(smax / 127)
 * out invalid_count int32 [1] or NULL: if not NULL, the number of codes outside
 *                  {-1,0,+1} is ADDED to it (the caller zeroes it first).
 * A row whose scales are all zero gets q = 0 and row_scale = 0.
 * Requires K > 0, K % 128 == 0.
 */
size_t tl_packed_bytes(int64_t N, int64_t K);
int tl_pack_weights(const int8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                    uint32_t *packed, int8_t *q, float *row_scale, int32_t *invalid_count,
                    void *stream);

/*
 * tl_hadamard_blk -- block rotation of the layer input.
 *   [P1] "前提" (Hadamard rotation on the input side) and "1. TP=2 への移植"
 *   (Sylvester type, 1024-wide blocks, sign table keyed by the layer width).
 * in  x      bf16 [T, K] (raw bits)
 * in  signs  int8 [K] of +-1, or NULL for all +1; applied to x before H
 * out xr     f32  [T, K]: for each token and block j,
 *            xr[t, 1024 j + i] = (1/32) sum_m (-1)^popcount(i & m) d[1024 j + m] x[t, 1024 j + m]
 *            computed exactly (binary64 butterflies) and rounded once to f32.
 *            The result is exact before that rounding whenever the x values are
 *            multiples of 2^-31 below 2^8 in magnitude (bf16 with |x| >= 2^-24).
 * Requires K > 0, K % 1024 == 0.
 */
int tl_hadamard_blk(const uint16_t *x, int64_t T, int64_t K, const int8_t *signs, float *xr,
                    void *stream);

/*
 * tl_hadamard_half, tl_hadamard_join -- the rotation of a 1024-block that a
 * K-shard boundary splits in the middle, in two stages with an exchange of the
 * stage results between the two ranks in between.
 *   [P1] "1. TP=2 への移植" (17408 / 2 = 8704 falls in the middle of a block;
 *   H1024 [a; b] = [H512 a + H512 b; H512 a - H512 b]: each rank transforms its
 *   own 512 columns, the results are exchanged, the rank with the first half
 *   keeps the sum, the other the difference).
 * tl_hadamard_half:
 * in  x      bf16 [T, 512] with rows ldx elements apart (ldx >= 512, ldx % 8 == 0,
 *            so a column slice of the rank's [T, K_shard] input can be passed)
 * in  signs  int8 [512] of +-1 for these columns, or NULL for all +1
 * out u      f64  [T, 512] dense: u[t, i] = sum_m (-1)^popcount(i & m) d[m] x[t, m]
 *            (no 1/32), exact in binary64 for inputs that are multiples of 2^-31
 *            below 2^8 in magnitude (bf16 with |x| >= 2^-24).
 * tl_hadamard_join:
 * in  u_lo, u_hi  f64 [T, 512]: the stage results of the block's first and second
 *            512 columns (one computed here, one received from the other rank)
 * in  half   0 for the rank that holds the first half, 1 for the other
 * out xr     f32 [T, 512] with rows ldxr elements apart (ldxr >= 512, ldxr % 4 == 0):
 *            half 0: fl32((u_lo + u_hi) / 32), half 1: fl32((u_lo - u_hi) / 32) --
 *            bit for bit the columns tl_hadamard_blk produces for that half.
 * The exchange itself (512 binary64 values per token each way) is the caller's.
 */
int tl_hadamard_half(const uint16_t *x, int64_t T, int64_t ldx, const int8_t *signs, double *u,
                     void *stream);
int tl_hadamard_join(const double *u_lo, const double *u_hi, int64_t T, int half, float *xr,
                     int64_t ldxr, void *stream);

/*
 * tl_gemv_ternary -- decode GEMV, y = W xr for 1..64 tokens.
 *   [P1] "前提" (y = W (H_blk x), W = code * group scale).
 * in  xr      f32    [b, K]      rotated activations (tl_hadamard_blk output)
 * in  packed  uint32 tiles      from tl_pack_weights (tl_packed_bytes(N, K) bytes)
 * in  scales  fp16   [N, K/128]
 * out y       [b, N] of y_dtype: y[t,n] = sum_g s[n,g] sum_{k in g} code[n,k] xr[t,k]
 * workspace   device scratch of at least tl_gemv_workspace_size(b, K, N) bytes,
 *             16-byte aligned; its contents on entry do not matter.
 * Numerics: each weight is read once for all b tokens; group sums run on int8
 * matrix cores with each token's activations held as a 15-bit fixed-point value
 * split into two int8 limbs, scaled per token and 1024-wide block of K (scale
 * |x|max / 32639 of that block), and group results are accumulated in f32.
 * Relative Frobenius error against exact arithmetic is about 3e-5 on the
 * generator's data (bound used by the tests: 1e-3).  In general each activation
 * is off by at most 2^-16 of the largest magnitude in its own block (15 bits per
 * block, whatever the other blocks hold), so the error of y[t, n] is at most
 * about 2^-16 sum_g |s[n,g]| sum_{k in g} |code[n,k]| max_blk(k) |xr[t,.]|: the
 * relative error stays near 3e-5 unless y itself is small against that sum
 * (heavy cancellation) or a block's values spread over more than 15 bits.
 * One matrix-core operand holds 16 tokens: b > 16 runs ceil(b/16) chunks of 16
 * tokens side by side in the same launch, each streaming the weights itself
 * (chunks of one row range share an L2), so the time grows with the chunk count
 * (tl_linear_path tells when the prefill path is the faster choice).
 * Requires 0 <= b <= 64, K > 0, K % 128 == 0.
 */
size_t tl_gemv_workspace_size(int64_t b, int64_t K, int64_t N);
int tl_gemv_ternary(const float *xr, int64_t b, int64_t K, int64_t N, const uint32_t *packed,
                    const uint16_t *scales, void *y, int y_dtype, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * The two stages of tl_gemv_ternary, for callers that apply several weight
 * matrices to the same rotated input (e.g. q/k/v or gate/up as separate
 * layers) or that time the stages apart:
 *   tl_gemv_prepare  writes the activation limbs and their per-block scales of
 *                    xr [b, K] into the workspace (one kernel, one wavefront per
 *                    token and 1024-block);
 *   tl_gemv_prepared runs the weight-streaming kernel on a workspace that
 *                    tl_gemv_prepare filled for the same b and K (one kernel).
 * tl_gemv_ternary(...) is exactly tl_gemv_prepare followed by tl_gemv_prepared.
 * The workspace must stay unmodified between the two calls.
 */
int tl_gemv_prepare(const float *xr, int64_t b, int64_t K, void *workspace,
                    size_t workspace_bytes, void *stream);
int tl_gemv_prepared(const void *workspace, size_t workspace_bytes, int64_t b, int64_t K,
                     int64_t N, const uint32_t *packed, const uint16_t *scales, void *y,
                     int y_dtype, void *stream);

/*
 * tl_gemv_ternary_q8 -- decode GEMV against int8 activations (the int8 decode
 * variant [P1] "5." weighed and set aside for its extra error: the page's dp4a
 * kernel; here int8 matrix cores).
 *   [P1] "前提" (y = W (H_blk x)), "4. 効いた高速化" (per-token int8 activations).
 * in  xq, tok_scale  int8 [b, K], f32 [b]: the rotated activations quantised per
 *                    token by tl_quant_act_int8 (or tl_quant_act_int8_x)
 * in  packed, scales as for tl_gemv_ternary
 * out y       [b, N] of y_dtype:
 *             y[t,n] = tok_scale[t] * sum_g s[n,g] sum_{k in g} code[n,k] xq[t,k]
 *             (group sums exact in int32, f32 accumulation over the groups)
 * One matrix-core chain per group and b*K activation bytes, against two limb
 * chains and 2*b*K for tl_gemv_ternary; the result carries the activation
 * rounding (about 8e-3 relative against the exact layer on the generator's data,
 * against about 3e-5 for tl_gemv_ternary).  No workspace.
 * Requires 0 <= b <= 16, K > 0, K % 128 == 0, and a wave's share of the group
 * pairs must fit its registers: every b is supported for K <= 18432, larger K
 * only while b (K + 16) <= 96 KiB (TL_ERR_UNSUPPORTED otherwise).
 */
int tl_gemv_ternary_q8(const int8_t *xq, const float *tok_scale, int64_t b, int64_t K, int64_t N,
                       const uint32_t *packed, const uint16_t *scales, void *y, int y_dtype,
                       void *stream);

/*
 * tl_quant_act_int8 -- per-token int8 quantisation of rotated activations.
 *   [P1] "4. 効いた高速化" (activations quantised to int8 per token after the
 *   rotation, which evens out outliers).
 * in  xr         f32  [T, K]
 * out xq         int8 [T, K]  clamp( RNE( fl32(xr / sx_t) ), -127, 127 )
 * out tok_scale  f32  [T]     sx_t = fl32(amax_t / 127), amax_t = max_k |xr[t,k]|
 * A token with amax = 0 gets sx = 0 and xq = 0.  Divisions are correctly rounded.
 * Requires K > 0, K % 128 == 0.
 */
int tl_quant_act_int8(const float *xr, int64_t T, int64_t K, int8_t *xq, float *tok_scale,
                      void *stream);

/*
 * Fused layer inputs: the block rotation and the step that consumes it in one
 * launch, so the rotated activations are never written to memory.
 *   [P1] "前提" (rotation of the input), "4. 効いた高速化" (int8 per token after
 *   the rotation).  Outputs are bit-identical to the unfused sequences:
 *     tl_gemv_prepare_x   == tl_hadamard_blk then tl_gemv_prepare
 *     tl_gemv_ternary_x   == tl_hadamard_blk then tl_gemv_ternary
 *     tl_quant_act_int8_x == tl_hadamard_blk then tl_quant_act_int8
 *   except tl_gemv_ternary_x (and the GEMV path of tl_linear_apply) for one
 *   token with N <= 12288 and K <= 6144 (N <= 8192 at K = 6144) or two tokens
 *   with N <= 6144 and K <= 4096, K a multiple of 1024: there a
 *   single kernel rotates, splits into limbs and runs the GEMV, each workgroup
 *   rotating the blocks it needs; its limbs are the same, but it adds the
 *   group results in another order, so its output is not bit-identical to the
 *   sequence (the same error against the exact layer, about 3e-5), and the
 *   workspace (still required) is not used.
 * in  x       bf16 [b or T, K] raw layer input; signs as in tl_hadamard_blk.
 * Requires K % 1024 == 0 and K <= 65536 (TL_ERR_UNSUPPORTED above: use the
 * unfused calls); other arguments as in the unfused entry points.
 */
int tl_gemv_prepare_x(const uint16_t *x, int64_t b, int64_t K, const int8_t *signs,
                      void *workspace, size_t workspace_bytes, void *stream);
int tl_gemv_ternary_x(const uint16_t *x, int64_t b, int64_t K, int64_t N, const int8_t *signs,
                      const uint32_t *packed, const uint16_t *scales, void *y, int y_dtype,
                      void *workspace, size_t workspace_bytes, void *stream);
int tl_quant_act_int8_x(const uint16_t *x, int64_t T, int64_t K, const int8_t *signs, int8_t *xq,
                        float *tok_scale, void *stream);

/*
 * tl_gemm_int8_rescale -- prefill int8 GEMM and rescale.
 *   [P1] "4. 効いた高速化" (W_int8 = code * q exactly in int8; one int8 GEMM,
 *   then a per-row and per-token rescale).
 * in  xq         int8   [M, K]     from tl_quant_act_int8
 * in  tok_scale  f32    [M]
 * in  packed     uint32 tiles     from tl_pack_weights
 * in  q          int8   [N, K/128] from tl_pack_weights
 * in  row_scale  f32    [N]        from tl_pack_weights
 * out y          [M, N] of y_dtype: y = fl32( fl32(acc) * row_scale[n] ) * tok_scale[m]
 * out acc_out    int32  [M, N] or NULL: acc[m,n] = sum_k xq[m,k] code[n,k] q[n,k/128]
 *                (exact; |acc| <= K * 127^2, so K <= 133143 keeps it in int32)
 * workspace      device scratch of at least tl_gemm_workspace_size(M, K, N)
 *                bytes (may be NULL when that size is 0).  Layout: 256 int32
 *                counters (one per K-split tile; at most 256 are ever used),
 *                then the int32 partial tiles of the K-split work.  It must be
 *                zero-filled before its first use; every call leaves the
 *                counters at zero again, so one workspace can be reused, also
 *                across shapes, without clearing.  Calls that overlap in time
 *                must not share one.
 * The size depends only on (M, K, N): the schedule is fixed for the 256
 * compute units of gfx950 (whole rounds of 512 tiles, two per compute unit,
 * of 128 x 256 or, with fewer than 512 such tiles, of 128 x 128; the left-over
 * tiles split along K into up to 6 pieces or cut into sub-tiles).
 * Requires K > 0, K % 128 == 0, K <= 133120.
 */
size_t tl_gemm_workspace_size(int64_t M, int64_t K, int64_t N);
int tl_gemm_int8_rescale(const int8_t *xq, const float *tok_scale, int64_t M, int64_t K,
                         int64_t N, const uint32_t *packed, const int8_t *q,
                         const float *row_scale, void *y, int y_dtype, int32_t *acc_out,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * tl_linear_apply -- the whole layer from the raw input, y = W (H_blk x) for T
 * tokens, on the path that tl_linear_path(T, K, N) names:
 *   TL_PATH_GEMV  rotation fused into the limb prep, then the two-limb GEMV
 *                 (tl_gemv_ternary_x); relative error about 3e-5;
 *   TL_PATH_INT8  rotation fused into the per-token int8 quantisation, then the
 *                 int8 GEMM + rescale (tl_quant_act_int8_x, tl_gemm_int8_rescale);
 *                 relative error about 1e-2 against the exact layer (the
 *                 activation and scale rounding of [P1] "4. 効いた高速化").
 *   [P1] "前提" (the layer), "4. 効いた高速化" (the prefill path); the choice by
 *   token count mirrors the page's decode / prefill split.
 * tl_linear_path: up to 16 tokens the GEMV; 17..64 tokens the GEMV while
 * ceil(T/16) * N * K <= 2^27 (every 16-token chunk streams all weights
 * again), else the int8 path; above 64 tokens the int8 path.
 * The rule follows a measured token sweep of both paths at the qkv
 * (5120 -> 10240), gate_up (5120 -> 34816) and down (17408 -> 5120) shapes.
 * in  x          bf16 [T, K] raw layer input; signs as in tl_hadamard_blk
 * in  packed, scales, q, row_scale  from tl_pack_weights (all four are required
 *                whichever path runs)
 * out y          [T, N] of y_dtype
 * workspace      device scratch of at least tl_linear_workspace_size(T, K, N)
 *                bytes, zero-filled before its first use (its first KiB holds the
 *                int8 GEMM's split-K counters, which every call leaves at zero, as
 *                for tl_gemm_int8_rescale); calls that overlap in time must not
 *                share one.
 * Requires K % 1024 == 0 and K <= 65536 (TL_ERR_UNSUPPORTED above).
 */
#define TL_PATH_GEMV 0
#define TL_PATH_INT8 1
int tl_linear_path(int64_t T, int64_t K, int64_t N);
size_t tl_linear_workspace_size(int64_t T, int64_t K, int64_t N);
int tl_linear_apply(const uint16_t *x, int64_t T, int64_t K, int64_t N, const int8_t *signs,
                    const uint32_t *packed, const uint16_t *scales, const int8_t *q,
                    const float *row_scale, void *y, int y_dtype, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * tl_read_probe -- measurement helper, not a step of the layer: one launch that
 * only reads `bytes` (a multiple of 16) from src, the way the decode GEMV streams
 * its weights (1 KB per wavefront load, all of a wavefront's loads at once), and
 * writes nothing but possibly one word of *sink.  Its duration is the floor a
 * single launch reading that many bytes reaches on this chip (launch, first
 * memory round trip and tail included), beside which the GEMV's launch time can
 * be put.  src and sink are device pointers, 16-byte aligned.
 */
int tl_read_probe(const void *src, size_t bytes, uint32_t *sink, void *stream);

/*
 * tl_mfma_probe -- measurement helper, not a step of the layer: one launch of 512
 * workgroups of 256 threads (two per compute unit, as the prefill GEMM runs) in
 * which every wavefront issues iters x 8 v_mfma_i32_32x32x32_i8 on eight
 * independent accumulators (65536 int8 operations each) and nothing else, with
 * constant operands (random_operands = 0: every byte 1) or random-looking ones
 * (two sets hashed from the lane and workgroup, alternating from one
 * instruction to the next).  Its duration gives the int8 matrix-core
 * rate the chip sustains with each kind of data, beside which the GEMM's can be
 * put: 512 * 4 * iters * 8 * 65536 operations.  sink is a device pointer,
 * 16-byte aligned, of which at most one word is written.
 * Errors: TL_ERR_SHAPE for iters <= 0, TL_ERR_NULLPTR, TL_ERR_ALIGN.
 */
int tl_mfma_probe(int random_operands, int iters, uint32_t *sink, void *stream);

/*
 * tl_linear_apply_noalloc -- tl_linear_apply without a workspace argument and
 * without any allocation, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid it.
 * It runs the same kernels as tl_linear_apply (same path rule, same outputs, bit
 * for bit) with the workspace taken from a static device array of
 * tl_noalloc_scratch_bytes() bytes, one per GPU, held until the process ends.
 * The first call on a device looks the array up and zeroes its counter region
 * (one small kernel on `stream`); later calls leave the counters at zero as
 * tl_linear_apply does.  Every call on one GPU shares that GPU's array: calls
 * that overlap in time on one GPU (two streams, two host threads) race and must
 * be serialised by the caller.  A request whose workspace
 * (tl_linear_workspace_size(T, K, N)) exceeds the array returns TL_ERR_SCRATCH
 * before anything is launched; so do all other argument errors of
 * tl_linear_apply, with the same codes.
 */
size_t tl_noalloc_scratch_bytes(void);
int tl_linear_apply_noalloc(const uint16_t *x, int64_t T, int64_t K, int64_t N, const int8_t *signs,
                            const uint32_t *packed, const uint16_t *scales, const int8_t *q,
                            const float *row_scale, void *y, int y_dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TL_H */
