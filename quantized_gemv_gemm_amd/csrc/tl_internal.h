// Internal declarations shared by the host API and the kernel translation units.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "tl.h"

namespace tl {

constexpr int kGroup = 128;   // weights per fp16 scale along K
constexpr int kHBlock = 1024; // Hadamard block width

// name of the last kernel launched by this host thread
void set_last_kernel(const char *name);

int64_t packed_words(int64_t N, int64_t K);
hipError_t launch_pack(const int8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                       uint32_t *packed, int8_t *q, float *row_scale, int32_t *invalid_count,
                       hipStream_t stream);

hipError_t launch_hadamard(const uint16_t *x, int64_t T, int64_t K, const int8_t *signs,
                           float *xr, hipStream_t stream);

hipError_t launch_quant(const float *xr, int64_t T, int64_t K, int8_t *xq, float *tok_scale,
                        hipStream_t stream);

// Decode activation limbs in the GEMV workspace.  b <= 8: row-major rows, hi
// limbs [b][K + 16] then lo limbs [b][K + 16].  b > 8: the operand order of
// v_mfma_i32_16x16x64_i8, so that every operand load reads 1 KB contiguously:
// tokens in chunks of 16 (chunk c = t / 16 owns 32 K bytes at 32 K c); inside a
// chunk, for group g, 64-k half h and limb l, 64 lanes x 16 bytes, where lane
// r + 16 q holds A row r (token 16 c + 4 (r % 4) + r / 4) and
// k = 128 g + 32 q + 16 h + j.
// Limb scales: sigma[t][j] = |x|max / 32639 of token t's 1024-block j (the last
// block may be shorter), limb_blocks(K) per token, after the limbs.
constexpr int kLimbRowPad = 16;
constexpr int kTokChunk = 16;      // tokens per MFMA operand (and per GEMV grid row)
constexpr int kGemvMaxTokens = 64; // decode tokens per call
__host__ __device__ inline int64_t limb_chunks(int64_t b) { return (b + kTokChunk - 1) / kTokChunk; }
__host__ __device__ inline int limb_blocks(int64_t K) { return int((K + kHBlock - 1) / kHBlock); }
__host__ __device__ inline int64_t limb_region_bytes(int64_t b, int64_t K) {
  return b > 8 ? 32 * K * limb_chunks(b) : 2 * b * (K + kLimbRowPad);
}
__host__ __device__ inline int64_t limb_frag_offset(int t, int64_t k, int limb, int64_t K) {
  const int64_t g = k >> 7;
  const int kk = int(k & 127);
  const int tc = t & (kTokChunk - 1);
  const int row = 4 * (tc & 3) + (tc >> 2);
  return 32 * K * (t / kTokChunk) +
         (((((g * 2 + ((kk >> 4) & 1)) * 2 + limb) * 64 + row + 16 * (kk >> 5)) << 4) + (kk & 15));
}

size_t gemv_workspace_bytes(int64_t b, int64_t K, int64_t N);
// false when the weight-stream variant for (b, K, N) would not fit a compute unit
// (its LDS or workgroup size); the entry points then return TL_ERR_UNSUPPORTED
bool gemv_supported(int64_t b, int64_t K, int64_t N);
hipError_t launch_gemv_prepare(const float *xr, int64_t b, int64_t K, void *workspace,
                               hipStream_t stream);
hipError_t launch_gemv_main(const void *workspace, int64_t b, int64_t K, int64_t N,
                            const uint32_t *packed, const uint16_t *scales, void *y, int y_dtype,
                            hipStream_t stream);

// fused rotation -> GEMV limbs / int8 quantisation (k_rotq.hip)
bool fused_input_supported(int64_t K);
hipError_t launch_gemv_prepare_x(const uint16_t *x, int64_t b, int64_t K, const int8_t *signs,
                                 int8_t *xhi, int64_t Kp, float *sigma, hipStream_t stream);
hipError_t launch_quant_x(const uint16_t *x, int64_t T, int64_t K, const int8_t *signs, int8_t *xq,
                          float *tok_scale, hipStream_t stream);
// the GEMV workspace carved for the fused prep (k_gemv.hip)
hipError_t launch_gemv_prepare_rotated(const uint16_t *x, int64_t b, int64_t K, const int8_t *signs,
                                       void *workspace, hipStream_t stream);

// rotation + limbs + GEMV in one launch for one or two tokens (k_gemv.hip)
bool gemv_rot_supported(int64_t b, int64_t K, int64_t N);
hipError_t launch_gemv_rot(const uint16_t *x, int64_t b, int64_t K, int64_t N, const int8_t *signs,
                           const uint32_t *packed, const uint16_t *scales, void *y, int y_dtype,
                           hipStream_t stream);

// decode GEMV against int8 activations (k_gemv.hip)
bool gemv_q8_supported(int64_t b, int64_t K, int64_t N);
hipError_t launch_gemv_q8(const int8_t *xq, const float *tok_scale, int64_t b, int64_t K, int64_t N,
                          const uint32_t *packed, const uint16_t *scales, void *y, int y_dtype,
                          hipStream_t stream);

// split-block rotation stages (k_split.hip)
hipError_t launch_hadamard_half(const uint16_t *x, int64_t T, int64_t ldx, const int8_t *signs,
                                double *u, hipStream_t stream);
hipError_t launch_hadamard_join(const double *u_lo, const double *u_hi, int64_t T, int half, float *xr,
                                int64_t ldxr, hipStream_t stream);

// measurement helper: a launch that only reads `bytes` (k_probe.hip)
hipError_t launch_read_probe(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream);
hipError_t launch_mfma_probe(int random, int iters, uint32_t *sink, hipStream_t stream);

size_t gemm_workspace_bytes(int64_t M, int64_t K, int64_t N);
hipError_t launch_gemm(const int8_t *xq, const float *tok_scale, int64_t M, int64_t K, int64_t N,
                       const uint32_t *packed, const int8_t *q, const float *row_scale, void *y,
                       int y_dtype, int32_t *acc_out, void *workspace, hipStream_t stream);

// whole layer from the raw input (tl_api.cpp): the checks that need no workspace,
// then the workspace checks and the launches on the path tl_linear_path names
size_t linear_scratch_bytes(int64_t T, int64_t K, int64_t N);
int linear_check(const uint16_t *x, int64_t T, int64_t K, int64_t N, const uint32_t *packed,
                 const uint16_t *scales, const int8_t *q, const float *row_scale, void *y, int y_dtype);
int linear_run(const uint16_t *x, int64_t T, int64_t K, int64_t N, const int8_t *signs,
               const uint32_t *packed, const uint16_t *scales, const int8_t *q, const float *row_scale,
               void *y, int y_dtype, void *workspace, size_t workspace_bytes, hipStream_t st);

}  // namespace tl
