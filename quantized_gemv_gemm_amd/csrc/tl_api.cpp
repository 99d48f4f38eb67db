// Host side of the C ABI declared in include/tl.h: argument checks, then launches.
// Every check runs before any HIP call, so a rejected call touches neither the
// GPU nor the outputs.
#include <stdint.h>
#include <string.h>

#include "tl_internal.h"

namespace tl {
static thread_local const char *g_last_kernel = "";
static thread_local const char *g_last_error = "";
void set_last_kernel(const char *name) { g_last_kernel = name; }
}  // namespace tl

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
  const void *p;
  size_t bytes;
};

bool overlap(Span a, Span b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// outputs must not overlap inputs or each other
bool any_alias(const Span *in, int nin, const Span *out, int nout) {
  for (int o = 0; o < nout; ++o) {
    for (int i = 0; i < nin; ++i)
      if (overlap(out[o], in[i])) return true;
    for (int j = o + 1; j < nout; ++j)
      if (overlap(out[o], out[j])) return true;
  }
  return false;
}

int from_hip(hipError_t e) {
  if (e == hipSuccess) return TL_OK;
  tl::g_last_error = hipGetErrorString(e);
  return TL_ERR_LAUNCH;
}

constexpr int64_t kMaxDim = int64_t(1) << 31;  // rows, tokens and K stay below 2^31

}  // namespace

extern "C" {

int tl_abi_version(void) { return TL_ABI_VERSION; }

const char *tl_status_string(int s) {
  switch (s) {
    case TL_OK: return "ok";
    case TL_ERR_NULLPTR: return "a required pointer is NULL";
    case TL_ERR_SHAPE: return "invalid shape (negative, too large, or not a required multiple)";
    case TL_ERR_ALIGN: return "pointer not 16-byte aligned";
    case TL_ERR_DTYPE: return "y_dtype must be TL_BF16 or TL_F32";
    case TL_ERR_LAUNCH: return "HIP runtime error during launch";
    case TL_ERR_UNSUPPORTED: return "no kernel variant for this request";
    case TL_ERR_WORKSPACE: return "workspace missing or too small";
    case TL_ERR_ALIAS: return "an output overlaps an input or another output";
    case TL_ERR_SCRATCH:
      return "request needs more scratch than the no-allocation entry point's static buffer holds";
    default: return "unknown status";
  }
}

const char *tl_last_kernel_name(void) { return tl::g_last_kernel; }

const char *tl_last_error_detail(void) { return tl::g_last_error; }

size_t tl_packed_bytes(int64_t N, int64_t K) {
  if (N < 0 || K <= 0 || K % tl::kGroup || N >= kMaxDim || K >= kMaxDim) return 0;
  return size_t(tl::packed_words(N, K)) * 4;
}

int tl_pack_weights(const int8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                    uint32_t *packed, int8_t *q, float *row_scale, int32_t *invalid_count,
                    void *stream) {
  if (N < 0 || K <= 0 || K % tl::kGroup || N >= kMaxDim || K >= kMaxDim) return TL_ERR_SHAPE;
  if (N == 0) return TL_OK;
  if (!codes || !scales || !packed || !q || !row_scale) return TL_ERR_NULLPTR;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(packed) || !aligned16(q) ||
      !aligned16(row_scale))
    return TL_ERR_ALIGN;
  const size_t G = size_t(K / tl::kGroup);
  Span in[] = {{codes, size_t(N) * K}, {scales, size_t(N) * G * 2}};
  Span out[] = {{packed, size_t(tl::packed_words(N, K)) * 4}, {q, size_t(N) * G}, {row_scale, size_t(N) * 4},
                {invalid_count, invalid_count ? 4u : 0u}};
  if (any_alias(in, 2, out, 4)) return TL_ERR_ALIAS;
  return from_hip(tl::launch_pack(codes, scales, N, K, packed, q, row_scale, invalid_count,
                                  static_cast<hipStream_t>(stream)));
}

int tl_hadamard_blk(const uint16_t *x, int64_t T, int64_t K, const int8_t *signs, float *xr,
                    void *stream) {
  if (T < 0 || K <= 0 || K % tl::kHBlock || T >= kMaxDim || K >= kMaxDim) return TL_ERR_SHAPE;
  if (T == 0) return TL_OK;
  if (!x || !xr) return TL_ERR_NULLPTR;
  if (!aligned16(x) || !aligned16(xr) || (signs && !aligned16(signs))) return TL_ERR_ALIGN;
  Span in[] = {{x, size_t(T) * K * 2}, {signs, signs ? size_t(K) : 0u}};
  Span out[] = {{xr, size_t(T) * K * 4}};
  if (any_alias(in, 2, out, 1)) return TL_ERR_ALIAS;
  return from_hip(tl::launch_hadamard(x, T, K, signs, xr, static_cast<hipStream_t>(stream)));
}

int tl_hadamard_half(const uint16_t *x, int64_t T, int64_t ldx, const int8_t *signs, double *u,
                     void *stream) {
  if (T < 0 || T >= kMaxDim || ldx < tl::kHBlock / 2 || ldx >= kMaxDim) return TL_ERR_SHAPE;
  if (T == 0) return TL_OK;
  if (!x || !u) return TL_ERR_NULLPTR;
  if (!aligned16(x) || ldx % 8 || !aligned16(u)) return TL_ERR_ALIGN;
  const size_t half = tl::kHBlock / 2;
  Span in[] = {{x, (size_t(T - 1) * ldx + half) * 2}, {signs, signs ? half : 0u}};
  Span out[] = {{u, size_t(T) * half * 8}};
  if (any_alias(in, 2, out, 1)) return TL_ERR_ALIAS;
  return from_hip(tl::launch_hadamard_half(x, T, ldx, signs, u, static_cast<hipStream_t>(stream)));
}

int tl_hadamard_join(const double *u_lo, const double *u_hi, int64_t T, int half, float *xr,
                     int64_t ldxr, void *stream) {
  if (T < 0 || T >= kMaxDim || ldxr < tl::kHBlock / 2 || ldxr >= kMaxDim || (half != 0 && half != 1))
    return TL_ERR_SHAPE;
  if (T == 0) return TL_OK;
  if (!u_lo || !u_hi || !xr) return TL_ERR_NULLPTR;
  if (!aligned16(u_lo) || !aligned16(u_hi) || !aligned16(xr) || ldxr % 4) return TL_ERR_ALIGN;
  const size_t hb = tl::kHBlock / 2;
  Span in[] = {{u_lo, size_t(T) * hb * 8}, {u_hi, size_t(T) * hb * 8}};
  Span out[] = {{xr, (size_t(T - 1) * ldxr + hb) * 4}};
  if (any_alias(in, 2, out, 1)) return TL_ERR_ALIAS;
  return from_hip(tl::launch_hadamard_join(u_lo, u_hi, T, half, xr, ldxr, static_cast<hipStream_t>(stream)));
}

size_t tl_gemv_workspace_size(int64_t b, int64_t K, int64_t N) {
  if (b < 0 || b > tl::kGemvMaxTokens || K <= 0 || K % tl::kGroup || N < 0) return 0;
  return tl::gemv_workspace_bytes(b, K, N);
}

namespace {
int check_gemv_shape(int64_t b, int64_t K, int64_t N, int64_t bmax = tl::kGemvMaxTokens) {
  if (b < 0 || b > bmax || N < 0 || K <= 0 || K % tl::kGroup || N >= kMaxDim || K >= kMaxDim)
    return TL_ERR_SHAPE;
  return TL_OK;
}
}  // namespace

int tl_gemv_prepare(const float *xr, int64_t b, int64_t K, void *workspace, size_t workspace_bytes,
                    void *stream) {
  if (int s = check_gemv_shape(b, K, 0)) return s;
  if (b == 0) return TL_OK;
  if (!xr) return TL_ERR_NULLPTR;
  const size_t need = tl::gemv_workspace_bytes(b, K, 0);
  if (!workspace || workspace_bytes < need) return TL_ERR_WORKSPACE;
  if (!aligned16(xr) || !aligned16(workspace)) return TL_ERR_ALIGN;
  Span in[] = {{xr, size_t(b) * K * 4}};
  Span out[] = {{workspace, need}};
  if (any_alias(in, 1, out, 1)) return TL_ERR_ALIAS;
  return from_hip(tl::launch_gemv_prepare(xr, b, K, workspace, static_cast<hipStream_t>(stream)));
}

int tl_gemv_prepared(const void *workspace, size_t workspace_bytes, int64_t b, int64_t K, int64_t N,
                     const uint32_t *packed, const uint16_t *scales, void *y, int y_dtype,
                     void *stream) {
  if (int s = check_gemv_shape(b, K, N)) return s;
  if (y_dtype != TL_BF16 && y_dtype != TL_F32) return TL_ERR_DTYPE;
  if (b == 0 || N == 0) return TL_OK;
  if (!packed || !scales || !y) return TL_ERR_NULLPTR;
  const size_t need = tl::gemv_workspace_bytes(b, K, N);
  if (!workspace || workspace_bytes < need) return TL_ERR_WORKSPACE;
  if (!aligned16(packed) || !aligned16(scales) || !aligned16(y) || !aligned16(workspace))
    return TL_ERR_ALIGN;
  const size_t G = size_t(K / tl::kGroup);
  const size_t ysz = size_t(b) * N * (y_dtype == TL_F32 ? 4 : 2);
  Span in[] = {{workspace, need}, {packed, size_t(tl::packed_words(N, K)) * 4}, {scales, size_t(N) * G * 2}};
  Span out[] = {{y, ysz}};
  if (any_alias(in, 3, out, 1)) return TL_ERR_ALIAS;
  if (!tl::gemv_supported(b, K, N)) return TL_ERR_UNSUPPORTED;
  return from_hip(tl::launch_gemv_main(workspace, b, K, N, packed, scales, y, y_dtype,
                                       static_cast<hipStream_t>(stream)));
}

int tl_gemv_ternary(const float *xr, int64_t b, int64_t K, int64_t N, const uint32_t *packed,
                    const uint16_t *scales, void *y, int y_dtype, void *workspace,
                    size_t workspace_bytes, void *stream) {
  if (int s = check_gemv_shape(b, K, N)) return s;
  if (y_dtype != TL_BF16 && y_dtype != TL_F32) return TL_ERR_DTYPE;
  if (b == 0 || N == 0) return TL_OK;
  if (!xr || !packed || !scales || !y) return TL_ERR_NULLPTR;
  const size_t need = tl::gemv_workspace_bytes(b, K, N);
  if (!workspace || workspace_bytes < need) return TL_ERR_WORKSPACE;
  if (!aligned16(xr) || !aligned16(packed) || !aligned16(scales) || !aligned16(y) ||
      !aligned16(workspace))
    return TL_ERR_ALIGN;
  const size_t G = size_t(K / tl::kGroup);
  const size_t ysz = size_t(b) * N * (y_dtype == TL_F32 ? 4 : 2);
  Span in[] = {{xr, size_t(b) * K * 4}, {packed, size_t(tl::packed_words(N, K)) * 4}, {scales, size_t(N) * G * 2}};
  Span out[] = {{y, ysz}, {workspace, need}};
  if (any_alias(in, 3, out, 2)) return TL_ERR_ALIAS;
  if (!tl::gemv_supported(b, K, N)) return TL_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = tl::launch_gemv_prepare(xr, b, K, workspace, st);
  if (e != hipSuccess) return from_hip(e);
  return from_hip(tl::launch_gemv_main(workspace, b, K, N, packed, scales, y, y_dtype, st));
}

int tl_gemv_prepare_x(const uint16_t *x, int64_t b, int64_t K, const int8_t *signs,
                      void *workspace, size_t workspace_bytes, void *stream) {
  if (int s = check_gemv_shape(b, K, 0)) return s;
  if (K % tl::kHBlock) return TL_ERR_SHAPE;
  if (!tl::fused_input_supported(K)) return TL_ERR_UNSUPPORTED;
  if (b == 0) return TL_OK;
  if (!x) return TL_ERR_NULLPTR;
  const size_t need = tl::gemv_workspace_bytes(b, K, 0);
  if (!workspace || workspace_bytes < need) return TL_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(workspace) || (signs && !aligned16(signs))) return TL_ERR_ALIGN;
  Span in[] = {{x, size_t(b) * K * 2}, {signs, signs ? size_t(K) : 0u}};
  Span out[] = {{workspace, need}};
  if (any_alias(in, 2, out, 1)) return TL_ERR_ALIAS;
  return from_hip(tl::launch_gemv_prepare_rotated(x, b, K, signs, workspace,
                                                  static_cast<hipStream_t>(stream)));
}

int tl_gemv_ternary_x(const uint16_t *x, int64_t b, int64_t K, int64_t N, const int8_t *signs,
                      const uint32_t *packed, const uint16_t *scales, void *y, int y_dtype,
                      void *workspace, size_t workspace_bytes, void *stream) {
  if (int s = check_gemv_shape(b, K, N)) return s;
  if (K % tl::kHBlock) return TL_ERR_SHAPE;
  if (!tl::fused_input_supported(K)) return TL_ERR_UNSUPPORTED;
  if (y_dtype != TL_BF16 && y_dtype != TL_F32) return TL_ERR_DTYPE;
  if (b == 0 || N == 0) return TL_OK;
  if (!x || !packed || !scales || !y) return TL_ERR_NULLPTR;
  const size_t need = tl::gemv_workspace_bytes(b, K, N);
  if (!workspace || workspace_bytes < need) return TL_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(packed) || !aligned16(scales) || !aligned16(y) ||
      !aligned16(workspace) || (signs && !aligned16(signs)))
    return TL_ERR_ALIGN;
  const size_t G = size_t(K / tl::kGroup);
  const size_t ysz = size_t(b) * N * (y_dtype == TL_F32 ? 4 : 2);
  Span in[] = {{x, size_t(b) * K * 2}, {signs, signs ? size_t(K) : 0u},
               {packed, size_t(tl::packed_words(N, K)) * 4}, {scales, size_t(N) * G * 2}};
  Span out[] = {{y, ysz}, {workspace, need}};
  if (any_alias(in, 4, out, 2)) return TL_ERR_ALIAS;
  if (!tl::gemv_rot_supported(b, K, N) && !tl::gemv_supported(b, K, N)) return TL_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (tl::gemv_rot_supported(b, K, N))
    return from_hip(tl::launch_gemv_rot(x, b, K, N, signs, packed, scales, y, y_dtype, st));
  hipError_t e = tl::launch_gemv_prepare_rotated(x, b, K, signs, workspace, st);
  if (e != hipSuccess) return from_hip(e);
  return from_hip(tl::launch_gemv_main(workspace, b, K, N, packed, scales, y, y_dtype, st));
}

int tl_quant_act_int8_x(const uint16_t *x, int64_t T, int64_t K, const int8_t *signs, int8_t *xq,
                        float *tok_scale, void *stream) {
  if (T < 0 || K <= 0 || K % tl::kHBlock || T >= kMaxDim || K >= kMaxDim) return TL_ERR_SHAPE;
  if (!tl::fused_input_supported(K)) return TL_ERR_UNSUPPORTED;
  if (T == 0) return TL_OK;
  if (!x || !xq || !tok_scale) return TL_ERR_NULLPTR;
  if (!aligned16(x) || !aligned16(xq) || !aligned16(tok_scale) || (signs && !aligned16(signs)))
    return TL_ERR_ALIGN;
  Span in[] = {{x, size_t(T) * K * 2}, {signs, signs ? size_t(K) : 0u}};
  Span out[] = {{xq, size_t(T) * K}, {tok_scale, size_t(T) * 4}};
  if (any_alias(in, 2, out, 2)) return TL_ERR_ALIAS;
  return from_hip(tl::launch_quant_x(x, T, K, signs, xq, tok_scale, static_cast<hipStream_t>(stream)));
}

int tl_gemv_ternary_q8(const int8_t *xq, const float *tok_scale, int64_t b, int64_t K, int64_t N,
                       const uint32_t *packed, const uint16_t *scales, void *y, int y_dtype,
                       void *stream) {
  if (int s = check_gemv_shape(b, K, N, tl::kTokChunk)) return s;
  if (y_dtype != TL_BF16 && y_dtype != TL_F32) return TL_ERR_DTYPE;
  if (b == 0 || N == 0) return TL_OK;
  if (!xq || !tok_scale || !packed || !scales || !y) return TL_ERR_NULLPTR;
  if (!aligned16(xq) || !aligned16(packed) || !aligned16(scales) || !aligned16(y)) return TL_ERR_ALIGN;
  if (!tl::gemv_q8_supported(b, K, N)) return TL_ERR_UNSUPPORTED;
  const size_t G = size_t(K / tl::kGroup);
  const size_t ysz = size_t(b) * N * (y_dtype == TL_F32 ? 4 : 2);
  Span in[] = {{xq, size_t(b) * K}, {tok_scale, size_t(b) * 4}, {packed, size_t(tl::packed_words(N, K)) * 4},
               {scales, size_t(N) * G * 2}};
  Span out[] = {{y, ysz}};
  if (any_alias(in, 4, out, 1)) return TL_ERR_ALIAS;
  return from_hip(tl::launch_gemv_q8(xq, tok_scale, b, K, N, packed, scales, y, y_dtype,
                                     static_cast<hipStream_t>(stream)));
}

int tl_quant_act_int8(const float *xr, int64_t T, int64_t K, int8_t *xq, float *tok_scale,
                      void *stream) {
  if (T < 0 || K <= 0 || K % tl::kGroup || T >= kMaxDim || K >= kMaxDim) return TL_ERR_SHAPE;
  if (T == 0) return TL_OK;
  if (!xr || !xq || !tok_scale) return TL_ERR_NULLPTR;
  if (!aligned16(xr) || !aligned16(xq) || !aligned16(tok_scale)) return TL_ERR_ALIGN;
  Span in[] = {{xr, size_t(T) * K * 4}};
  Span out[] = {{xq, size_t(T) * K}, {tok_scale, size_t(T) * 4}};
  if (any_alias(in, 1, out, 2)) return TL_ERR_ALIAS;
  return from_hip(tl::launch_quant(xr, T, K, xq, tok_scale, static_cast<hipStream_t>(stream)));
}

int tl_read_probe(const void *src, size_t bytes, uint32_t *sink, void *stream) {
  if (bytes < 16 || bytes % 16 || bytes / 16 / 512 > 0x7FFFFFFF) return TL_ERR_SHAPE;
  if (!src || !sink) return TL_ERR_NULLPTR;
  if (!aligned16(src) || !aligned16(sink)) return TL_ERR_ALIGN;
  Span in[] = {{src, bytes}};
  Span out[] = {{sink, 4}};
  if (any_alias(in, 1, out, 1)) return TL_ERR_ALIAS;
  return from_hip(tl::launch_read_probe(src, bytes, sink, static_cast<hipStream_t>(stream)));
}

int tl_mfma_probe(int random_operands, int iters, uint32_t *sink, void *stream) {
  if (iters <= 0) return TL_ERR_SHAPE;
  if (!sink) return TL_ERR_NULLPTR;
  if (!aligned16(sink)) return TL_ERR_ALIGN;
  return from_hip(tl::launch_mfma_probe(random_operands ? 1 : 0, iters, sink, static_cast<hipStream_t>(stream)));
}

size_t tl_gemm_workspace_size(int64_t M, int64_t K, int64_t N) {
  if (M < 0 || N < 0 || K <= 0 || K % tl::kGroup) return 0;
  return tl::gemm_workspace_bytes(M, K, N);
}

int tl_gemm_int8_rescale(const int8_t *xq, const float *tok_scale, int64_t M, int64_t K,
                         int64_t N, const uint32_t *packed, const int8_t *q,
                         const float *row_scale, void *y, int y_dtype, int32_t *acc_out,
                         void *workspace, size_t workspace_bytes, void *stream) {
  if (M < 0 || N < 0 || K <= 0 || K % tl::kGroup || K > 133120 || M >= kMaxDim || N >= kMaxDim)
    return TL_ERR_SHAPE;
  if (y_dtype != TL_BF16 && y_dtype != TL_F32) return TL_ERR_DTYPE;
  if (M == 0 || N == 0) return TL_OK;
  if (!xq || !tok_scale || !packed || !q || !row_scale || !y) return TL_ERR_NULLPTR;
  if (!aligned16(xq) || !aligned16(tok_scale) || !aligned16(packed) || !aligned16(q) ||
      !aligned16(row_scale) || !aligned16(y) || (acc_out && !aligned16(acc_out)) ||
      (workspace && !aligned16(workspace)))
    return TL_ERR_ALIGN;
  const size_t need = tl::gemm_workspace_bytes(M, K, N);
  if (need && (!workspace || workspace_bytes < need)) return TL_ERR_WORKSPACE;
  const size_t G = size_t(K / tl::kGroup);
  const size_t ysz = size_t(M) * N * (y_dtype == TL_F32 ? 4 : 2);
  Span in[] = {{xq, size_t(M) * K}, {tok_scale, size_t(M) * 4}, {packed, size_t(tl::packed_words(N, K)) * 4},
               {q, size_t(N) * G}, {row_scale, size_t(N) * 4}};
  Span out[] = {{y, ysz}, {acc_out, acc_out ? size_t(M) * N * 4 : 0u}, {workspace, need}};
  if (any_alias(in, 5, out, 3)) return TL_ERR_ALIAS;
  return from_hip(tl::launch_gemm(xq, tok_scale, M, K, N, packed, q, row_scale, y, y_dtype,
                                  acc_out, workspace, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// whole layer from the raw input, path chosen by the token count
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kLinCounters = 1024;  // the GEMM's split-K counters: kept at offset 0 for both paths

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

struct LinearLayout {
  int path;
  size_t gemm_ws;  // counters + partials (0: the GEMM runs unsplit)
  size_t xq, sx;   // offsets of the int8 path's activations and token scales
  size_t total;
};

LinearLayout linear_layout(int64_t T, int64_t K, int64_t N) {
  LinearLayout l{};
  l.path = tl_linear_path(T, K, N);
  if (l.path == TL_PATH_GEMV) {
    l.total = kLinCounters + tl::gemv_workspace_bytes(T, K, N);
  } else {
    l.gemm_ws = tl::gemm_workspace_bytes(T, K, N);
    l.xq = align256(l.gemm_ws > kLinCounters ? l.gemm_ws : kLinCounters);
    l.sx = l.xq + align256(size_t(T) * K);
    l.total = l.sx + align256(size_t(T) * 4);
  }
  return l;
}

}  // namespace

namespace tl {

size_t linear_scratch_bytes(int64_t T, int64_t K, int64_t N) { return linear_layout(T, K, N).total; }

int linear_check(const uint16_t *x, int64_t T, int64_t K, int64_t N, const uint32_t *packed,
                 const uint16_t *scales, const int8_t *q, const float *row_scale, void *y, int y_dtype) {
  if (T < 0 || N < 0 || K <= 0 || K % tl::kHBlock || T >= kMaxDim || N >= kMaxDim || K >= kMaxDim)
    return TL_ERR_SHAPE;
  if (!tl::fused_input_supported(K)) return TL_ERR_UNSUPPORTED;
  if (y_dtype != TL_BF16 && y_dtype != TL_F32) return TL_ERR_DTYPE;
  if (T == 0 || N == 0) return TL_OK;
  if (!x || !packed || !scales || !q || !row_scale || !y) return TL_ERR_NULLPTR;
  return TL_OK;
}

int linear_run(const uint16_t *x, int64_t T, int64_t K, int64_t N, const int8_t *signs,
               const uint32_t *packed, const uint16_t *scales, const int8_t *q, const float *row_scale,
               void *y, int y_dtype, void *workspace, size_t workspace_bytes, hipStream_t st) {
  const LinearLayout l = linear_layout(T, K, N);
  if (!workspace || workspace_bytes < l.total) return TL_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(packed) || !aligned16(scales) || !aligned16(q) ||
      !aligned16(row_scale) || !aligned16(y) || !aligned16(workspace) || (signs && !aligned16(signs)))
    return TL_ERR_ALIGN;
  const size_t G = size_t(K / tl::kGroup);
  const size_t ysz = size_t(T) * N * (y_dtype == TL_F32 ? 4 : 2);
  Span in[] = {{x, size_t(T) * K * 2}, {signs, signs ? size_t(K) : 0u},
               {packed, size_t(tl::packed_words(N, K)) * 4}, {scales, size_t(N) * G * 2},
               {q, size_t(N) * G}, {row_scale, size_t(N) * 4}};
  Span out[] = {{y, ysz}, {workspace, l.total}};
  if (any_alias(in, 6, out, 2)) return TL_ERR_ALIAS;
  char *ws = static_cast<char *>(workspace);
  if (l.path == TL_PATH_GEMV && !tl::gemv_rot_supported(T, K, N) && !tl::gemv_supported(T, K, N))
    return TL_ERR_UNSUPPORTED;
  if (l.path == TL_PATH_GEMV) {
    if (tl::gemv_rot_supported(T, K, N))
      return from_hip(tl::launch_gemv_rot(x, T, K, N, signs, packed, scales, y, y_dtype, st));
    void *gw = ws + kLinCounters;
    hipError_t e = tl::launch_gemv_prepare_rotated(x, T, K, signs, gw, st);
    if (e != hipSuccess) return from_hip(e);
    return from_hip(tl::launch_gemv_main(gw, T, K, N, packed, scales, y, y_dtype, st));
  }
  int8_t *xq = reinterpret_cast<int8_t *>(ws + l.xq);
  float *sx = reinterpret_cast<float *>(ws + l.sx);
  hipError_t e = tl::launch_quant_x(x, T, K, signs, xq, sx, st);
  if (e != hipSuccess) return from_hip(e);
  return from_hip(tl::launch_gemm(xq, sx, T, K, N, packed, q, row_scale, y, y_dtype, nullptr,
                                  l.gemm_ws ? workspace : nullptr, st));
}

}  // namespace tl

extern "C" {

int tl_linear_path(int64_t T, int64_t K, int64_t N) {
  if (T <= tl::kTokChunk) return TL_PATH_GEMV;
  if (T > tl::kGemvMaxTokens) return TL_PATH_INT8;
  // 17..64 tokens: the GEMV runs one chunk of 16 tokens per grid row, each
  // streaming all N x K weights again, while the int8 path's time hardly grows
  // with T at this size; the GEMV stays ahead up to about 2^27 streamed weights
  // (qkv 5120 x 10240: two chunks; down 17408 x 5120 and gate_up 5120 x 34816:
  // none beyond the first).
  const int64_t streamed = tl::limb_chunks(T) * N * K;
  return streamed <= (int64_t(1) << 27) ? TL_PATH_GEMV : TL_PATH_INT8;
}

size_t tl_linear_workspace_size(int64_t T, int64_t K, int64_t N) {
  if (T < 0 || N < 0 || K <= 0 || K % tl::kHBlock || T >= kMaxDim || N >= kMaxDim) return 0;
  return linear_layout(T, K, N).total;
}

int tl_linear_apply(const uint16_t *x, int64_t T, int64_t K, int64_t N, const int8_t *signs,
                    const uint32_t *packed, const uint16_t *scales, const int8_t *q,
                    const float *row_scale, void *y, int y_dtype, void *workspace,
                    size_t workspace_bytes, void *stream) {
  if (int s = tl::linear_check(x, T, K, N, packed, scales, q, row_scale, y, y_dtype)) return s;
  if (T == 0 || N == 0) return TL_OK;
  return tl::linear_run(x, T, K, N, signs, packed, scales, q, row_scale, y, y_dtype, workspace,
                        workspace_bytes, static_cast<hipStream_t>(stream));
}

}  // extern "C"
