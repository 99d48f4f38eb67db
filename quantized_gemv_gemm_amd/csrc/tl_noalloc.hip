// tl_linear_apply_noalloc: the layer entry point with its workspace in a static
// device array instead of a caller buffer, for callers that cannot allocate
// (graph capture, serving loops).  The kernels are tl_linear_apply's.
#include <hip/hip_runtime.h>

#include <mutex>

#include "tl_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB per GPU, held until the process ends
constexpr size_t kCounterBytes = 1024;               // the split-K counter region at its start
constexpr int kMaxDevices = 64;

// The array's name is a host-side stand-in; device code is handed the address
// that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch`, per device (nullptr until set up)

__global__ void zero_words(uint32_t *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// the array's device address on the current device; its counter region is
// zeroed (a kernel on `st`, never a memset) the first time
hipError_t device_scratch(hipStream_t st, void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    const int n = int(kCounterBytes / 4);
    hipLaunchKernelGGL(zero_words, dim3((n + 255) / 256), dim3(256), 0, st, static_cast<uint32_t *>(p), n);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t tl_noalloc_scratch_bytes(void) { return kScratchBytes; }

int tl_linear_apply_noalloc(const uint16_t *x, int64_t T, int64_t K, int64_t N, const int8_t *signs,
                            const uint32_t *packed, const uint16_t *scales, const int8_t *q,
                            const float *row_scale, void *y, int y_dtype, void *stream) {
  if (int s = tl::linear_check(x, T, K, N, packed, scales, q, row_scale, y, y_dtype)) return s;
  if (T == 0 || N == 0) return TL_OK;
  if (tl::linear_scratch_bytes(T, K, N) > kScratchBytes) return TL_ERR_SCRATCH;
  hipStream_t st = static_cast<hipStream_t>(stream);
  void *ws = nullptr;
  if (device_scratch(st, &ws) != hipSuccess) return TL_ERR_LAUNCH;
  return tl::linear_run(x, T, K, N, signs, packed, scales, q, row_scale, y, y_dtype, ws, kScratchBytes, st);
}

}  // extern "C"
