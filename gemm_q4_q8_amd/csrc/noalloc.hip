// The library-owned scratch of lmhead_argmax_noalloc: one file-scope device
// array per GPU, for callers that cannot allocate (code under HIP graph
// capture, serving loops that forbid hipMalloc).
//
// Host code never uses the array's name as an address: the first call on a
// device (with that device current) looks the address up with
// hipGetSymbolAddress and keeps it per device; kernels receive that pointer
// as their workspace argument, as they receive the caller's workspace in
// lmhead_argmax.
#include <mutex>

#include "internal.h"
#include "qgemm.h"

namespace qg {

static __device__ __align__(256) uint8_t scratch[QG_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[MAX_DEVICES];

int noalloc_scratch(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    record_hip_error(e);
    return QG_EHIP;
  }
  if (dev < 0 || dev >= MAX_DEVICES) return QG_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      record_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return QG_EHIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QG_OK;
}

// Zero n words from p (a fill kernel, not hipMemsetAsync, so the call may
// be captured into a HIP graph).
__global__ void __launch_bounds__(256) clear_words_kernel(uint32_t *p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

int launch_clear_words(void *p, int n, hipStream_t stream) {
  if (n <= 0) return QG_OK;
  clear_hip_error();
  hipLaunchKernelGGL(clear_words_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, (uint32_t *)p, n);
  return launch_status();
}

}  // namespace qg
