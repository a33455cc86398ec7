// dg_noalloc.hip -- the allocation-free masked-layout entry point.
//
// For callers that cannot allocate device memory while they run (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// the masked MoE decode GEMM with its split-K partials in a fixed scratch
// buffer instead of a buffer from the library's pool, so split K is kept
// where the default entry point drops it (under capture) and no call
// allocates.  The scratch is a file-scope device array, one copy per GPU,
// held until the process ends; every call on a GPU shares it.
#include <mutex>

#include "../../include/dg.h"
#include "dg_kernel.h"

namespace {

constexpr int kMaxDevices = 64;
constexpr size_t kScratchFloats = size_t(1) << 24;  // 64 MB of fp32 split-K partials

static __device__ __align__(256) float scratch[kScratchFloats];

std::mutex g_mutex;
float* g_scratch[kMaxDevices];  // the device address of `scratch` on each GPU

// The current device's copy of `scratch`: its address is looked up once per
// device, with that device current, and used from then on (in host code the
// array's name only stands in for the symbol).  Null if the lookup fails.
float* device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch[dev] = static_cast<float*>(ptr);
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" dg_status dg_grouped_fp8_masked_noalloc(const void* a, const float* sa, const void* b, const float* sb,
                                                   void* c, const int32_t* masked_m, int num_groups, int m_max,
                                                   int n, int k, hipStream_t stream) {
  return dg::grouped_masked(a, sa, b, sb, c, masked_m, num_groups, m_max, n, k, stream, device_scratch,
                            kScratchFloats);
}
