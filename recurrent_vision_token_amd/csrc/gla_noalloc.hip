// gla_chunk_fwd_noalloc: the float16 forward with its span states in a fixed
// device array instead of the workspace cache, for callers that cannot
// allocate (see include/gla.h).  The operation, the kernels and the work
// split are those of gla_chunk_fwd.

#include <hip/hip_runtime.h>

#include <mutex>

#include "gla.h"
#include "gla_internal.h"

// Span states of the no-allocation entry; one copy per device, held until the
// process ends.  In host code this name stands for the device array but is not
// its address: only the pointer hipGetSymbolAddress gives is passed to kernels.
static __device__ __align__(256) float scratch[GLA_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on device dev (the current device), looked up
// once per device; null if the device index is out of range or the lookup fails.
void* scratch_on(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int gla_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                     const void* log_alpha, int scan_dir, int B, int heads, int H,
                                     int W, int d_k, int d_v, int chunk, void* out,
                                     float* final_state, void* stream) {
  return gla::forward_no_alloc(q, k, v, log_alpha, scan_dir, B, heads, H, W, d_k, d_v, chunk, out,
                               final_state, stream, scratch_on, GLA_NOALLOC_SCRATCH_BYTES);
}
