// The workspace of tf_prefill_noalloc: one file-scope device array per GPU, so that entry
// point allocates nothing. The HIP runtime places a copy of the array on every GPU the
// library's code is loaded on and keeps it until the process ends.
#include <mutex>

#include "tf_internal.h"

namespace tfp {

// In host code `scratch` names a host-side stand-in, not device memory: only the address
// hipGetSymbolAddress returns (per device) may be handed to kernels or copies.
static __device__ __align__(256) char scratch[NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_addr[MAX_DEVICES] = {};
}  // namespace

hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    // first call on this device (it is current): the device address of its copy
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255)) return hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  *out = g_addr[dev];
  return hipSuccess;
}

}  // namespace tfp
