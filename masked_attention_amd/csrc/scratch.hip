// Library-owned scratch memory for rk_masked_attn_fwd_noalloc: one array
// per GPU the library runs on, in place of the caller's attention
// workspace (the rotated keys and the partial results of split items).
// The array is a module global: the runtime places a copy on a GPU when it
// loads this module there and keeps it until the process ends.  Host code
// never uses the array's name as a device address; it asks the runtime for
// the address on the current GPU once and keeps it.
#include <mutex>

#include "rk_internal.h"

static __device__ __align__(256) unsigned char scratch[RK_STATIC_SCRATCH_BYTES];

namespace rk {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices];  // scratch's address on each device, once looked up

}  // namespace

hipError_t static_scratch(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_addr[dev] = ptr;
  }
  *out = g_addr[dev];
  return hipSuccess;
}

}  // namespace rk
