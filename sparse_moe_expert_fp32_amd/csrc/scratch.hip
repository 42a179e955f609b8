// The library's fixed device scratch, for the entry point that allocates
// nothing (moe_expert_fwd_noalloc): a file-scope device array that the code
// object carries, so each GPU the library runs on holds one copy of it from
// module load to process end.
//
// In host code `scratch` is only a stand-in symbol, not a device address:
// every host-side use goes through the address that hipGetSymbolAddress
// returns for the current device, looked up once per device and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace moe {

namespace {

__device__ __attribute__((aligned(256))) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace moe
