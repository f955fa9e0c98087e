// Library-owned device scratch for rope_sdpa_fwd_noalloc: a file-scope device array that
// takes the place of the caller's workspace for callers that cannot allocate.  Each device
// the library runs on holds its own copy until the process ends.  Its device address is
// looked up once per device (hipGetSymbolAddress, with that device current) and kept; host
// code never uses the array's name as an address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "rs_internal.h"

namespace rs {

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {nullptr};
}  // namespace

int scratch_address(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p || ((uintptr_t)p) % 256 != 0) return (int)hipErrorInvalidValue;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return 0;
}

}  // namespace rs
