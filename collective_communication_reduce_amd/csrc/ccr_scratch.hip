// Fixed device scratch for the entry points that allocate nothing
// (ccr_sendrecv_batch_noalloc): a file-scope device array each GPU holds
// from the library's first use on that device until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address on each GPU comes from hipGetSymbolAddress, taken once per
// device (with that device current) when the first context on it is
// created, and only that address is ever handed to kernels or copies.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ccr_internal.h"

namespace {

__device__ __align__(256) char scratch[ccr::kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
char* g_addr[kMaxDevices] = {};

}  // namespace

namespace ccr {

hipError_t resolve_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_addr[device]) return hipSuccess;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e == hipSuccess) g_addr[device] = static_cast<char*>(p);
  if (cur != device) (void)hipSetDevice(cur);
  return e;
}

char* scratch_address(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  return g_addr[device];
}

}  // namespace ccr
