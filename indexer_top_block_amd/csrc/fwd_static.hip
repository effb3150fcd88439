// The library's static scratch: device memory that sparse_attn_fwd_noalloc uses for
// the split-KV partial results instead of a caller workspace, for callers that
// cannot allocate.  Each GPU the library runs on holds its own copy of the array
// (SA_STATIC_SCRATCH_BYTES) until the process ends.
//
// In host code the array's name is only a host-side stand-in: its device address on
// the current GPU comes from hipGetSymbolAddress, looked up once per device and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sa_launch.hpp"
#include "sparse_attn.h"

static __device__ __align__(256) unsigned char scratch[SA_STATIC_SCRATCH_BYTES];

namespace sa {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with `dev` current: this device's copy
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace sa
