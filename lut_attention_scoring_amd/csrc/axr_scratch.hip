// Library-held scratch memory for callers that cannot allocate device memory
// (code under graph capture, serving loops, harnesses that forbid hipMalloc):
// axr_score_softmax_noalloc keeps its split-T partials here instead of in a
// caller workspace.  Each device holds its own copy of the array, at its own
// address, until the process ends.  Host code never passes the array's name
// to a kernel (that name is a host-side stand-in); it uses the device address
// that hipGetSymbolAddress returns, looked up once per device with that
// device current and kept here.

#include <hip/hip_runtime.h>

#include <mutex>

#include "axr_internal.h"

namespace axr {
namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

int scratch_address(void** ptr) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return static_cast<int>(err);
  if (dev < 0 || dev >= kMaxDevices) return static_cast<int>(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return static_cast<int>(err);
    if (p == nullptr) return static_cast<int>(hipErrorInvalidSymbol);
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return 0;
}

}  // namespace axr
