// The library's own scratch for hs2_full_attn_select_noalloc: one statically sized
// device array per GPU, so that callers which cannot allocate (code under HIP graph
// capture, serving loops that forbid allocation) need no workspace.
//
// In host code the array's name is only a host-side stand-in; its device address
// comes from hipGetSymbolAddress, taken once per device with that device current,
// and only that address is passed to kernels.  Every call on one GPU shares the
// array and it keeps the last call's contents: no kernel of the full layer reads
// workspace memory that the same call has not written first, so nothing is cleared;
// calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "hs2_internal.h"

namespace hs2 {
namespace {

static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace hs2
