// The forward for callers that cannot allocate (code under HIP graph capture, serving loops,
// harnesses that forbid hipMalloc): gdn_chunk_fwd_noalloc runs gdn_chunk_fwd with its workspace
// in a static device array of fixed size instead of caller memory.
//
// The array lives in device memory of every GPU the library is loaded on, for the life of the
// process.  In host code its name is only a stand-in for the symbol, never a device address: the
// address comes from hipGetSymbolAddress, called once per device with that device current, and
// only that address is handed to kernels.  Every call on one device shares that device's array
// (and it keeps the last call's contents), so calls that overlap on one device race.
#include <mutex>

#include "gdn_internal.h"

namespace gdn {
namespace {

__device__ __attribute__((aligned(256))) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
void *g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

}  // namespace

hipError_t static_scratch(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace gdn
