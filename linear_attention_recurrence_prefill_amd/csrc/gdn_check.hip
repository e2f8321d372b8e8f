// Device-side checks: the validation of a cu_seqlens table on the device, and the library's
// per-device check words (the debug mode's validation result and the fault flags kernels set).
//
// The pages' library refuses what it cannot run ("How to Speed Up GDN Kernels for Qwen Models",
// section "Using it, and the fine print"), and a packed batch whose boundaries are wrong mixes
// documents ("Step 10 · Making it fast": the packing cross-contamination test).  Offsets that
// only exist on the device cannot be checked by the host before a launch, so this kernel reads
// them on the device and reports what it found.
#include <mutex>

#include "gdn_internal.h"

namespace gdn {

// Per-device words: [0] the last validation status written by the debug mode, [1] fault flags set
// by kernels (kFaultDiagWait: one of the forward kernel's bounded waits between its waves, for the
// diagonal blocks or for the normalised tiles, ran out), [2], [3] unused.  Each device holds its own
// copy; the host reaches it only through the address hipGetSymbolAddress returns on that device.
__device__ __attribute__((aligned(16))) uint32_t check_words[4];

namespace {

constexpr int kMaxDevices = 64;
uint32_t *g_words[kMaxDevices] = {};
std::mutex g_words_mu;

__global__ __launch_bounds__(256) void validate_cu_kernel(const int32_t *__restrict__ cu, int N,
                                                          int64_t T, int32_t *status,
                                                          uint32_t *faults_to_clear) {
  __shared__ uint32_t red;
  if (threadIdx.x == 0) red = 0u;
  __syncthreads();
  uint32_t f = 0u;
  for (int n = threadIdx.x; n < N; n += blockDim.x) {
    const int32_t a = cu[n], b = cu[n + 1];
    if (b < a) f |= kCuDescending;
    if (b < 0 || (int64_t)b > T) f |= kCuOutOfRange;
  }
  if (threadIdx.x == 0) {
    if (cu[0] != 0) f |= kCuFirstNotZero;
    if ((int64_t)cu[N] != T) f |= kCuLastNotTotal;
  }
  if (f) atomicOr(&red, f);
  __syncthreads();
  if (threadIdx.x == 0) {
    *status = (int32_t)red;
    if (faults_to_clear != nullptr) *faults_to_clear = 0u;
  }
}

}  // namespace

hipError_t device_check_words(uint32_t **words) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_words_mu);
  if (g_words[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(check_words));
    if (e != hipSuccess) return e;
    g_words[dev] = static_cast<uint32_t *>(p);
  }
  *words = g_words[dev];
  return hipSuccess;
}

hipError_t launch_validate_cu(const int32_t *cu, int32_t N, int64_t T, int32_t *status,
                              uint32_t *faults_to_clear, hipStream_t stream) {
  hipLaunchKernelGGL(validate_cu_kernel, dim3(1), dim3(256), 0, stream, cu, N, T, status,
                     faults_to_clear);
  return hipGetLastError();
}

}  // namespace gdn
