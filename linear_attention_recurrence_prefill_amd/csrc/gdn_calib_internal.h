// Launchers of the calibration kernels (gdn_calib.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// dst[0 .. units16) = src[0 .. units16) in 16-byte units; at most 16 workgroups per CU.
hipError_t launch_calib_copy(const void *src, void *dst, int64_t units16, int cus,
                             hipStream_t stream);
// `waves` one-wave workgroups of `iters` x 4 bf16 32 x 32 x 16 MFMAs each; out holds waves x 64 floats.
hipError_t launch_calib_mfma(float *out, int waves, int iters, hipStream_t stream);

}  // namespace gdn
