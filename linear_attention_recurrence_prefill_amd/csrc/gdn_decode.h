// Internal interface of the single-token decode step (gdn_decode.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Per (sequence b, head h), sequence-major: q, k [B, HK, D] and v, o [B, H, D] in the input
// dtype, g [B, H] fp32, beta [B, H] in the input dtype, state [B, H, D, D] fp32 (read and
// overwritten).  l2norm: q and k rows divided by sqrt(|row|^2 + kL2NormEps) first.
struct DecodeArgs {
  const void *q, *k, *v;
  const float *g;
  const void *beta;
  float *state;
  void *o;
  int32_t B, H, HK;
  int32_t l2norm;
  float scale;
};

hipError_t launch_decode_step(const DecodeArgs &a, int D, bool bf16, hipStream_t stream);

}  // namespace gdn
