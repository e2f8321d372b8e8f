// Internal interface between the C ABI (gdn_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kChunk = 64;
constexpr int kPlanHeader = 2;  // plan[0] = number of units, plan[1] = segment length (chunks)

// Arguments of the fused forward kernel.  A "unit" is one (sequence, chunk range) pair from the
// plan; the kernel runs one workgroup per (unit, head).
struct FwdArgs {
  const void *q, *k, *v;
  const float *g;
  const void *beta;
  const int32_t *cu;
  const float *h0;
  int64_t h0_stride;
  void *o;
  float *ht;
  const int32_t *plan;    // [kPlanHeader + 3 * max_units]: seq, first chunk, end chunk
  const int32_t *chunk0;  // [N + 1]: index of each sequence's first chunk among all chunks
  float *dbg_gamma, *dbg_tmat, *dbg_w, *dbg_u, *dbg_hc, *dbg_delta;  // intermediates (or null)
  int64_t T;
  int32_t N, H;
  float scale;
  float log_thr;
  int32_t truncate;
};

// One workgroup: validates cu_seqlens on the device and writes the unit list (every sequence
// split into segments of L chunks, or whole when L == 0) and each sequence's first chunk index.
// An invalid cu_seqlens yields zero units (nothing is computed).
hipError_t launch_plan(const int32_t *cu, int32_t N, int64_t T, int32_t L, int32_t *plan,
                       int32_t *chunk0, int64_t max_units, hipStream_t stream);

// Final states of sequences with no tokens: ht = h0 (or zero).
hipError_t launch_empty_states(const int32_t *cu, int32_t N, int32_t H, int32_t D,
                               const float *h0, int64_t h0_stride, float *ht,
                               hipStream_t stream);

// The fused chunked forward over all (unit, head) pairs.
hipError_t launch_fwd(const FwdArgs &a, int D, bool bf16, bool dump, int64_t max_units,
                      hipStream_t stream);

// Writes the plan with warmup windows to out (see gdn_chunk_fwd_plan).
hipError_t launch_plan_export(const int32_t *plan, const int32_t *cu, const float *g, int32_t H,
                              float log_thr, int32_t truncate, int64_t max_units, int32_t *out,
                              int64_t capacity, hipStream_t stream);

}  // namespace gdn
