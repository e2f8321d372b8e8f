// Backward of the chunked gated delta rule on gfx950 (in progress: entry points validate and
// report that the backward kernels are not built yet).
#include <hip/hip_runtime.h>

#include "../../include/gdn.h"

extern "C" {

gdn_status gdn_chunk_bwd_workspace_size(const gdn_problem *p, size_t *bytes) {
  if (!p || !bytes) return GDN_ERR_NULL_ARG;
  *bytes = 0;
  return GDN_ERR_BAD_MODE;
}

gdn_status gdn_chunk_bwd(const gdn_problem *p, const void *q, const void *k, const void *v,
                         const float *g, const void *beta, const int32_t *cu_seqlens,
                         const float *h0, const void *dout, const float *dht, void *dq, void *dk,
                         void *dv, float *dg, void *dbeta, float *dh0, void *workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  return GDN_ERR_BAD_MODE;
}
}
