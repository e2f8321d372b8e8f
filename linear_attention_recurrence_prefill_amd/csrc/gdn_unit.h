// Work-unit lookup shared by the forward and backward kernels.
#pragma once

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

// Finds unit u by scanning the sequence table 64 entries at a time.  Called by one full wave;
// every lane returns the same result.  Returns false when u is past the last unit, and also when
// the scanned part of cu_seqlens is malformed (cu[0] != 0, a descending pair, or an offset past
// T): then no unit is found, so no workgroup indexes memory from a bad table.  Every sequence
// before the one returned, and the returned one, have been checked, which bounds the chunk and
// unit counts before it by the ones the host sized its buffers for.  With L == 0 and no chunk
// base asked for, unit u is sequence u without a scan; the caller checks its range.
__device__ inline bool find_unit(const int32_t *cu, int N, int64_t T, int L, int u,
                                 bool need_base, int lane, Unit &out) {
  if (L == 0 && !need_base) {
    if (u >= N) return false;
    out.seq = u;
    out.c0 = 0;
    out.c1 = max(0, (cu[u + 1] - cu[u] + kChunk - 1) / kChunk);
    out.chunk_base = 0;
    return true;
  }
  if (cu[0] != 0) return false;
  int64_t units_before = 0, chunks_before = 0;
  for (int base = 0; base < N; base += 64) {
    const int n = base + lane;
    int ch = 0, un = 0;
    bool bad = false;
    if (n < N) {
      const int a = cu[n], b = cu[n + 1];
      bad = b < a || (int64_t)b > T;
      ch = bad ? 0 : (b - a + kChunk - 1) / kChunk;
      un = L > 0 ? max(1, (ch + L - 1) / L) : 1;
    }
    if (__ballot(bad)) return false;
    int sun = un, sch = ch;  // inclusive scans over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int a = __shfl_up(sun, off, 64), b = __shfl_up(sch, off, 64);
      if (lane >= off) {
        sun += a;
        sch += b;
      }
    }
    const uint64_t hit = __ballot(n < N && units_before + sun > u);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      const int seq = base + l;
      const int ch_s = __shfl(ch, l, 64);
      const int64_t first_unit = units_before + __shfl(sun - un, l, 64);
      const int s = (int)(u - first_unit);
      out.seq = seq;
      out.c0 = L > 0 ? s * L : 0;
      out.c1 = L > 0 ? min(ch_s, (s + 1) * L) : ch_s;
      out.chunk_base = chunks_before + __shfl(sch - ch, l, 64);
      return true;
    }
    units_before += __shfl(sun, 63, 64);
    chunks_before += __shfl(sch, 63, 64);
  }
  return false;
}

}  // namespace gdn
