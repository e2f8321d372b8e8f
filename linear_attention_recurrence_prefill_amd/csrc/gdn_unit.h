// Work-unit lookup shared by the forward and backward kernels.
#pragma once

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

// The sequence with the u-th most chunks, ties in sequence order (u < N <= kMaxLongestFirst).
// Called by one full wave; every lane returns the same result.  Lane l holds the chunk counts of
// sequences l, l + 64, .., and ranks them against every count, broadcast by shuffles.
__device__ inline int seq_by_length(const int32_t *cu, int N, int u, int lane) {
  int len[4], rank[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = lane + 64 * j;
    len[j] = n < N ? max(0, (cu[n + 1] - cu[n] + kChunk - 1) / kChunk) : -1;
    rank[j] = 0;
  }
#pragma unroll
  for (int j2 = 0; j2 < 4; ++j2) {
    if (64 * j2 >= N) break;
    for (int m2 = 0; m2 < 64; ++m2) {
      const int m = 64 * j2 + m2;
      const int lm = __shfl(len[j2], m2, 64);  // -1 past N: ranks no valid sequence
#pragma unroll
      for (int j = 0; j < 4; ++j)
        rank[j] += (lm > len[j] || (lm == len[j] && m < lane + 64 * j)) ? 1 : 0;
    }
  }
  int seq = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint64_t hit = __ballot(lane + 64 * j < N && rank[j] == u);
    if (hit) seq = 64 * j + __builtin_ctzll(hit);
  }
  return seq;
}

// Finds unit u by scanning the sequence table 64 entries at a time.  Called by one full wave;
// every lane returns the same result.  Returns false when u is past the last unit, and also when
// the scanned part of cu_seqlens is malformed (cu[0] != 0, a descending pair, or an offset past
// T): then no unit is found, so no workgroup indexes memory from a bad table.  Every sequence
// before the one returned, and the returned one, have been checked, which bounds the chunk and
// unit counts before it by the ones the host sized its buffers for.  With L == 0 and no chunk
// base asked for, unit u is sequence u without a scan (with longest_first, the sequence with the
// u-th most chunks, N <= kMaxLongestFirst); the caller checks its range.
__device__ inline bool find_unit(const int32_t *cu, int N, int64_t T, int L, int u,
                                 bool need_base, int lane, Unit &out, bool longest_first = false) {
  if (L == 0 && !need_base) {
    if (u >= N) return false;
    const int seq = longest_first ? seq_by_length(cu, N, u, lane) : u;
    out.seq = seq;
    out.c0 = 0;
    out.c1 = max(0, (cu[seq + 1] - cu[seq] + kChunk - 1) / kChunk);
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
