// Tile movement and scheduling helpers shared by the forward kernels.
#pragma once

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

// Warmup window of a segment starting at chunk c0 > 0 of its sequence ("Lever 1"): whole
// preceding chunks are added one at a time (c0-1, c0-2, ...) until their summed g is below
// thr; returns the window's first chunk (0 when it reaches the sequence start).  One full
// wave calls it; each chunk's sum is formed in fp64 by the same lane-tree on every lane, and
// the chunks are added in order, four chunks' loads in flight at a time.
__device__ inline int warm_window(const float *__restrict__ g, int64_t ts0, int c0, int h, int H,
                                  float thr, int lane) {
  double acc = 0.0;
  int w = c0;
  while (w > 0 && !(acc < (double)thr)) {
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // chunks w - 1 .. w - 4 (those below 0 are not used)
      const int cj = max(w - 1 - j, 0);
      x[j] = g[(ts0 + (int64_t)cj * kChunk + lane) * H + h];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double sj = wave_sum_f64((double)x[j]);
      if (w > 0 && !(acc < (double)thr)) {
        --w;
        acc += sj;
      }
    }
  }
  return w;
}

// The same window on the other side, for the truncate mode's reverse chain: the gradient of the
// state after a segment that ends before chunk c1 < nc of its sequence takes the contributions of
// later chunks through the chunk maps transposed, which decay as the forward maps do.  Whole
// following chunks are added one at a time (c1, c1 + 1, ...) until their summed g is below thr;
// returns the window's end (exclusive; nc when it reaches the sequence end).  Tokens past ts1
// (the sequence's ragged last chunk) add nothing.  One full wave calls it.
__device__ inline int warm_window_rev(const float *__restrict__ g, int64_t ts0, int64_t ts1, int c1,
                                      int nc, int h, int H, float thr, int lane) {
  double acc = 0.0;
  int e = c1;
  while (e < nc && !(acc < (double)thr)) {
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // chunks e .. e + 3 (those at or past nc are not used)
      const int64_t t = ts0 + (int64_t)min(e + j, nc - 1) * kChunk + lane;
      x[j] = t < ts1 ? g[t * H + h] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double sj = wave_sum_f64((double)x[j]);
      if (e < nc && !(acc < (double)thr)) {
        ++e;
        acc += sj;
      }
    }
  }
  return e;
}

// Lower-triangular 16x16 tiles (bi, bj), bj <= bi, of a 64x64 matrix, numbered row by row:
// tau = bi (bi + 1) / 2 + bj, 0 <= tau < 10.
__device__ __forceinline__ int tile_bi(int tau) {
  return tau >= 6 ? 3 : (tau >= 3 ? 2 : (tau >= 1 ? 1 : 0));
}
__device__ __forceinline__ int tile_bj(int tau) {
  const int bi = tile_bi(tau);
  return tau - bi * (bi + 1) / 2;
}

template <class E, int D, int LDE>
__device__ __forceinline__ void load_tile(E *__restrict__ dst, const E *__restrict__ src,
                                          int64_t t0, int n, int h, int H, int tid) {
  constexpr int EPU = 16 / (int)sizeof(E);  // elements per 16-byte unit
  constexpr int UPR = D / EPU;              // units per row
#pragma unroll
  for (int u = tid; u < 64 * UPR; u += 256) {
    const int r = u / UPR, cu16 = u % UPR;
    uint4 val = {0u, 0u, 0u, 0u};
    if (r < n) val = *reinterpret_cast<const uint4 *>(src + ((t0 + r) * H + h) * D + cu16 * EPU);
    *reinterpret_cast<uint4 *>(dst + r * LDE + cu16 * EPU) = val;
  }
}

template <class E, int D, int LDE>
__device__ __forceinline__ void store_tile(E *__restrict__ dst, const E *__restrict__ src,
                                           int64_t t0, int n, int h, int H, int tid) {
  constexpr int EPU = 16 / (int)sizeof(E);
  constexpr int UPR = D / EPU;
#pragma unroll
  for (int u = tid; u < 64 * UPR; u += 256) {
    const int r = u / UPR, cu16 = u % UPR;
    if (r < n)
      *reinterpret_cast<uint4 *>(dst + ((t0 + r) * H + h) * D + cu16 * EPU) =
          *reinterpret_cast<const uint4 *>(src + r * LDE + cu16 * EPU);
  }
}

}  // namespace gdn
