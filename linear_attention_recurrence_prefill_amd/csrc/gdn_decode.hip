// Single-token decode step of the gated delta rule on gfx950: every (sequence, head) state
// advances by one token, in place.  "How to Speed Up GDN Kernels for Qwen Models" (section
// "FAQ") sets decode apart as its own regime: one token, the recurrent step.
//
// Per state S (d x d fp32) with the token's q, k, v, g, beta:
//     S' = e^g (I - beta k k^T) S + beta k v^T,     o = scale S'^T q.
// With u = k^T S and w = q^T S (one pass over S gives both) this is
//     t  = v - e^g u,    S' = e^g S + beta k t^T,    o = scale (e^g w + beta (q . k) t),
// so S is read once and written once: the step is bound by HBM bandwidth (2 d^2 fp32 per state).
// With the q/k L2 normalisation, q = rq q_in and k = rk k_in with the rows' inverse norms: the
// factors fold into u, w, q . k and beta, and the rows are never rewritten.
//
// One workgroup of 256 threads per (sequence, head).  Thread (row group rg, column group cg)
// holds rows rg * RPT .. + RPT - 1 of columns 4 cg .. 4 cg + 3 in registers (16-byte loads and
// stores; a wave covers whole 512-byte rows); the column sums u and w are reduced across row
// groups through LDS in a fixed order.
#include "gdn_decode.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

__device__ __forceinline__ float ld_any(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_any(const bf16 *p, int64_t i) { return (float)p[i]; }
__device__ __forceinline__ void st_any(float *p, int64_t i, float x) { p[i] = x; }
__device__ __forceinline__ void st_any(bf16 *p, int64_t i, float x) { p[i] = (bf16)x; }

}  // namespace

template <int D, class E>
__global__ __launch_bounds__(256) void decode_step_kernel(DecodeArgs a) {
  constexpr int CG = D / 4;      // column groups of 4
  constexpr int RG = 256 / CG;   // row groups
  constexpr int RPT = D / RG;    // rows per thread
  __shared__ float sq[D], sk[D], sv[D], st[D];
  __shared__ __attribute__((aligned(16))) float pu[RG][D], pw[RG][D];
  __shared__ float sqk, srq, srk;
  const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG;
  const int64_t bh = blockIdx.x;  // (sequence, head) pair, sequence-major
  const int64_t bk = bh / a.H * a.HK + (int)(bh % a.H) / (a.H / a.HK);  // (sequence, key head)
  const E *q = static_cast<const E *>(a.q) + bk * D;
  const E *k = static_cast<const E *>(a.k) + bk * D;
  const E *v = static_cast<const E *>(a.v) + bh * D;
  float *S = a.state + bh * D * D;
  if (tid < D) {
    sq[tid] = ld_any(q, tid);
    sk[tid] = ld_any(k, tid);
    sv[tid] = ld_any(v, tid);
  }
  // this thread's block of the state
  f32x4 x[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    x[i] = *reinterpret_cast<const f32x4 *>(S + (int64_t)(rg * RPT + i) * D + 4 * cg);
  const float eg = __expf(a.g[bh]);
  const float beta = ld_any(static_cast<const E *>(a.beta), bh);
  __syncthreads();
  if (tid < 64) {  // q . k (and |q|^2, |k|^2 for the normalisation), fixed order
    float s = 0.f, nq = 0.f, nk = 0.f;
    for (int i = tid; i < D; i += 64) {
      s += sq[i] * sk[i];
      nq += sq[i] * sq[i];
      nk += sk[i] * sk[i];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      s += __shfl_xor(s, off, 64);
      nq += __shfl_xor(nq, off, 64);
      nk += __shfl_xor(nk, off, 64);
    }
    if (tid == 0) {
      const float rq = a.l2norm ? 1.f / sqrtf(nq + kL2NormEps) : 1.f;
      const float rk = a.l2norm ? 1.f / sqrtf(nk + kL2NormEps) : 1.f;
      sqk = rq * rk * s;
      srq = rq;
      srk = rk;
    }
  }
  f32x4 u = zero4(), w = zero4();
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg * RPT + i;
    u += sk[r] * x[i];
    w += sq[r] * x[i];
  }
  *reinterpret_cast<f32x4 *>(&pu[rg][4 * cg]) = u;
  *reinterpret_cast<f32x4 *>(&pw[rg][4 * cg]) = w;
  __syncthreads();
  if (tid < D) {
    float us = 0.f, ws = 0.f;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      us += pu[g][tid];
      ws += pw[g][tid];
    }
    us *= srk;  // the normalised rows' u and w (factors 1 without the normalisation)
    ws *= srq;
    const float t = sv[tid] - eg * us;
    st[tid] = beta * srk * t;
    st_any(static_cast<E *>(a.o) + bh * D, tid, a.scale * (eg * ws + beta * sqk * t));
  }
  __syncthreads();
  const f32x4 bt = *reinterpret_cast<const f32x4 *>(&st[4 * cg]);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg * RPT + i;
    *reinterpret_cast<f32x4 *>(S + (int64_t)r * D + 4 * cg) = eg * x[i] + sk[r] * bt;
  }
}

hipError_t launch_decode_step(const DecodeArgs &a, int D, bool is_bf16, hipStream_t stream) {
  const int64_t n = (int64_t)a.B * a.H;
  if (n <= 0) return hipSuccess;
  const dim3 grid((unsigned)n), block(256);
  if (D == 128) {
    if (is_bf16) hipLaunchKernelGGL((decode_step_kernel<128, bf16>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((decode_step_kernel<128, float>), grid, block, 0, stream, a);
  } else {
    if (is_bf16) hipLaunchKernelGGL((decode_step_kernel<64, bf16>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((decode_step_kernel<64, float>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace gdn
