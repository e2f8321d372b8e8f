// Exact split of the forward: the middle pass, which turns every unit's pair (B, M) into the
// true state at the unit's start.
//
// The recurrence over one unit's chunks is affine in the state it starts from: after the unit
// the state is M S_start + B, with B the state reached from zero and M the state reached from
// the identity with V = 0 (the product of the chunks' transitions e^{gamma_last} I - K'^T W of
// "How to Speed Up GDN Kernels for Qwen Models", section "What GDN actually computes", with
// K' = diag(e^{gamma_last - gamma}) K).  The first pass computes (B, M) for all units at once,
// this pass walks each sequence's units in order, S_start(u + 1) = M_u S_start(u) + B_u from
// the sequence's initial state, and the last pass reruns every unit from its true start with
// the output.  The result equals the unsplit recurrence up to rounding.
//
// One workgroup per (16-column block, head, sequence): the columns of the state are independent
// under left multiplication by M, so the eight column blocks of a head walk the units without
// talking to each other.  Eight waves, wave w owning state rows 16 w .. 16 w + 15 of the block,
// products in fp32 (v_mfma_f32_16x16x4_f32).
#include "gdn_bwd_internal.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kD = 128;
constexpr int kLS = kD + 4;  // fp32 row stride of the transposed column block in LDS

// Units of sequence n for segment length L (max(1, ceil(chunks / L)) each, in sequence order, as
// the forward's unit lookup numbers them): the first unit's index and the count.  Called by one
// full wave; every lane returns the same result.  Returns false when cu_seqlens is malformed up to
// and including sequence n (cu[0] != 0, a descending pair or an offset past T), as the unit
// lookup of the other passes does.
__device__ bool seq_units(const int32_t *cu, int N, int64_t T, int L, int n, int lane,
                          int64_t &first, int &count) {
  if (cu[0] != 0) return false;
  auto bad = [&](int m) { return cu[m + 1] < cu[m] || (int64_t)cu[m + 1] > T; };
  auto units_of = [&](int m) {
    const int ch = max(0, (cu[m + 1] - cu[m] + kChunk - 1) / kChunk);
    return max(1, (ch + L - 1) / L);
  };
  int64_t before = 0;
  for (int base = 0; base <= n; base += 64) {
    const int m = base + lane;
    if (__ballot(m <= n && bad(m))) return false;
    int x = m < n ? units_of(m) : 0;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    before += x;
  }
  first = before;
  count = units_of(n);
  return true;
}

}  // namespace

// kReverse: the backward's walk, from each sequence's last unit to its first (the maps are the
// reverse chain's, S the state gradient at a unit's end, s.h0 the gradient after the sequence).
template <bool kReverse>
__global__ __launch_bounds__(512) void affine_scan_kernel(SplitArgs s) {
  __shared__ __attribute__((aligned(16))) float st[16 * kLS];  // st[col * kLS + row]
  const int cb = blockIdx.x, h = blockIdx.y, n = blockIdx.z, H = s.H;
  const int lane = threadIdx.x & 63, gq = lane >> 4, cl = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t first = 0;
  int count = 0;
  if (!seq_units(s.cu, s.N, s.T, s.L, n, lane, first, count)) return;
  // never past the units the buffers were sized for (a device table that disagrees with the
  // host copy the caller planned with)
  if (first >= s.units) return;
  if (first + count > s.units) count = (int)(s.units - first);
  const int row0 = 16 * w + 4 * gq, col = 16 * cb + cl;  // this lane: rows row0 .. row0 + 3
  const int64_t dd = (int64_t)kD * kD;

  f32x4 S = zero4();
  if (s.h0 != nullptr) {
    const float *hp = s.h0 + (int64_t)n * s.h0_stride + h * dd;
#pragma unroll
    for (int i = 0; i < 4; ++i) S[i] = hp[(row0 + i) * kD + col];
  }
  for (int step = 0; step < count; ++step) {
    const int64_t u = first + (kReverse ? count - 1 - step : step);
    float *dst = s.unit_h0 + (u * H + h) * dd;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[(row0 + i) * kD + col] = S[i];
    if (step + 1 == count) break;
    // S <- M_u S + B_u.  The contraction index of MFMA j of block b is 16 b + 4 gq + j on both
    // operands, so that each lane reads 4 consecutive entries of M's row and of S's column.
    *reinterpret_cast<f32x4 *>(&st[cl * kLS + row0]) = S;
    __syncthreads();
    const float *Mu = s.unit_bm + ((s.units + u) * H + h) * dd;
    const float *Bu = s.unit_bm + (u * H + h) * dd;
    f32x4 acc;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = Bu[(row0 + i) * kD + col];
    const float *mrow = Mu + (int64_t)(16 * w + cl) * kD + 4 * gq;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const f32x4 a4 = *reinterpret_cast<const f32x4 *>(mrow + 16 * b);
      const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&st[cl * kLS + 16 * b + 4 * gq]);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = mma_f32(a4[j], b4[j], acc);
    }
    __syncthreads();  // every wave has read the block before it is overwritten
    S = acc;
  }
}

hipError_t launch_affine_scan(const SplitArgs &s, hipStream_t stream) {
  if (s.N <= 0) return hipSuccess;
  hipLaunchKernelGGL(affine_scan_kernel<false>, dim3(kD / 16, s.H, s.N), dim3(512), 0, stream, s);
  return hipGetLastError();
}

hipError_t launch_affine_scan_reverse(const SplitArgs &s, hipStream_t stream) {
  if (s.N <= 0) return hipSuccess;
  hipLaunchKernelGGL(affine_scan_kernel<true>, dim3(kD / 16, s.H, s.N), dim3(512), 0, stream, s);
  return hipGetLastError();
}

}  // namespace gdn
