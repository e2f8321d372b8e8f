// Exact split of the forward: the middle pass, which turns every unit's pair (B, M) into the
// true state at the unit's start; and the same walk in reverse for the backward.
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
// The backward's state gradient obeys the transposed map: the gradient at a unit's start is
// M_u^T times the gradient at its end plus B'_u (the unit's own contribution, from a zero end
// gradient), so the reverse walk applies the forward's M transposed.
//
// One workgroup of eight waves per (16-column block, head, sequence): the columns of the state are
// independent under left multiplication by M.  Wave w computes rows 16 w .. 16 w + 15 of the block
// with v_mfma_f32_16x16x32_bf16 on split operands (x = hi + lo, two bf16 each; the product hi hi' +
// hi lo' + lo hi', about 16 significant bits per operand), its rows of M (or M^T) prefetched into
// registers kPre units ahead (the first passes store the maps in the order of these MFMA operands,
// M already split, so each load instruction reads 1 KiB of consecutive bytes and the walk converts
// none of them), so each step waits only for the state of the step before: written to LDS as a bf16
// head and remainder, column-major, in one of two buffers (one barrier per step).  The eight column
// blocks of one (head, sequence) get workgroup ids congruent modulo 8, which round-robin dispatch
// places on one XCD, so their reads of the same M share its L2.
#include "gdn_bwd_internal.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kD = 128;
constexpr int kPre = 4;           // units whose maps are in flight ahead of the one applied
constexpr int kSR = 2 * kD + 16;  // bytes per column of the bf16 state block in LDS (padded)

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

__device__ __forceinline__ f32x4 to_f32x4(bf16x4 x) { return __builtin_convertvector(x, f32x4); }

}  // namespace

// kReverse: the backward's walk, from each sequence's last unit to its first, with the maps
// M_u^T (the forward's M, stored transposed by the first pass of the backward's recompute) and
// B'_u; S is the state gradient at a unit's end and s.h0 the gradient after the sequence.
template <bool kReverse>
__global__ __launch_bounds__(512) void affine_scan_kernel(SplitArgs s) {
  __shared__ __attribute__((aligned(16))) char s_hi[2][16 * kSR];
  __shared__ __attribute__((aligned(16))) char s_lo[2][16 * kSR];
  const int id = blockIdx.x;
  const int cb = (id >> 3) & 7;
  const int64_t pair = (id & 7) + 8 * (int64_t)(id >> 6);
  const int H = s.H;
  if (pair >= (int64_t)H * s.N) return;
  const int h = (int)(pair % H), n = (int)(pair / H);
  const int lane = threadIdx.x & 63, gq = lane >> 4, cl = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int64_t first = 0;
  int count = 0;
  if (!seq_units(s.cu, s.N, s.T, s.L, n, lane, first, count)) return;
  // the same in every lane: scalar registers, so the walk's branches are scalar
  first = (int64_t)__builtin_amdgcn_readfirstlane((unsigned)(first & 0xffffffff)) |
          ((int64_t)__builtin_amdgcn_readfirstlane((unsigned)(first >> 32)) << 32);
  count = __builtin_amdgcn_readfirstlane(count);
  // never past the units the buffers were sized for (a device table that disagrees with the
  // host copy the caller planned with)
  if (first >= s.units) return;
  if (first + count > s.units) count = (int)(s.units - first);
  const int rowC = 16 * w + 4 * gq;  // rows rowC .. rowC + 3 of the result in this lane
  const int col = 16 * cb + cl;
  const int64_t dd = (int64_t)kD * kD;

  f32x4 S = zero4();
  if (s.h0 != nullptr) {
    const float *hp = s.h0 + (int64_t)n * s.h0_stride + (int64_t)h * dd;
#pragma unroll
    for (int i = 0; i < 4; ++i) S[i] = hp[(rowC + i) * kD + col];
  }
  // the start state has landed before any map is fetched, so that no wait for it is left in the
  // walk (where it would also hold back the maps in flight)
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  // the walk's first unit, and the elements between the maps (states) of consecutive steps;
  // the maps are stored in this pass's operand order (map_m_hi_byte, map_b_index): this lane's
  // eight bf16 heads of M for k-step ks are the 16 bytes at float 256 (8 w + 2 ks) + 4 lane and
  // their remainders the 16 bytes at 256 (8 w + 2 ks + 1) + 4 lane, its four entries of B the
  // 16 bytes at 4 (64 (8 cb + w) + lane)
  const int64_t u0 = kReverse ? first + count - 1 : first;
  const int64_t ustep = (kReverse ? -(int64_t)H : (int64_t)H) * dd;
  const float *m0 = s.unit_m + (u0 * H + h) * dd + 256 * 8 * w + 4 * lane;
  const float *b0 = s.unit_b + (u0 * H + h) * dd + 4 * (64 * (8 * cb + w) + lane);
  float *s0 = s.unit_h0 + (u0 * H + h) * dd + (int64_t)rowC * kD + col;
  auto store = [&](int step) {
    float *dst = s0 + step * ustep;
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i * kD] = S[i];
  };
  store(0);
  const int nmaps = count - 1;  // maps applied along the walk
  if (nmaps <= 0) return;
  // The maps of step m (m < nmaps): this lane's eight A-operand items of M (M^T) for each of the
  // four 32-wide k-steps (k = 32 ks + 8 gq + 0..7), and its four entries of B.  Fetches past the
  // last map reload the last one (unused), so the pipeline has no branches.
  f32x4 am[kPre][8], bm[kPre];
  auto fetch = [&](f32x4(&a)[8], f32x4 &b, int m) {
    const int64_t off = min(m, nmaps - 1) * ustep;
#pragma unroll
    for (int q = 0; q < 8; ++q) a[q] = *reinterpret_cast<const f32x4 *>(m0 + off + 256 * q);
    b = *reinterpret_cast<const f32x4 *>(b0 + off);
  };
  // S <- M S + B with the maps of slot j (M^T in the reverse walk); the state goes through LDS as
  // a bf16 head and remainder, column-major, in the buffer of the step's parity
  auto apply = [&](f32x4(&a)[8], f32x4 &b, int parity) {
    char *bh = s_hi[parity], *bl = s_lo[parity];
    {
      const bf16x4 hi = to_bf16x4(S);
      *reinterpret_cast<bf16x4 *>(bh + cl * kSR + rowC * 2) = hi;
      *reinterpret_cast<bf16x4 *>(bl + cl * kSR + rowC * 2) = to_bf16x4(S - to_f32x4(hi));
    }
    __syncthreads();
    f32x4 acc0 = b, acc1 = zero4(), acc2 = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      // M as stored: the k-step's eight bf16 heads, then its eight remainders
      const bf16x8 ahi = __builtin_bit_cast(bf16x8, a[2 * ks]);
      const bf16x8 alo = __builtin_bit_cast(bf16x8, a[2 * ks + 1]);
      const int off = cl * kSR + (32 * ks + 8 * gq) * 2;
      const bf16x8 bhi = *reinterpret_cast<const bf16x8 *>(bh + off);
      const bf16x8 blo = *reinterpret_cast<const bf16x8 *>(bl + off);
      acc0 = mma_bf16(ahi, bhi, acc0);
      acc1 = mma_bf16(ahi, blo, acc1);
      acc2 = mma_bf16(alo, bhi, acc2);
    }
    S = acc0 + (acc1 + acc2);
  };
#pragma unroll
  for (int p = 0; p < kPre; ++p) fetch(am[p], bm[p], p);
  int m = 0;
  for (; m + kPre <= nmaps; m += kPre) {
#pragma unroll
    for (int j = 0; j < kPre; ++j) {
      apply(am[j], bm[j], j & 1);
      fetch(am[j], bm[j], m + j + kPre);
      store(m + j + 1);
    }
  }
  // the remaining maps (fewer than kPre) are in slots 0 .. nmaps - m - 1
#pragma unroll
  for (int j = 0; j < kPre - 1; ++j) {
    if (m + j >= nmaps) break;
    apply(am[j], bm[j], j & 1);
    store(m + j + 1);
  }
}

static_assert(kPre % 2 == 0, "the LDS buffer of a step is chosen by the step's parity");

namespace {
hipError_t launch_scan(const SplitArgs &s, bool reverse, hipStream_t stream) {
  if (s.N <= 0) return hipSuccess;
  const int64_t groups = ((int64_t)s.H * s.N + 7) / 8;
  if (groups * 64 > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(groups * 64));
  if (reverse)
    hipLaunchKernelGGL(affine_scan_kernel<true>, grid, dim3(512), 0, stream, s);
  else
    hipLaunchKernelGGL(affine_scan_kernel<false>, grid, dim3(512), 0, stream, s);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_affine_scan(const SplitArgs &s, hipStream_t stream) {
  return launch_scan(s, false, stream);
}

hipError_t launch_affine_scan_reverse(const SplitArgs &s, hipStream_t stream) {
  return launch_scan(s, true, stream);
}

}  // namespace gdn
