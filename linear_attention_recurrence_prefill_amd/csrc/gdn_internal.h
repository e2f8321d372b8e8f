// Internal interface between the C ABI (gdn_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

constexpr int kChunk = 64;
// eps of the optional q/k L2 normalisation: row / sqrt(|row|^2 + eps)
constexpr float kL2NormEps = 1e-6f;

// Most sequences an unsplit forward takes longest first (the ranking runs in one wave per
// workgroup, four sequences per lane).
constexpr int kMaxLongestFirst = 256;

// Status bits of the cu_seqlens validation (gdn_validate_cu_seqlens).
constexpr uint32_t kCuFirstNotZero = 1u;  // cu[0] != 0
constexpr uint32_t kCuDescending = 2u;    // cu[n + 1] < cu[n] for some n
constexpr uint32_t kCuLastNotTotal = 4u;  // cu[N] != T
constexpr uint32_t kCuOutOfRange = 8u;    // some cu[n + 1] outside [0, T]
// Fault flags kernels set in the per-device check words (gdn_device_faults).
constexpr uint32_t kFaultDiagWait = 1u;   // a bounded wait between the forward's waves ran out

// Bytes of the static device scratch array behind gdn_chunk_fwd_noalloc (gdn_noalloc.hip).
constexpr size_t kStaticScratchBytes = (size_t)128 << 20;
// The current device's address of that array (hipGetSymbolAddress on first use per device).
hipError_t static_scratch(void **ptr);

// The current device's check words ([0] validation status, [1] fault flags), from
// hipGetSymbolAddress on first use per device.
hipError_t device_check_words(uint32_t **words);
// Validates cu [N + 1] against T on the device: writes the status bits to *status (0 = valid),
// and clears *faults_to_clear when not null.
hipError_t launch_validate_cu(const int32_t *cu, int32_t N, int64_t T, int32_t *status,
                              uint32_t *faults_to_clear, hipStream_t stream);

// Arguments of the fused forward kernel.  A "unit" is one (sequence, chunk range) pair: each
// sequence is one unit (L == 0) or is split into units of L chunks; the kernel runs one
// workgroup per (unit, head) and finds its unit from cu_seqlens itself.
struct FwdArgs {
  const void *q, *k, *v;
  const float *g;
  const void *beta;
  const int32_t *cu;
  const float *h0;
  int64_t h0_stride;
  void *o;
  float *ht;
  float *dbg_gamma, *dbg_tmat, *dbg_w, *dbg_u, *dbg_hc, *dbg_delta;  // intermediates (or null)
  uint16_t *dump_hc;  // the pipelined kernel's recompute pass: start states in bf16 [Nc, H, D, D]
  float *dump_rk;     // ... with l2norm: the inverse norms of K's rows [T, HK] (or null)
  int64_t T;
  int32_t N, H;
  int32_t HK;  // heads of q and k (H / HK value heads share one)
  int32_t L;  // segment length in chunks, 0 = whole sequences
  float scale;
  float log_thr;
  int32_t truncate;
  int32_t l2norm;  // q and k rows divided by sqrt(|row|^2 + kL2NormEps) inside the kernel
  // exact split (pipelined kernel only): per-unit start states [units, H, D, D] for the final
  // pass, or the first pass's outputs [2, units, H, D * D] (B from zero in map_b_index order, M
  // from the identity split into bf16 head and remainder, map_m_hi_byte)
  const float *unit_h0;
  float *unit_out;
  int64_t units;
  uint32_t *faults;  // the device's fault flags (kFault*), or null
  // exact split's first pass for the backward: when not null, M^T of every unit but a
  // sequence's first goes here too ([units, H, D * D], split as M; the reverse walk of
  // the state gradient applies M^T), and M is then also formed for each sequence's last unit
  float *unit_mt;
  // unsplit runs of the pipelined kernel: 1 = workgroups take the sequences longest first, with
  // the grid transposed to (H, N) so that every head of the longest sequence starts first
  int32_t longest_first;
};

// Layouts of a unit's maps (B and M, 128 x 128 each, 64 KiB) as the exact split's first passes
// write them and its middle pass reads them: in the order of that pass's MFMA operands, so that
// each of its load instructions reads 1 KiB of consecutive bytes.  The middle pass computes, per
// 16-column block cb of the state and per wave w (rows 16 w .. 16 w + 15), B + M S with
// v_mfma_f32_16x16x32_bf16; lane l = 16 gq + cl takes, of M, row 16 w + cl at k = 32 ks + 8 gq +
// j (j < 8) for the four k-steps ks, and of B, rows 16 w + 4 gq + i (i < 4) of column 16 cb + cl.
// B is fp32.  M is stored split, as the middle pass multiplies it: M = hi + lo with hi = bf16(M)
// and lo = bf16(M - hi); lane l's 32 bytes of k-step ks are the eight heads (item j at bytes 2 j)
// and then the eight remainders, and the k-steps of a wave's rows follow one another in 2 KiB
// units (1 KiB of heads, then 1 KiB of remainders, over the 64 lanes).
// Byte offset of M[r][k]'s head within the map; its remainder is 1 KiB further on.
__host__ __device__ inline int64_t map_m_hi_byte(int r, int k) {
  const int w = r >> 4, cl = r & 15, ks = k >> 5, gq = (k >> 3) & 3, half = (k >> 2) & 1;
  return (((int64_t)(w * 4 + ks) * 2) * 64 + 16 * gq + cl) * 16 + 2 * (4 * half + (k & 3));
}
__host__ __device__ inline int64_t map_b_index(int r, int c) {  // element B[r][c]
  const int cb = c >> 4, w = r >> 4, gq = (r >> 2) & 3;
  return ((int64_t)((cb * 8 + w) * 64 + 16 * gq + (c & 15)) * 4) + (r & 3);
}

// Arguments of the exact split's middle pass (gdn_fwd_split.hip).
struct SplitArgs {
  const int32_t *cu;
  int64_t T;
  int32_t N, H, L;
  const float *h0;
  int64_t h0_stride;
  const float *unit_b;   // [units, H, D * D]: each unit's B (B' in the reverse walk), map_b_index
  const float *unit_m;   // [units, H, D * D]: each unit's M (M^T in the reverse walk), split (map_m_hi_byte)
  float *unit_h0;        // [units, H, D, D]: the true state at each unit's start (end)
  int64_t units;
};

// Arguments of the backward kernels (see gdn_bwd.hip).  Workspace arrays (fp32):
//   gamma [T, H], tmat [Nc, H, 64, 64], w [Nc, H, 64, D], hc [Nc, H, D, D], delta [T, H, D]
//   from the forward recompute; dhn [Nc, H, D, D] (state gradient after each chunk) and
//   ddelta [T, H, D] from the reverse chain.  bf16 inputs with d = 128 keep the per-chunk states
//   in bf16 instead (hc_b16, dhn_b16; hc and dhn null): the products that use them take bf16
//   operands, as the forward's do.
struct BwdArgs {
  const void *q, *k, *v, *beta, *dout;
  const float *g, *dht;
  const int32_t *cu;
  void *dq, *dk, *dv, *dbeta;
  float *dg, *dh0_seq;
  const float *gamma, *tmat, *w, *hc, *delta;
  float *dhn, *ddelta;
  const uint16_t *hc_b16;  // bf16 bit patterns
  uint16_t *dhn_b16;
  // grouped heads (HK < H): dq and dk of every value head, fp32 [T, H, D], summed per key head
  // afterwards (null when HK == H: dq and dk are written directly)
  float *dq_part, *dk_part;
  // q/k L2 normalisation: the inverse row norms 1 / sqrt(|row|^2 + eps) of q and k, fp32 [T, HK]
  // (null: no normalisation).  The kernels fold them into their per-token factors and write
  // r * (gradient of the normalised rows) to dq_part, dk_part; l2norm_bwd_kernel finishes.
  const float *rq, *rk;
  int64_t T;
  int32_t N, H;
  int32_t HK;  // heads of q and k
  float scale;
};

// A work unit: one sequence, or a segment of it (see gdn_unit.h).
struct Unit {
  int seq, c0, c1;      // chunk range [c0, c1) counted from the sequence's first chunk
  int64_t chunk_base;   // index of the sequence's first chunk among all chunks (if asked)
};
// The fused chunked forward over all (unit, head) pairs.
hipError_t launch_fwd(const FwdArgs &a, int D, bool bf16, bool dump, int64_t max_units,
                      hipStream_t stream);

// bf16 forward sized for two workgroups per CU (gdn_fwd_fast.hip); no intermediates.
hipError_t launch_fwd_fast(const FwdArgs &a, int D, int64_t max_units, hipStream_t stream);

// bf16, d = 128: warp-specialised pipeline, one workgroup per CU (gdn_fwd_ws.hip).
hipError_t launch_fwd_ws(const FwdArgs &a, int64_t max_units, hipStream_t stream);
int fwd_ws_blocks_per_cu();
// Exact split: the first pass (B and M of every unit, no output; grid (units, H, 2)) and the
// middle pass (each sequence's units in order: S_start(u + 1) = M_u S_start(u) + B_u).
hipError_t launch_fwd_ws_transition(const FwdArgs &a, int64_t units, hipStream_t stream);
// The backward's recompute on the same pipeline: no output, the per-chunk start states, Delta and
// gamma to a.dbg_hc, a.dbg_delta, a.dbg_gamma (from a.unit_h0 per unit when given).
hipError_t launch_fwd_ws_dump(const FwdArgs &a, int64_t max_units, hipStream_t stream);
hipError_t launch_affine_scan(const SplitArgs &s, hipStream_t stream);

// Workgroups of a forward kernel that fit on one CU at once (from the runtime's occupancy query).
int fwd_blocks_per_cu(int D, bool bf16);
int fwd_fast_blocks_per_cu(int D);

// Writes the plan with warmup windows to out (see gdn_chunk_fwd_plan).
hipError_t launch_plan_export(const int32_t *cu, int32_t N, int64_t T, const float *g, int32_t H,
                              int32_t L, float log_thr, int32_t truncate, int64_t max_units,
                              int32_t *out, int64_t capacity, hipStream_t stream);

// Backward: reverse state-gradient chain (one workgroup per (sequence, head)), per-chunk
// gradients (one workgroup per (chunk, head)) and the sum of dh0 over sequences that share one
// initial state.
hipError_t launch_bwd_chain(const BwdArgs &b, int D, bool bf16, hipStream_t stream);
hipError_t launch_bwd_grad(const BwdArgs &b, int D, bool bf16, int64_t max_chunks,
                           hipStream_t stream);
hipError_t launch_sum_dh0(const float *dh0_seq, int32_t N, int32_t H, int32_t D, float *dh0,
                          hipStream_t stream);
// dst[n] = src[n * src_stride] for N states [H, D, D] (fp32); zeros when src is NULL.
hipError_t launch_copy_states(const float *src, int64_t src_stride, int32_t N, int32_t H,
                              int32_t D, float *dst, hipStream_t stream);
// Grouped heads: out[t, hk, :] = sum over the H / HK value heads of key head hk of part[t, h, :]
// (fixed order), in the input dtype.
// Inverse L2 norms 1 / sqrt(|row|^2 + kL2NormEps) of the `rows` rows of x ([rows, D], bf16 or
// fp32) into r [rows].
hipError_t launch_row_rnorm(const void *x, int64_t rows, int32_t D, bool bf16, float *r,
                            hipStream_t stream);
// Backward of the q/k L2 normalisation, with the per-key-head sum of grouped heads: for each row
// (t, hk) of x [T, HK, D], Z = sum over the H / HK value heads of part [T, H, D] (each holding
// r * the gradient of the normalised row) and dx = Z - r^2 x (x . Z), into out (x's dtype).
hipError_t launch_l2norm_bwd(const float *part, const void *x, const float *r, int64_t T,
                             int32_t H, int32_t HK, int32_t D, bool bf16, void *out,
                             hipStream_t stream);
hipError_t launch_group_sum(const float *part, int64_t T, int32_t H, int32_t HK, int32_t D,
                            bool bf16, void *out, hipStream_t stream);

}  // namespace gdn
