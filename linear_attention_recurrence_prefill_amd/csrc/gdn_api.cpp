// C ABI of the gated delta rule library: argument validation, workspace sizing, the segment
// plan's host-side parameters and kernel dispatch.  Declarations and conventions: include/gdn.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/gdn.h"
#include "../../include/gdn_calib.h"
#include "gdn_bwd_internal.h"
#include "gdn_calib_internal.h"
#include "gdn_decode.h"
#include "gdn_internal.h"

static_assert(GDN_NOALLOC_SCRATCH_BYTES == gdn::kStaticScratchBytes,
              "the header's scratch size is the library's");

namespace {

thread_local char g_err[512] = "";

gdn_status fail(gdn_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

gdn_status hip_fail(hipError_t e, const char *what) {
  return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Debug mode (GDN_DEBUG=1 in the environment, or gdn_set_debug): every compute call first
// validates cu_seqlens on the device and returns GDN_ERR_BAD_SHAPE before any compute launch if
// it is malformed or differs from the host copy the call was given, and after its launches
// synchronises the stream and returns GDN_ERR_DEVICE_CHECK if a kernel set a fault flag.
std::atomic<int> g_debug{-1};

bool debug_on() {
  int d = g_debug.load(std::memory_order_relaxed);
  if (d < 0) {
    const char *e = std::getenv("GDN_DEBUG");
    d = (e != nullptr && e[0] != '\0' && std::strcmp(e, "0") != 0) ? 1 : 0;
    int expected = -1;
    g_debug.compare_exchange_strong(expected, d);
    d = g_debug.load(std::memory_order_relaxed);
  }
  return d == 1;
}

gdn_status debug_validate(const int32_t *cu, int32_t N, int64_t T, const int32_t *cu_host,
                          hipStream_t stream) {
  uint32_t *words = nullptr;
  hipError_t e = gdn::device_check_words(&words);
  if (e != hipSuccess) return hip_fail(e, "debug mode: check words");
  e = gdn::launch_validate_cu(cu, N, T, reinterpret_cast<int32_t *>(words), words + 1, stream);
  if (e != hipSuccess) return hip_fail(e, "debug mode: cu_seqlens validation launch");
  uint32_t status = 0;
  e = hipMemcpyAsync(&status, words, sizeof(status), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "debug mode: cu_seqlens validation");
  if (status != 0)
    return fail(GDN_ERR_BAD_SHAPE,
                "cu_seqlens on the device is malformed (flags 0x%x:%s%s%s%s); nothing launched",
                status, (status & gdn::kCuFirstNotZero) ? " cu[0] != 0" : "",
                (status & gdn::kCuDescending) ? " descending offsets" : "",
                (status & gdn::kCuLastNotTotal) ? " cu[N] != total_tokens" : "",
                (status & gdn::kCuOutOfRange) ? " offsets outside [0, total_tokens]" : "");
  if (cu_host != nullptr) {  // the host copy plans the split: it must be the device table
    int32_t part[1024];      // read back in pieces, with no allocation
    for (int64_t i0 = 0; i0 <= N; i0 += 1024) {
      const int64_t cnt = std::min<int64_t>(1024, (int64_t)N + 1 - i0);
      e = hipMemcpyAsync(part, cu + i0, sizeof(int32_t) * cnt, hipMemcpyDeviceToHost, stream);
      if (e == hipSuccess) e = hipStreamSynchronize(stream);
      if (e != hipSuccess) return hip_fail(e, "debug mode: cu_seqlens read-back");
      for (int64_t i = 0; i < cnt; ++i)
        if (part[i] != cu_host[i0 + i])
          return fail(GDN_ERR_BAD_SHAPE,
                      "cu_seqlens_host[%lld] = %d differs from the device cu_seqlens (%d); "
                      "nothing launched",
                      (long long)(i0 + i), cu_host[i0 + i], part[i]);
    }
  }
  return GDN_OK;
}

gdn_status debug_faults(hipStream_t stream) {
  uint32_t *words = nullptr;
  hipError_t e = gdn::device_check_words(&words);
  if (e != hipSuccess) return hip_fail(e, "debug mode: check words");
  uint32_t flags = 0;
  e = hipMemcpyAsync(&flags, words + 1, sizeof(flags), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "debug mode: fault flags");
  if (flags != 0)
    return fail(GDN_ERR_DEVICE_CHECK, "a kernel set fault flags 0x%x%s", flags,
                (flags & gdn::kFaultDiagWait) ? " (a bounded wait between the forward "
                                                "kernel's waves ran out)" : "");
  return GDN_OK;
}

uint32_t *fault_word() {
  uint32_t *words = nullptr;
  return gdn::device_check_words(&words) == hipSuccess ? words + 1 : nullptr;
}

// Per-device properties cache: is the device gfx950, and its CU count.
struct DevInfo {
  int checked = 0;
  int is_gfx950 = 0;
  int cus = 0;
};
constexpr int kMaxDevices = 64;
DevInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

gdn_status device_info(int *cus);

// The forward kernel a problem runs on: for bf16 inputs the warp-specialised pipeline (d = 128)
// or the 8-wave kernel (d = 64); otherwise the general kernel (fp32 inputs, and the variant that
// writes intermediates).
enum class FwdKernel { kGeneral, kFast, kPipelined };
FwdKernel fwd_kernel_for(const gdn_problem *p, bool dump) {
  if (p->dtype != GDN_DTYPE_BF16 || dump) return FwdKernel::kGeneral;
  return p->d_k == 128 ? FwdKernel::kPipelined : FwdKernel::kFast;
}

// P of the latency model: workgroups that run at once = CUs x resident workgroups per CU.
gdn_status parallel_slots(const gdn_problem *p, bool dump, int *slots) {
  if (p->num_slots > 0) {
    *slots = p->num_slots;
    return GDN_OK;
  }
  int cus = 0;
  gdn_status s = device_info(&cus);
  if (s != GDN_OK) return s;
  int per_cu = 1;
  switch (fwd_kernel_for(p, dump)) {
    case FwdKernel::kPipelined: per_cu = gdn::fwd_ws_blocks_per_cu(); break;
    case FwdKernel::kFast: per_cu = gdn::fwd_fast_blocks_per_cu(p->d_k); break;
    default: per_cu = gdn::fwd_blocks_per_cu(p->d_k, p->dtype == GDN_DTYPE_BF16);
  }
  *slots = cus * per_cu;
  return GDN_OK;
}

gdn_status device_info(int *cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(GDN_ERR_UNSUPPORTED_ARCH, "device %d", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DevInfo &d = g_dev[dev];
  if (!d.checked) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    d.is_gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cus = prop.multiProcessorCount;
    d.checked = 1;
  }
  if (!d.is_gfx950) return fail(GDN_ERR_UNSUPPORTED_ARCH, "device %d is not gfx950", dev);
  if (cus) *cus = d.cus;
  return GDN_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

gdn_status check_problem(const gdn_problem *p) {
  if (!p) return fail(GDN_ERR_NULL_ARG, "problem is NULL");
  if (p->total_tokens < 0 || p->total_tokens > INT32_MAX)
    return fail(GDN_ERR_BAD_SHAPE, "total_tokens %lld out of range", (long long)p->total_tokens);
  if (p->num_seqs < 1) return fail(GDN_ERR_BAD_SHAPE, "num_seqs must be >= 1");
  if (p->num_heads < 1 || p->num_heads > 65535)
    return fail(GDN_ERR_BAD_SHAPE, "num_heads must be in [1, 65535]");
  if (!((p->d_k == 64 || p->d_k == 128) && p->d_v == p->d_k))
    return fail(GDN_ERR_BAD_SHAPE, "head dims must be d_k = d_v in {64, 128}");
  if (p->chunk != gdn::kChunk) return fail(GDN_ERR_BAD_SHAPE, "chunk must be 64");
  if (p->dtype != GDN_DTYPE_F32 && p->dtype != GDN_DTYPE_BF16)
    return fail(GDN_ERR_BAD_DTYPE, "dtype %d", p->dtype);
  if (p->mode != GDN_MODE_EXACT && p->mode != GDN_MODE_TRUNCATE)
    return fail(GDN_ERR_BAD_MODE, "mode %d", p->mode);
  if (p->mode == GDN_MODE_TRUNCATE && !(p->trunc_log_threshold < 0.f))
    return fail(GDN_ERR_BAD_MODE, "trunc_log_threshold must be negative");
  if (p->seg_chunks < 0 || p->num_slots < 0)
    return fail(GDN_ERR_BAD_SHAPE, "seg_chunks / num_slots out of range");
  if (p->num_k_heads < 0 || p->num_k_heads > p->num_heads ||
      (p->num_k_heads > 0 && p->num_heads % p->num_k_heads != 0))
    return fail(GDN_ERR_BAD_SHAPE, "num_k_heads must be 0 or a divisor of num_heads");
  if (p->qk_l2norm != 0 && p->qk_l2norm != 1)
    return fail(GDN_ERR_BAD_MODE, "qk_l2norm must be 0 or 1");
  if (p->reserved != 0) return fail(GDN_ERR_BAD_SHAPE, "reserved must be 0");
  if (p->h0_seq_stride < 0) return fail(GDN_ERR_BAD_SHAPE, "h0_seq_stride must be >= 0");
  if (!std::isfinite(p->scale)) return fail(GDN_ERR_BAD_SHAPE, "scale must be finite");
  return GDN_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Heads of q and k (num_k_heads, 0 meaning one per value head).
int32_t k_heads(const gdn_problem *p) { return p->num_k_heads > 0 ? p->num_k_heads : p->num_heads; }

// Number of chunks: exact from the host copy of cu_seqlens, else ceil(T / 64).
int64_t count_chunks(const gdn_problem *p, const int32_t *cu_host) {
  if (!cu_host) return ceil_div(p->total_tokens, gdn::kChunk);
  int64_t nc = 0;
  for (int32_t n = 0; n < p->num_seqs; ++n) nc += ceil_div(cu_host[n + 1] - cu_host[n], gdn::kChunk);
  return nc;
}

// Segment length of the truncate mode ("How to Speed Up GDN Kernels for Qwen Models", section
// "Lever 1"): the latency-optimal length is proportional to sqrt(H * Nc / P); it is scaled by 3,
// rounded to the nearest power of two in log2 and floored at 4 chunks, and the split is used
// only when num_seqs * H does not fill the P workgroup slots.  Returns 0 for no split.  The exact
// mode splits by the same rule where the exact split is available (see split_available).
int32_t segment_chunks(const gdn_problem *p, int64_t nchunks, int32_t P, bool split_ok) {
  if (p->mode != GDN_MODE_TRUNCATE && !(p->mode == GDN_MODE_EXACT && split_ok)) return 0;
  if (p->seg_chunks > 0) return p->seg_chunks;
  if ((int64_t)p->num_seqs * p->num_heads >= P) return 0;
  const double lstar = 3.0 * std::sqrt((double)p->num_heads * (double)nchunks / (double)P);
  const int e = (int)std::floor(std::log2(lstar) + 0.5);
  int32_t L = (int32_t)std::ldexp(1.0, e);
  return L < 4 ? 4 : L;
}

// Units (workgroups per head) of the plan: a sequence of c chunks gives max(1, ceil(c / L))
// units (one when L == 0).  Exact with the host copy of cu_seqlens, else an upper bound.
int64_t max_units(const gdn_problem *p, const int32_t *cu_host, int32_t L) {
  if (L <= 0) return p->num_seqs;
  if (cu_host) {
    int64_t u = 0;
    for (int32_t n = 0; n < p->num_seqs; ++n) {
      const int64_t c = ceil_div(cu_host[n + 1] - cu_host[n], gdn::kChunk);
      u += c > 0 ? ceil_div(c, L) : 1;
    }
    return u;
  }
  return ceil_div(ceil_div(p->total_tokens, gdn::kChunk) + p->num_seqs, L) + p->num_seqs;
}

// Segment length of the exact split, forward and backward (a design of this library: the split
// is not on the pages).  The split's last pass runs one workgroup per (unit, head), as the
// truncate mode does, after a first pass with one or two workgroups per (unit, head) and a walk
// along each sequence's units; one workgroup fits per CU.  The length is the smallest one, not
// below the latency model's, for which the last pass's workgroups fit in one round of the P
// slots: a second, partly filled round costs a whole segment's time, while a round with fewer
// workgroups runs each chunk faster.  Measured on the 65K-token training batch (six documents,
// 8 heads): forward 0.365 ms at 16 chunks, 0.276 ms at 35 (this rule), 0.320 ms at 64; backward
// 2.21 ms at 16, 1.95 ms at 36.  The latency model's floor keeps the walk along a sequence short
// when there are few heads.  Exact unit counts need the host copy of cu_seqlens; without it the
// unit bound makes the length somewhat longer.
int32_t exact_segment_chunks(const gdn_problem *p, const int32_t *cu_host, int32_t L, int32_t P) {
  if (L <= 0 || p->seg_chunks > 0) return L;
  const auto fits = [&](int64_t len) { return max_units(p, cu_host, (int32_t)len) * p->num_heads <= P; };
  if (fits(L)) return L;
  // the units fall as the length grows: the smallest fitting length by bisection, at most the
  // total chunk count (where every sequence is one unit)
  int64_t hi = std::max<int64_t>(L, ceil_div(p->total_tokens, gdn::kChunk) + 1);
  if (!fits(hi)) return (int32_t)std::min<int64_t>(hi, INT32_MAX);
  int64_t lo = L;  // lo does not fit, hi fits
  while (hi - lo > 1) {
    const int64_t mid = lo + (hi - lo) / 2;
    (fits(mid) ? hi : lo) = mid;
  }
  return (int32_t)hi;
}

gdn_status check_cu_host(const gdn_problem *p, const int32_t *cu_host) {
  if (!cu_host) return GDN_OK;
  if (cu_host[0] != 0 || cu_host[p->num_seqs] != p->total_tokens)
    return fail(GDN_ERR_BAD_SHAPE, "cu_seqlens_host must start at 0 and end at total_tokens");
  for (int32_t n = 0; n < p->num_seqs; ++n)
    if (cu_host[n + 1] < cu_host[n]) return fail(GDN_ERR_BAD_SHAPE, "cu_seqlens_host descends");
  return GDN_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// The exact mode's split (three passes: every unit's affine map (B, M) from its chunks, the maps
// composed along each sequence into true start states, every unit rerun from its start) is built
// on the pipelined bf16 d = 128 kernel; other configurations run the exact mode unsplit.
bool split_available(const gdn_problem *p, bool dump) {
  return fwd_kernel_for(p, dump) == FwdKernel::kPipelined;
}

struct FwdLayout {
  int32_t L = 0;
  int64_t units = 0;
  bool split = false;     // exact mode through the three-pass split
  size_t unit_bm = 0;     // split: offset of the per-unit (B, M) pairs, [2, units, H, D, D] fp32
  size_t unit_h0 = 0;     // split: offset of the per-unit start states, [units, H, D, D] fp32
  size_t total = 0;       // workspace bytes (zero unless split)
};

gdn_status fwd_layout(const gdn_problem *p, const int32_t *cu_host, bool dump, FwdLayout *lay) {
  const bool split_ok = split_available(p, dump);
  int slots = 1;
  if ((p->mode == GDN_MODE_TRUNCATE || (p->mode == GDN_MODE_EXACT && split_ok)) &&
      p->seg_chunks == 0) {
    gdn_status s = parallel_slots(p, dump, &slots);
    if (s != GDN_OK) return s;
  }
  const int64_t nc = count_chunks(p, cu_host);
  lay->L = segment_chunks(p, nc, slots, split_ok);
  if (p->mode == GDN_MODE_EXACT) lay->L = exact_segment_chunks(p, cu_host, lay->L, slots);
  lay->units = max_units(p, cu_host, lay->L);
  // an exact-mode split in which every sequence stays one unit is no split
  if (p->mode == GDN_MODE_EXACT && lay->L > 0 && cu_host && lay->units == p->num_seqs) {
    lay->L = 0;
    lay->units = p->num_seqs;
  }
  if (lay->units > INT32_MAX) return fail(GDN_ERR_BAD_SHAPE, "too many work units");
  lay->split = p->mode == GDN_MODE_EXACT && lay->L > 0;
  lay->total = 0;
  if (lay->split) {
    const size_t per = (size_t)lay->units * p->num_heads * p->d_k * p->d_v * sizeof(float);
    lay->unit_bm = 0;
    lay->unit_h0 = align_up(2 * per);
    lay->total = align_up(lay->unit_h0 + per);
  }
  return GDN_OK;
}

struct Tensors {
  const void *q, *k, *v;
  const float *g;
  const void *beta;
  const int32_t *cu;
  const float *h0;
  void *o;
  float *ht;
};

// The per-token arrays may be NULL only when there are no tokens.
// need_o: false for the backward's recompute on the pipelined kernel, which writes no output
gdn_status check_tensors(const Tensors &t, int64_t T, bool need_o = true) {
  if (!t.cu || (T > 0 && (!t.q || !t.k || !t.v || !t.g || !t.beta || (need_o && !t.o))))
    return fail(GDN_ERR_NULL_ARG, "q, k, v, g, beta, cu_seqlens and o are required");
  const void *ptrs[] = {t.q, t.k, t.v, t.g, t.beta, t.o};
  for (const void *x : ptrs)
    if (!aligned16(x)) return fail(GDN_ERR_BAD_ALIGNMENT, "tensor pointers must be 16-byte aligned");
  if ((t.h0 && !aligned16(t.h0)) || (t.ht && !aligned16(t.ht)))
    return fail(GDN_ERR_BAD_ALIGNMENT, "h0 / ht must be 16-byte aligned");
  return GDN_OK;
}

gdn_status launch_fwd_passes(const gdn_problem *p, const Tensors &t, const FwdLayout &lay,
                             bool dump, float *dbg[6], void *ws, hipStream_t stream);

gdn_status run_fwd(const gdn_problem *p, const Tensors &t, const int32_t *cu_host, bool dump,
                   float *dbg[6], void *ws, size_t ws_bytes, hipStream_t stream) {
  gdn_status s = check_problem(p);
  if (s != GDN_OK) return s;
  s = check_tensors(t, p->total_tokens);
  if (s != GDN_OK) return s;
  s = check_cu_host(p, cu_host);
  if (s != GDN_OK) return s;
  s = device_info(nullptr);
  if (s != GDN_OK) return s;
  if (p->total_tokens == 0) {  // every sequence is empty: its final state is its initial state
    if (!t.ht) return GDN_OK;
    hipError_t e = gdn::launch_copy_states(t.h0, p->h0_seq_stride, p->num_seqs, p->num_heads,
                                           p->d_k, t.ht, stream);
    return e == hipSuccess ? GDN_OK : hip_fail(e, "final states of empty sequences");
  }
  FwdLayout lay;
  s = fwd_layout(p, cu_host, dump, &lay);
  if (s != GDN_OK) return s;
  if (ws_bytes < lay.total)
    return fail(GDN_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes", lay.total);
  if (lay.total > 0 && !aligned16(ws)) return fail(GDN_ERR_BAD_ALIGNMENT, "workspace alignment");
  if (debug_on()) {
    s = debug_validate(t.cu, p->num_seqs, p->total_tokens, cu_host, stream);
    if (s != GDN_OK) return s;
    s = launch_fwd_passes(p, t, lay, dump, dbg, ws, stream);
    return s != GDN_OK ? s : debug_faults(stream);
  }
  return launch_fwd_passes(p, t, lay, dump, dbg, ws, stream);
}

// The forward's launches for a checked problem: one kernel, or the exact split's three passes.
gdn_status launch_fwd_passes(const gdn_problem *p, const Tensors &t, const FwdLayout &lay,
                             bool dump, float *dbg[6], void *ws, hipStream_t stream) {
  gdn::FwdArgs a{};
  a.q = t.q;
  a.k = t.k;
  a.v = t.v;
  a.g = t.g;
  a.beta = t.beta;
  a.cu = t.cu;
  a.h0 = t.h0;
  a.h0_stride = p->h0_seq_stride;
  a.o = t.o;
  a.ht = t.ht;
  if (dump) {
    a.dbg_gamma = dbg[0];
    a.dbg_tmat = dbg[1];
    a.dbg_w = dbg[2];
    a.dbg_u = dbg[3];
    a.dbg_hc = dbg[4];
    a.dbg_delta = dbg[5];
  }
  a.T = p->total_tokens;
  a.N = p->num_seqs;
  a.H = p->num_heads;
  a.HK = k_heads(p);
  a.L = lay.L;
  a.scale = p->scale;
  a.log_thr = p->trunc_log_threshold;
  a.truncate = (p->mode == GDN_MODE_TRUNCATE && lay.L > 0) ? 1 : 0;
  a.l2norm = p->qk_l2norm;
  a.faults = fault_word();
  hipError_t e;
  if (lay.split) {
    char *base = static_cast<char *>(ws);
    float *bm = reinterpret_cast<float *>(base + lay.unit_bm);
    float *uh0 = reinterpret_cast<float *>(base + lay.unit_h0);
    a.units = lay.units;
    a.unit_out = bm;
    e = gdn::launch_fwd_ws_transition(a, lay.units, stream);
    if (e != hipSuccess) return hip_fail(e, "exact split: first pass");
    gdn::SplitArgs sa{};
    sa.cu = t.cu;
    sa.T = p->total_tokens;
    sa.N = p->num_seqs;
    sa.H = p->num_heads;
    sa.L = lay.L;
    sa.h0 = t.h0;
    sa.h0_stride = p->h0_seq_stride;
    sa.unit_b = bm;
    sa.unit_m = bm + lay.units * p->num_heads * p->d_k * p->d_v;
    sa.unit_h0 = uh0;
    sa.units = lay.units;
    e = gdn::launch_affine_scan(sa, stream);
    if (e != hipSuccess) return hip_fail(e, "exact split: start states");
    a.unit_out = nullptr;
    a.unit_h0 = uh0;
    e = gdn::launch_fwd_ws(a, lay.units, stream);
    if (e != hipSuccess) return hip_fail(e, "exact split: final pass");
    return GDN_OK;
  }
  switch (fwd_kernel_for(p, dump)) {
    case FwdKernel::kPipelined:
      // one workgroup per (sequence, head): the longest sequences first, so that no long one
      // starts late and stretches the tail of the launch
      a.longest_first = (lay.L == 0 && p->num_seqs >= 2 && p->num_seqs <= gdn::kMaxLongestFirst &&
                         lay.units <= 65535) ? 1 : 0;
      e = gdn::launch_fwd_ws(a, lay.units, stream);
      break;
    case FwdKernel::kFast: e = gdn::launch_fwd_fast(a, p->d_k, lay.units, stream); break;
    default: e = gdn::launch_fwd(a, p->d_k, p->dtype == GDN_DTYPE_BF16, dump, lay.units, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_problem_init(gdn_problem *p, int64_t total_tokens, int32_t num_seqs,
                            int32_t num_heads, int32_t head_dim) {
  if (!p) return fail(GDN_ERR_NULL_ARG, "problem is NULL");
  std::memset(p, 0, sizeof(*p));
  p->total_tokens = total_tokens;
  p->num_seqs = num_seqs;
  p->num_heads = num_heads;
  p->d_k = head_dim;
  p->d_v = head_dim;
  p->chunk = gdn::kChunk;
  p->dtype = GDN_DTYPE_BF16;
  p->mode = GDN_MODE_EXACT;
  p->trunc_log_threshold = -10.0f;
  p->scale = 1.0f;
  p->h0_seq_stride = (int64_t)num_heads * head_dim * head_dim;
  return GDN_OK;
}

gdn_status gdn_chunk_fwd_workspace_size(const gdn_problem *p, const int32_t *cu_seqlens_host,
                                        size_t *bytes) {
  gdn_status s = check_problem(p);
  if (s != GDN_OK) return s;
  if (!bytes) return fail(GDN_ERR_NULL_ARG, "bytes is NULL");
  s = check_cu_host(p, cu_seqlens_host);
  if (s != GDN_OK) return s;
  FwdLayout lay;
  s = fwd_layout(p, cu_seqlens_host, false, &lay);
  if (s != GDN_OK) return s;
  *bytes = lay.total;
  return GDN_OK;
}

gdn_status gdn_chunk_fwd(const gdn_problem *p, const void *q, const void *k, const void *v,
                         const float *g, const void *beta, const int32_t *cu_seqlens,
                         const int32_t *cu_seqlens_host, const float *h0, void *o, float *ht,
                         void *workspace, size_t workspace_bytes, hipStream_t stream) {
  Tensors t{q, k, v, g, beta, cu_seqlens, h0, o, ht};
  return run_fwd(p, t, cu_seqlens_host, false, nullptr, workspace, workspace_bytes, stream);
}

gdn_status gdn_chunk_fwd_noalloc(const gdn_problem *p, const void *q, const void *k,
                                 const void *v, const float *g, const void *beta,
                                 const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                                 const float *h0, void *o, float *ht, hipStream_t stream) {
  Tensors t{q, k, v, g, beta, cu_seqlens, h0, o, ht};
  gdn_status s = check_problem(p);
  if (s != GDN_OK) return s;
  s = check_tensors(t, p->total_tokens);
  if (s != GDN_OK) return s;
  s = check_cu_host(p, cu_seqlens_host);
  if (s != GDN_OK) return s;
  FwdLayout lay;
  s = fwd_layout(p, cu_seqlens_host, false, &lay);
  if (s != GDN_OK) return s;
  if (lay.total > gdn::kStaticScratchBytes)
    return fail(GDN_ERR_WORKSPACE_TOO_SMALL,
                "this problem needs %zu bytes of workspace; the static scratch of "
                "gdn_chunk_fwd_noalloc holds %zu (use gdn_chunk_fwd with a workspace)",
                lay.total, gdn::kStaticScratchBytes);
  s = device_info(nullptr);
  if (s != GDN_OK) return s;
  void *scratch = nullptr;
  const hipError_t e = gdn::static_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "static scratch address");
  return run_fwd(p, t, cu_seqlens_host, false, nullptr, scratch, gdn::kStaticScratchBytes,
                 stream);
}

gdn_status gdn_chunk_fwd_intermediates(const gdn_problem *p, const void *q, const void *k,
                                       const void *v, const float *g, const void *beta,
                                       const int32_t *cu_seqlens, const float *h0, void *o,
                                       float *ht, float *gamma, float *tmat, float *w, float *u,
                                       float *hc, float *delta, void *workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  if (p && p->mode != GDN_MODE_EXACT)
    return fail(GDN_ERR_BAD_MODE, "intermediates are defined for the exact mode only");
  Tensors t{q, k, v, g, beta, cu_seqlens, h0, o, ht};
  float *dbg[6] = {gamma, tmat, w, u, hc, delta};
  return run_fwd(p, t, nullptr, true, dbg, workspace, workspace_bytes, stream);
}

gdn_status gdn_chunk_fwd_plan(const gdn_problem *p, const float *g, const int32_t *cu_seqlens,
                              const int32_t *cu_seqlens_host, int32_t *plan_out,
                              int64_t plan_capacity, void *workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  gdn_status s = check_problem(p);
  if (s != GDN_OK) return s;
  if ((!g && p->total_tokens > 0) || !cu_seqlens || !plan_out)
    return fail(GDN_ERR_NULL_ARG, "g, cu_seqlens, plan_out");
  s = check_cu_host(p, cu_seqlens_host);
  if (s != GDN_OK) return s;
  s = device_info(nullptr);
  if (s != GDN_OK) return s;
  FwdLayout lay;
  s = fwd_layout(p, cu_seqlens_host, false, &lay);
  if (s != GDN_OK) return s;
  if (workspace_bytes < lay.total)
    return fail(GDN_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes", lay.total);
  (void)workspace;
  if (plan_capacity < 2) return fail(GDN_ERR_BAD_SHAPE, "plan_capacity must be >= 2");
  if (debug_on()) {
    s = debug_validate(cu_seqlens, p->num_seqs, p->total_tokens, cu_seqlens_host, stream);
    if (s != GDN_OK) return s;
  }
  const int truncate = (p->mode == GDN_MODE_TRUNCATE && lay.L > 0) ? 1 : 0;
  hipError_t e = gdn::launch_plan_export(cu_seqlens, p->num_seqs, p->total_tokens, g,
                                         p->num_heads, lay.L, p->trunc_log_threshold, truncate,
                                         lay.units, plan_out, plan_capacity, stream);
  if (e != hipSuccess) return hip_fail(e, "plan export launch");
  return GDN_OK;
}

}  // extern "C"

// ------------------------------------------------------------------------- backward
namespace {

struct BwdLayout {
  int64_t nc = 0;  // chunk-count bound: ceil(T / 64) + N
  // the recompute and the reverse chain split into units (bf16, d = 128): segment length and
  // unit bound; through the exact split, or (truncate mode) with warmup windows
  int32_t L = 0;
  int64_t units = 0;
  bool truncate = false;
  size_t gamma = 0, tmat = 0, w = 0, hc = 0, delta = 0, o = 0, dhn = 0, ddelta = 0, dh0 = 0;
  size_t unit_bm = 0, unit_h0 = 0, unit_mt = 0;
  size_t dq_part = 0, dk_part = 0;  // grouped heads or qk_l2norm: per-value-head dq, dk (fp32)
  size_t rq = 0, rk = 0;            // qk_l2norm: inverse row norms of q and k (fp32 [T, Hk])
  size_t total = 0;
};

// bf16 inputs with d = 128 run the backward on the bf16-MFMA chain and gradient kernels (which
// need no W); everything else on the general fp32-MFMA kernels.
bool bwd_bf16_path(const gdn_problem *p) { return p->dtype == GDN_DTYPE_BF16 && p->d_k == 128; }

// The recompute's (and the reverse chain's) segment length: the forward's exact-split rule
// (measured on the 65K-token training workload: 2.42 ms per call at 16 chunks, 2.50 at 8, 2.54 at
// 32, 2.89 at 4); 0 (unsplit) where the forward would not split.  The truncate mode takes the
// same length: a unit then costs its own chunks plus a warmup window whose length does not
// depend on L, so the shortest length that fits one round is again the fastest.
gdn_status bwd_layout(const gdn_problem *p, const int32_t *cu_host, BwdLayout *L) {
  const int64_t T = p->total_tokens, H = p->num_heads, D = p->d_k;
  // per-chunk arrays on the chunk bound, whatever the host copy says: chunk indices come from
  // the device table
  L->nc = ceil_div(T, gdn::kChunk) + p->num_seqs;
  L->L = 0;
  L->units = 0;
  if (split_available(p, false)) {
    int slots = 1;
    if (p->seg_chunks == 0) {
      gdn_status s = parallel_slots(p, false, &slots);
      if (s != GDN_OK) return s;
    }
    gdn_problem pe = *p;
    pe.mode = GDN_MODE_EXACT;  // the backward is defined for the exact forward
    const int32_t Lf = segment_chunks(&pe, count_chunks(p, cu_host), slots, true);
    L->L = exact_segment_chunks(&pe, cu_host, Lf, slots);
    if (L->L > 0) L->units = max_units(p, cu_host, L->L);
    if (L->L > 0 && cu_host && L->units == p->num_seqs) {  // every sequence is one unit: no split
      L->L = 0;
      L->units = 0;
    }
    if (L->units > INT32_MAX) return fail(GDN_ERR_BAD_SHAPE, "too many work units");
  }
  const size_t esz = p->dtype == GDN_DTYPE_BF16 ? 2 : 4;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L->gamma = take(sizeof(float) * T * H);
  L->tmat = take(sizeof(float) * L->nc * H * 64 * 64);
  if (!bwd_bf16_path(p)) L->w = take(sizeof(float) * L->nc * H * 64 * D);  // W: general kernels only
  // per-chunk states h and dh': bf16 on the bf16 d = 128 kernels, fp32 on the general ones
  const size_t ssz = bwd_bf16_path(p) ? 2 : 4;
  L->hc = take(ssz * L->nc * H * D * D);
  L->delta = take(sizeof(float) * T * H * D);
  if (!bwd_bf16_path(p)) L->o = take(esz * T * H * D);  // the general recompute's output (unused)
  L->dhn = take(ssz * L->nc * H * D * D);
  L->ddelta = take(sizeof(float) * T * H * D);
  L->dh0 = take(sizeof(float) * p->num_seqs * H * D * D);
  L->truncate = L->L > 0 && p->mode == GDN_MODE_TRUNCATE;
  if (L->L > 0 && !L->truncate) {
    const size_t per = sizeof(float) * (size_t)L->units * H * D * D;
    L->unit_bm = take(2 * per);
    L->unit_h0 = take(per);
    L->unit_mt = take(per);  // M^T of each unit, for the reverse walk
  }
  // partials: grouped heads (summed per key head), and the general kernels' normalised q, k
  // (finished by the normalisation's backward kernel; the bf16 d = 128 kernel finishes in place)
  if (k_heads(p) < H || (p->qk_l2norm && !bwd_bf16_path(p))) {
    L->dq_part = take(sizeof(float) * T * H * D);
    L->dk_part = take(sizeof(float) * T * H * D);
  }
  if (p->qk_l2norm) {
    L->rq = take(sizeof(float) * T * k_heads(p));
    L->rk = take(sizeof(float) * T * k_heads(p));
  }
  L->total = off;
  return GDN_OK;
}

// Forward recompute of the backward for bf16 inputs with d = 128, on the pipelined forward kernel:
// the per-chunk start states, Delta and gamma, from all units in parallel when the recompute is
// split (every unit's affine map (B, M), then the maps composed along each sequence into true
// start states, as in the forward's exact split; or, in the truncate mode, each unit from the
// warmup window before it, as the truncate-mode forward runs).
gdn_status run_fwd_recompute_bf16(const gdn_problem *p, const Tensors &t, float *gamma,
                                  uint16_t *hc, float *delta, float *rk, const BwdLayout &L,
                                  char *base, hipStream_t stream) {
  gdn::FwdArgs a{};
  a.q = t.q;
  a.k = t.k;
  a.v = t.v;
  a.g = t.g;
  a.beta = t.beta;
  a.cu = t.cu;
  a.h0 = t.h0;
  a.h0_stride = p->h0_seq_stride;
  a.o = t.o;
  a.ht = nullptr;
  a.T = p->total_tokens;
  a.N = p->num_seqs;
  a.H = p->num_heads;
  a.HK = k_heads(p);
  a.L = L.L;
  a.scale = p->scale;
  a.log_thr = p->trunc_log_threshold;
  a.truncate = L.truncate ? 1 : 0;
  a.l2norm = p->qk_l2norm;
  a.faults = fault_word();
  hipError_t e;
  int64_t units = p->num_seqs;
  if (L.truncate) {
    units = L.units;
    a.units = L.units;
  } else if (L.L > 0) {
    float *bm = reinterpret_cast<float *>(base + L.unit_bm);
    float *uh0 = reinterpret_cast<float *>(base + L.unit_h0);
    units = L.units;
    a.units = L.units;
    a.unit_out = bm;
    a.unit_mt = reinterpret_cast<float *>(base + L.unit_mt);  // for the reverse walk
    e = gdn::launch_fwd_ws_transition(a, L.units, stream);
    if (e != hipSuccess) return hip_fail(e, "backward recompute: first pass");
    gdn::SplitArgs sa{};
    sa.cu = t.cu;
    sa.T = p->total_tokens;
    sa.N = p->num_seqs;
    sa.H = p->num_heads;
    sa.L = L.L;
    sa.h0 = t.h0;
    sa.h0_stride = p->h0_seq_stride;
    sa.unit_b = bm;
    sa.unit_m = bm + L.units * p->num_heads * p->d_k * p->d_v;
    sa.unit_h0 = uh0;
    sa.units = L.units;
    e = gdn::launch_affine_scan(sa, stream);
    if (e != hipSuccess) return hip_fail(e, "backward recompute: start states");
    a.unit_out = nullptr;
    a.unit_mt = nullptr;
    a.unit_h0 = uh0;
  }
  a.dbg_gamma = gamma;
  a.dump_hc = hc;
  a.dbg_delta = delta;
  a.dump_rk = rk;  // with l2norm: K's inverse row norms, as the recompute forms them
  e = gdn::launch_fwd_ws_dump(a, units, stream);
  if (e != hipSuccess) return hip_fail(e, "backward recompute: intermediates");
  return GDN_OK;
}

}  // namespace

extern "C" {

gdn_status gdn_chunk_bwd_workspace_size(const gdn_problem *p, const int32_t *cu_seqlens_host,
                                        size_t *bytes) {
  gdn_status s = check_problem(p);
  if (s != GDN_OK) return s;
  if (!bytes) return fail(GDN_ERR_NULL_ARG, "bytes is NULL");
  s = check_cu_host(p, cu_seqlens_host);
  if (s != GDN_OK) return s;
  BwdLayout L;
  s = bwd_layout(p, cu_seqlens_host, &L);
  if (s != GDN_OK) return s;
  *bytes = L.total;
  return GDN_OK;
}

gdn_status gdn_chunk_bwd(const gdn_problem *p, const void *q, const void *k, const void *v,
                         const float *g, const void *beta, const int32_t *cu_seqlens,
                         const int32_t *cu_seqlens_host, const float *h0, const void *dout,
                         const float *dht, void *dq, void *dk, void *dv, float *dg, void *dbeta,
                         float *dh0, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  gdn_status s = check_problem(p);
  if (s != GDN_OK) return s;
  s = check_cu_host(p, cu_seqlens_host);
  if (s != GDN_OK) return s;
  if (p->total_tokens > 0 && (!dout || !dq || !dk || !dv || !dg || !dbeta))
    return fail(GDN_ERR_NULL_ARG, "dout, dq, dk, dv, dg and dbeta are required");
  const void *ptrs[] = {dout, dq, dk, dv, dg, dbeta};
  for (const void *x : ptrs)
    if (!aligned16(x)) return fail(GDN_ERR_BAD_ALIGNMENT, "tensor pointers must be 16-byte aligned");
  if ((dht && !aligned16(dht)) || (dh0 && !aligned16(dh0)))
    return fail(GDN_ERR_BAD_ALIGNMENT, "dht / dh0 must be 16-byte aligned");
  if (p->total_tokens == 0) {  // no tokens: every state passes through unchanged, so dh0 = dht
    if (!cu_seqlens) return fail(GDN_ERR_NULL_ARG, "cu_seqlens is required");
    if (!dh0) return GDN_OK;
    s = device_info(nullptr);
    if (s != GDN_OK) return s;
    const bool shared = h0 != nullptr && p->h0_seq_stride == 0;
    const int64_t per_seq = (int64_t)p->num_heads * p->d_k * p->d_k;
    hipError_t e = (shared && dht)
                       ? gdn::launch_sum_dh0(dht, p->num_seqs, p->num_heads, p->d_k, dh0, stream)
                       : gdn::launch_copy_states(dht, per_seq, shared ? 1 : p->num_seqs,
                                                 p->num_heads, p->d_k, dh0, stream);
    return e == hipSuccess ? GDN_OK : hip_fail(e, "dh0 of empty sequences");
  }
  BwdLayout L;
  s = bwd_layout(p, cu_seqlens_host, &L);
  if (s != GDN_OK) return s;
  if (!workspace) return fail(GDN_ERR_NULL_ARG, "workspace is NULL");
  if (workspace_bytes < L.total)
    return fail(GDN_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes", L.total);
  if (!cu_seqlens) return fail(GDN_ERR_NULL_ARG, "cu_seqlens is required");
  const bool debug = debug_on();
  if (debug) {
    s = device_info(nullptr);
    if (s == GDN_OK)
      s = debug_validate(cu_seqlens, p->num_seqs, p->total_tokens, cu_seqlens_host, stream);
    if (s != GDN_OK) return s;
  }
  char *base = static_cast<char *>(workspace);
  float *gamma = reinterpret_cast<float *>(base + L.gamma);
  float *tmat = reinterpret_cast<float *>(base + L.tmat);
  const bool fast = bwd_bf16_path(p);
  float *w = fast ? nullptr : reinterpret_cast<float *>(base + L.w);
  float *hc = fast ? nullptr : reinterpret_cast<float *>(base + L.hc);
  uint16_t *hc_b16 = fast ? reinterpret_cast<uint16_t *>(base + L.hc) : nullptr;
  float *delta = reinterpret_cast<float *>(base + L.delta);
  // forward recompute with the per-chunk intermediates (the general kernels' o goes to scratch;
  // the pipelined kernel's recompute pass writes none)
  Tensors t{q, k, v, g, beta, cu_seqlens, h0, fast ? nullptr : base + L.o, nullptr};
  float *dbg[6] = {gamma, tmat, w, nullptr, hc, delta};
  if (fast) {
    s = check_tensors(t, p->total_tokens, false);
    if (s == GDN_OK) s = device_info(nullptr);
    if (s == GDN_OK)
      s = run_fwd_recompute_bf16(p, t, gamma, hc_b16, delta,
                                 p->qk_l2norm ? reinterpret_cast<float *>(base + L.rk) : nullptr,
                                 L, base, stream);
  } else {  // the general kernels' backward is unsplit: the exact one, whatever the mode
    gdn_problem pe = *p;
    pe.mode = GDN_MODE_EXACT;
    s = run_fwd(&pe, t, nullptr, true, dbg, nullptr, 0, stream);
  }
  if (s != GDN_OK) return s;
  gdn::BwdArgs b{};
  b.q = q;
  b.k = k;
  b.v = v;
  b.beta = beta;
  b.dout = dout;
  b.g = g;
  b.dht = dht;
  b.cu = cu_seqlens;
  b.dq = dq;
  b.dk = dk;
  b.dv = dv;
  b.dbeta = dbeta;
  b.dg = dg;
  const bool shared_h0 = (h0 != nullptr && p->h0_seq_stride == 0);
  // dh0 per sequence goes straight to the output, or to scratch when one state is shared
  b.dh0_seq = !dh0 ? nullptr : (shared_h0 ? reinterpret_cast<float *>(base + L.dh0) : dh0);
  b.gamma = gamma;
  b.tmat = tmat;
  b.w = w;
  b.hc = hc;
  b.hc_b16 = hc_b16;
  b.delta = delta;
  b.dhn = fast ? nullptr : reinterpret_cast<float *>(base + L.dhn);
  b.dhn_b16 = fast ? reinterpret_cast<uint16_t *>(base + L.dhn) : nullptr;
  const bool grouped = k_heads(p) < p->num_heads;
  const bool part = grouped || (p->qk_l2norm && !fast);
  b.dq_part = part ? reinterpret_cast<float *>(base + L.dq_part) : nullptr;
  b.dk_part = part ? reinterpret_cast<float *>(base + L.dk_part) : nullptr;
  float *rq = p->qk_l2norm ? reinterpret_cast<float *>(base + L.rq) : nullptr;
  float *rk = p->qk_l2norm ? reinterpret_cast<float *>(base + L.rk) : nullptr;
  b.rq = rq;
  b.rk = rk;
  b.ddelta = reinterpret_cast<float *>(base + L.ddelta);
  b.T = p->total_tokens;
  b.N = p->num_seqs;
  b.H = p->num_heads;
  b.HK = k_heads(p);
  b.scale = p->scale;
  hipError_t e;
  const bool bf = p->dtype == GDN_DTYPE_BF16;
  if (p->qk_l2norm) {  // the rows' inverse norms, folded in by the kernels below (K's come from
                       // the pipelined recompute, which forms them anyway)
    e = gdn::launch_row_rnorm(q, p->total_tokens * k_heads(p), p->d_k, bf, rq, stream);
    if (e == hipSuccess && !fast)
      e = gdn::launch_row_rnorm(k, p->total_tokens * k_heads(p), p->d_k, bf, rk, stream);
    if (e != hipSuccess) return hip_fail(e, "q/k inverse norms");
  }
  if (fast) {
    e = gdn::launch_bwd_tm(b, tmat, L.nc, stream);
    if (e != hipSuccess) return hip_fail(e, "backward: Tm");
    // reverse chain, through the exact split when the recompute was split (same units): the
    // transition pass writes B' over the recompute's B, and the reverse walk applies B' with the
    // M^T the recompute's first pass stored; in the truncate mode each unit's chain starts after
    // a warmup window instead
    gdn::BwdUnits u{};
    u.L = L.L;
    u.units = L.units;
    u.truncate = L.truncate ? 1 : 0;
    u.log_thr = p->trunc_log_threshold;
    if (L.L > 0 && !L.truncate) {
      float *bm = reinterpret_cast<float *>(base + L.unit_bm);
      float *dend = reinterpret_cast<float *>(base + L.unit_h0);
      u.unit_out = bm;
      e = gdn::launch_bwd_chain_bf16_transition(b, u, stream);
      if (e != hipSuccess) return hip_fail(e, "backward chain: first pass");
      gdn::SplitArgs sa{};
      sa.cu = cu_seqlens;
      sa.T = p->total_tokens;
      sa.N = p->num_seqs;
      sa.H = p->num_heads;
      sa.L = L.L;
      sa.h0 = dht;
      sa.h0_stride = (int64_t)p->num_heads * p->d_k * p->d_v;
      sa.unit_b = bm;
      sa.unit_m = reinterpret_cast<const float *>(base + L.unit_mt);
      sa.unit_h0 = dend;
      sa.units = L.units;
      e = gdn::launch_affine_scan_reverse(sa, stream);
      if (e != hipSuccess) return hip_fail(e, "backward chain: end gradients");
      u.unit_out = nullptr;
      u.unit_dend = dend;
    }
    e = gdn::launch_bwd_chain_bf16(b, u, stream);
    if (e != hipSuccess) return hip_fail(e, "backward chain launch");
    e = gdn::launch_bwd_grad_bf16(b, L.nc, stream);
    if (e != hipSuccess) return hip_fail(e, "backward gradient launch");
  } else {
    const bool bf16 = p->dtype == GDN_DTYPE_BF16;
    e = gdn::launch_bwd_chain(b, p->d_k, bf16, stream);
    if (e != hipSuccess) return hip_fail(e, "backward chain launch");
    e = gdn::launch_bwd_grad(b, p->d_k, bf16, L.nc, stream);
    if (e != hipSuccess) return hip_fail(e, "backward gradient launch");
  }
  if (p->qk_l2norm && !fast) {  // the normalisation's backward (and the per-key-head sums)
    e = gdn::launch_l2norm_bwd(b.dq_part, q, rq, p->total_tokens, p->num_heads, k_heads(p),
                               p->d_k, bf, dq, stream);
    if (e == hipSuccess)
      e = gdn::launch_l2norm_bwd(b.dk_part, k, rk, p->total_tokens, p->num_heads, k_heads(p),
                                 p->d_k, bf, dk, stream);
    if (e != hipSuccess) return hip_fail(e, "q/k normalisation backward");
  } else if (grouped) {  // dq, dk of each key head: the sum over its value heads
    e = gdn::launch_group_sum(b.dq_part, p->total_tokens, p->num_heads, k_heads(p), p->d_k,
                              bf, dq, stream);
    if (e == hipSuccess)
      e = gdn::launch_group_sum(b.dk_part, p->total_tokens, p->num_heads, k_heads(p), p->d_k,
                                bf, dk, stream);
    if (e != hipSuccess) return hip_fail(e, "grouped heads: dq, dk sums");
  }
  if (dh0 && shared_h0) {
    e = gdn::launch_sum_dh0(b.dh0_seq, p->num_seqs, p->num_heads, p->d_k, dh0, stream);
    if (e != hipSuccess) return hip_fail(e, "dh0 reduction launch");
  }
  return debug ? debug_faults(stream) : GDN_OK;
}

}  // extern "C"

extern "C" {

gdn_status gdn_decode_step(int32_t batch, int32_t num_heads, int32_t num_k_heads, int32_t head_dim,
                           int32_t dtype, int32_t qk_l2norm, float scale, const void *q,
                           const void *k, const void *v, const float *g, const void *beta,
                           float *state, void *o, hipStream_t stream) {
  if (batch < 1 || num_heads < 1 || (int64_t)batch * num_heads > INT32_MAX)
    return fail(GDN_ERR_BAD_SHAPE, "batch and num_heads must be >= 1");
  if (num_k_heads < 0 || num_k_heads > num_heads ||
      (num_k_heads > 0 && num_heads % num_k_heads != 0))
    return fail(GDN_ERR_BAD_SHAPE, "num_k_heads must be 0 or a divisor of num_heads");
  if (qk_l2norm != 0 && qk_l2norm != 1) return fail(GDN_ERR_BAD_MODE, "qk_l2norm must be 0 or 1");
  if (head_dim != 64 && head_dim != 128) return fail(GDN_ERR_BAD_SHAPE, "head_dim must be 64 or 128");
  if (dtype != GDN_DTYPE_F32 && dtype != GDN_DTYPE_BF16) return fail(GDN_ERR_BAD_DTYPE, "dtype %d", dtype);
  if (!std::isfinite(scale)) return fail(GDN_ERR_BAD_SHAPE, "scale must be finite");
  if (!q || !k || !v || !g || !beta || !state || !o)
    return fail(GDN_ERR_NULL_ARG, "q, k, v, g, beta, state and o are required");
  const void *ptrs[] = {q, k, v, state, o};
  for (const void *x : ptrs)
    if (!aligned16(x)) return fail(GDN_ERR_BAD_ALIGNMENT, "tensor pointers must be 16-byte aligned");
  gdn_status s = device_info(nullptr);
  if (s != GDN_OK) return s;
  gdn::DecodeArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.state = state;
  a.o = o;
  a.B = batch;
  a.H = num_heads;
  a.HK = num_k_heads > 0 ? num_k_heads : num_heads;
  a.l2norm = qk_l2norm;
  a.scale = scale;
  const hipError_t e = gdn::launch_decode_step(a, head_dim, dtype == GDN_DTYPE_BF16, stream);
  if (e != hipSuccess) return hip_fail(e, "decode step launch");
  return GDN_OK;
}

gdn_status gdn_calib_copy(const void *src, void *dst, size_t bytes, hipStream_t stream) {
  if (!src || !dst) return fail(GDN_ERR_NULL_ARG, "src and dst are required");
  if (!aligned16(src) || !aligned16(dst))
    return fail(GDN_ERR_BAD_ALIGNMENT, "src and dst must be 16-byte aligned");
  if (bytes == 0 || bytes % 16 != 0 || bytes > ((size_t)1 << 40))
    return fail(GDN_ERR_BAD_SHAPE, "bytes must be a positive multiple of 16 (at most 2^40)");
  int cus = 0;
  gdn_status s = device_info(&cus);
  if (s != GDN_OK) return s;
  const hipError_t e = gdn::launch_calib_copy(src, dst, (int64_t)(bytes / 16), cus, stream);
  if (e != hipSuccess) return hip_fail(e, "calibration copy launch");
  return GDN_OK;
}

gdn_status gdn_calib_mfma_bf16(float *out, int waves_per_cu, int iters, hipStream_t stream) {
  if (!out) return fail(GDN_ERR_NULL_ARG, "out is required");
  if (waves_per_cu < 1 || waves_per_cu > 8 || iters < 1 || iters > (1 << 20))
    return fail(GDN_ERR_BAD_SHAPE, "waves_per_cu must be in 1..8 and iters in 1..2^20");
  gdn_status s = device_info(nullptr);
  if (s != GDN_OK) return s;
  const hipError_t e = gdn::launch_calib_mfma(out, waves_per_cu * 256, iters, stream);
  if (e != hipSuccess) return hip_fail(e, "calibration MFMA launch");
  return GDN_OK;
}

gdn_status gdn_validate_cu_seqlens(const int32_t *cu_seqlens, int32_t num_seqs,
                                   int64_t total_tokens, int32_t *status, hipStream_t stream) {
  if (!cu_seqlens || !status) return fail(GDN_ERR_NULL_ARG, "cu_seqlens and status are required");
  if (num_seqs < 1) return fail(GDN_ERR_BAD_SHAPE, "num_seqs must be >= 1");
  if (total_tokens < 0 || total_tokens > INT32_MAX)
    return fail(GDN_ERR_BAD_SHAPE, "total_tokens %lld out of range", (long long)total_tokens);
  gdn_status s = device_info(nullptr);
  if (s != GDN_OK) return s;
  const hipError_t e = gdn::launch_validate_cu(cu_seqlens, num_seqs, total_tokens, status,
                                               nullptr, stream);
  if (e != hipSuccess) return hip_fail(e, "cu_seqlens validation launch");
  return GDN_OK;
}

gdn_status gdn_set_debug(int32_t on) {
  if (on != 0 && on != 1) return fail(GDN_ERR_BAD_MODE, "on must be 0 or 1");
  g_debug.store(on, std::memory_order_relaxed);
  return GDN_OK;
}

int32_t gdn_get_debug(void) { return debug_on() ? 1 : 0; }

gdn_status gdn_device_faults(uint32_t *flags, int32_t clear) {
  if (!flags) return fail(GDN_ERR_NULL_ARG, "flags is NULL");
  gdn_status s = device_info(nullptr);
  if (s != GDN_OK) return s;
  uint32_t *words = nullptr;
  hipError_t e = gdn::device_check_words(&words);
  if (e != hipSuccess) return hip_fail(e, "check words");
  e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(flags, words + 1, sizeof(uint32_t), hipMemcpyDeviceToHost);
  if (e == hipSuccess && clear) {
    const uint32_t zero = 0;
    e = hipMemcpy(words + 1, &zero, sizeof(zero), hipMemcpyHostToDevice);
  }
  if (e != hipSuccess) return hip_fail(e, "fault flags");
  return GDN_OK;
}

const char *gdn_status_string(gdn_status s) {
  switch (s) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL_ARG: return "a required pointer is NULL";
    case GDN_ERR_BAD_SHAPE: return "unsupported or inconsistent sizes";
    case GDN_ERR_BAD_DTYPE: return "unsupported dtype";
    case GDN_ERR_BAD_MODE: return "unsupported mode";
    case GDN_ERR_UNSUPPORTED_ARCH: return "device is not gfx950";
    case GDN_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case GDN_ERR_BAD_ALIGNMENT: return "tensor pointer not 16-byte aligned";
    case GDN_ERR_HIP: return "HIP runtime error";
    case GDN_ERR_DEVICE_CHECK: return "a device-side check failed";
  }
  return "unknown status";
}

const char *gdn_last_error(void) { return g_err; }

}  // extern "C"
