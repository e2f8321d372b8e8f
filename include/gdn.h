/*
 * gdn.h: C ABI of the MI355X (gfx950) Gated DeltaNet chunked prefill library.
 *
 * The operation (per head h of every packed sequence n), as stated on the page "How to Speed Up
 * GDN Kernels for Qwen Models", section "What GDN actually computes", and on "Musings on
 * long-context fine-tuning", section "Isolating the recurrent layers":
 *
 *     S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,    o_t = scale * S_t^T q_t
 *
 * with the d_k x d_v state S reset at every sequence start to that sequence's initial state
 * (or zero).  The library evaluates it in 64-token chunks (the chunked form of the same page:
 * gate cumsum, one 64x64 unit-lower-triangular solve per chunk and head, WY-form w/u, the
 * inter-chunk state chain and the output), on the stream the caller passes.
 *
 * Layouts (row-major, token-major, contiguous; T = total_tokens, N = num_seqs, H = num_heads):
 *   q, k        [T, Hk, d_k]     dtype (bf16 or fp32); Hk = num_k_heads (= H unless grouped)
 *   v, o        [T, H, d_v]      dtype
 *   g           [T, H]           fp32: the log-gate, alpha_t = exp(g_t)
 *   beta        [T, H]           dtype: the write strength
 *   cu_seqlens  [N + 1]          int32, device; cu_seqlens[0] = 0, cu_seqlens[N] = T, ascending
 *   h0          sequence n's state at h0 + n * h0_seq_stride, each [H, d_k, d_v] fp32;
 *               h0_seq_stride = 0 broadcasts one state to every sequence (a shared prefix, as in
 *               "Musings on long-context fine-tuning", section "Isolating the recurrent layers")
 *   ht          [N, H, d_k, d_v] fp32, the state after each sequence's last token
 *   T = 0 (every sequence empty) is allowed: the per-token pointers may then be NULL, each final
 *   state is its initial state and the backward's dh0 is dht.
 *
 * Conventions.
 *   Ownership: every tensor pointer is a device pointer owned by the caller; the library never
 *     allocates or frees device memory.  Scratch space is the caller's `workspace`, sized by the
 *     matching *_workspace_size call; tensors must be 16-byte aligned.
 *   Asynchrony: calls enqueue work on `stream` and return without a host synchronisation.
 *   Errors: arguments are validated before anything is enqueued; on an error nothing is written.
 *     A launch failure returns GDN_ERR_HIP.  gdn_last_error() gives a thread-local detail string.
 *     The contents of cu_seqlens are read on the device only (the host checks
 *     cu_seqlens_host when it is given).  On a malformed device table (cu[0] != 0, a descending
 *     pair, or an offset past T) the kernels find no work for the sequences from the first bad
 *     entry on and write nothing for them, so no access leaves the caller's buffers; the
 *     outputs of such a call are undefined.  gdn_validate_cu_seqlens checks a table on the
 *     device, and the debug mode (GDN_DEBUG=1 in the environment, or gdn_set_debug(1)) runs
 *     that check inside every compute call before its first launch, and also checks that
 *     cu_seqlens_host, when given, equals the device table (read back); either failure returns
 *     GDN_ERR_BAD_SHAPE with nothing launched.  After the launches it synchronises the stream
 *     and returns GDN_ERR_DEVICE_CHECK if a kernel set a fault flag (gdn_device_faults).
 *   Architecture: only gfx950 is supported; other devices return GDN_ERR_UNSUPPORTED_ARCH (the
 *     page's library likewise refuses hardware it was not built for, section "Using it, and the
 *     fine print").
 *   Threading: calls are re-entrant.  Global state: a per-device properties cache, the debug
 *     switch, and per device four words of device memory (the debug mode's validation status and
 *     the fault flags kernels set; a static device array, not an allocation).
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_NULL_ARG = 1,            /* a required pointer is NULL */
  GDN_ERR_BAD_SHAPE = 2,           /* sizes out of range or unsupported (d, chunk) */
  GDN_ERR_BAD_DTYPE = 3,           /* dtype not one of GDN_DTYPE_* */
  GDN_ERR_BAD_MODE = 4,            /* mode / algo / threshold not supported */
  GDN_ERR_UNSUPPORTED_ARCH = 5,    /* the current device is not gfx950 */
  GDN_ERR_WORKSPACE_TOO_SMALL = 6, /* workspace_bytes below the *_workspace_size figure */
  GDN_ERR_BAD_ALIGNMENT = 7,       /* a tensor pointer is not 16-byte aligned */
  GDN_ERR_HIP = 8,                 /* a HIP runtime call or kernel launch failed */
  GDN_ERR_DEVICE_CHECK = 9         /* debug mode: a kernel set a fault flag (gdn_device_faults) */
} gdn_status;

/* Element type of q, k, v, beta, o (and of dout, dq, dk, dv, dbeta in the backward). */
enum { GDN_DTYPE_F32 = 0, GDN_DTYPE_BF16 = 1 };

/* Forward mode.
 *   GDN_MODE_EXACT: the recurrence as defined.  With bf16 inputs and d = 128, when num_seqs *
 *     num_heads is below P the sequences are split into segments of L chunks exactly as in the
 *     truncate mode (L from the same latency model, or seg_chunks), and the result is still
 *     exact (up to rounding): every (segment, head) first computes the affine map its chunks
 *     apply to the state, S_end = M S_start + B (M from the identity with V = 0, B from zero);
 *     the maps are composed along each sequence from its initial state into the true state at
 *     every segment start; every segment then reruns from that state and writes its outputs.
 *     This needs 3 x 64 KiB of workspace per (segment, head) (gdn_chunk_fwd_workspace_size).
 *     Other configurations run every sequence as one chain of chunks.
 *   GDN_MODE_TRUNCATE: history truncation of "How to Speed Up GDN Kernels for Qwen Models",
 *     section "Lever 1: the gate is also a license to parallelize".  When num_seqs * num_heads
 *     is below P, the number of workgroups that run at once, each sequence is split into
 *     segments of L chunks, L = max(4, nearest power of two of 3 * sqrt(H * Nc / P)) with Nc the
 *     number of chunks (or L = seg_chunks if positive).  Every (segment, head) starts from zero at
 *     a warmup window: the shortest run of whole preceding chunks whose summed g is below
 *     trunc_log_threshold (-10 on the page), or from the true initial state when the window
 *     reaches the sequence start.  The error this introduces is bounded per token by
 *     ||q_t|| * exp(threshold) * ||S_exact(window start)||_2 when 0 <= beta ||k||^2 <= 2. */
enum { GDN_MODE_EXACT = 0, GDN_MODE_TRUNCATE = 1 };

typedef struct gdn_problem {
  int64_t total_tokens;      /* T = cu_seqlens[N] (>= 0) */
  int32_t num_seqs;          /* N >= 1 */
  int32_t num_heads;         /* H >= 1: heads of v, o, g, beta and of the state */
  int32_t d_k;               /* 64 or 128 */
  int32_t d_v;               /* equal to d_k */
  int32_t chunk;             /* 64 */
  int32_t dtype;             /* GDN_DTYPE_* */
  int32_t mode;              /* GDN_MODE_* */
  int32_t seg_chunks;        /* segment length where the mode splits (truncate; exact at bf16,
                              * d = 128): 0 = latency model, > 0 = forced */
  int32_t num_slots;         /* P of the latency model: workgroups that run at once; 0 = the
                              * device's CUs x resident workgroups per CU of the forward kernel
                              * (then the workspace query needs the device) */
  float trunc_log_threshold; /* truncate mode: -10 */
  float scale;               /* o_t = scale * S_t^T q_t (1 in the pages' formulation) */
  int32_t num_k_heads;       /* heads of q and k: 0 (= num_heads) or a divisor of num_heads;
                              * value head h reads key head h / (num_heads / num_k_heads) (the
                              * grouped layouts of "How to Speed Up GDN Kernels for Qwen Models",
                              * section "Using it, and the fine print", where value heads are a
                              * multiple of key heads) */
  int32_t qk_l2norm;         /* 1: q and k are L2-normalised per (token, head) row inside the
                              * kernels, q / sqrt(|q|^2 + 1e-6) (likewise k), and the backward
                              * returns the gradients of the raw q and k; 0: used as given.
                              * bf16 with d = 128 never rounds the normalised rows (the norms
                              * fold into the kernel's per-token factors); bf16 with d = 64 and
                              * the intermediates call round them to bf16. */
  int32_t reserved;          /* must be 0 */
  int64_t h0_seq_stride;     /* elements between consecutive sequences' h0; 0 = broadcast */
} gdn_problem;

/* Fills *p with defaults: chunk 64, dtype bf16, exact mode, threshold -10, scale 1, and the
 * given sizes.  The defaults follow "How to Speed Up GDN Kernels for Qwen Models": 64-token
 * chunks and head size 128 (section "Using it, and the fine print"), the e^-10 truncation
 * threshold (section "Lever 1"); the scale of 1 is the recurrence as written (section "What
 * GDN actually computes").  No allocation; returns GDN_ERR_NULL_ARG for a NULL p. */
gdn_status gdn_problem_init(gdn_problem *p, int64_t total_tokens, int32_t num_seqs,
                            int32_t num_heads, int32_t head_dim);

/* Bytes of device workspace gdn_chunk_fwd needs for *p (zero except for the exact mode's
 * split).  cu_seqlens_host (optional, N + 1 host int32) lets a split mode size its segment plan
 * exactly (without it the unit count is an upper bound); pass the same pointer (or NULL) to
 * gdn_chunk_fwd.  The operation is the forward described at the top of this file; the page
 * names no workspace (its kernels are separate launches, "How to Speed Up GDN Kernels for Qwen
 * Models", section "Lever 1"), so no passage applies to the figure itself.  Host only; the
 * latency model may query the current device (num_slots = 0). */
gdn_status gdn_chunk_fwd_workspace_size(const gdn_problem *p, const int32_t *cu_seqlens_host,
                                        size_t *bytes);

/* Forward of the chunked gated delta rule.  h0 may be NULL (zero initial states) and ht may be
 * NULL (final states not written).  o must not alias an input. */
gdn_status gdn_chunk_fwd(const gdn_problem *p, const void *q, const void *k, const void *v,
                         const float *g, const void *beta, const int32_t *cu_seqlens,
                         const int32_t *cu_seqlens_host, const float *h0, void *o, float *ht,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/* gdn_chunk_fwd for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same arguments without the
 * workspace, which comes from a static device array of GDN_NOALLOC_SCRATCH_BYTES (128 MiB) that
 * every GPU the library is loaded on holds until the process ends.  Calls nothing that
 * allocates.  A problem whose workspace (gdn_chunk_fwd_workspace_size) exceeds that size is
 * refused with GDN_ERR_WORKSPACE_TOO_SMALL before anything is enqueued (the exact mode's split
 * needs 192 KiB per (segment, head): up to 682 of them; the truncate mode and unsplit runs need
 * none).  All calls on one device share its array, so calls that overlap on one device race;
 * nothing in the array needs to start at zero. */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
gdn_status gdn_chunk_fwd_noalloc(const gdn_problem *p, const void *q, const void *k,
                                 const void *v, const float *g, const void *beta,
                                 const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                                 const float *h0, void *o, float *ht, hipStream_t stream);

/* The forward's segment plan, for inspection.  Runs the forward's own unit lookup and warmup
 * scan on the device and writes to plan_out (device int32, capacity plan_capacity entries):
 *   plan_out[0] = number of units U, plan_out[1] = segment length L (0 = unsplit),
 *   then for each unit u: seq, first chunk, end chunk (chunk numbers counted from the sequence's
 *   first chunk), then H warmup-window first chunks (same numbering).  A sequence with no
 *   tokens has one unit with an empty chunk range (it only writes the final state).
 * Needs plan_capacity >= 2 + U * (3 + H); entries past the capacity are not written.  The
 * workspace arguments are those of gdn_chunk_fwd. */
gdn_status gdn_chunk_fwd_plan(const gdn_problem *p, const float *g, const int32_t *cu_seqlens,
                              const int32_t *cu_seqlens_host, int32_t *plan_out,
                              int64_t plan_capacity, void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* The forward with every per-chunk intermediate of the chunked form written out (fp32), for
 * checking each step separately; exact mode only.  Chunk c counts the chunks of all sequences
 * in order.  Any output may be NULL.
 *   gamma [T, H]            within-chunk cumulative sum of g
 *   tmat  [Nc, H, 64, 64]   (I + A)^{-1}, A_ri = beta_r exp(gamma_r - gamma_i) k_r.k_i (i < r)
 *   w     [Nc, H, 64, d_k]  W = Tm diag(beta exp(gamma)) K
 *   u     [Nc, H, 64, d_v]  U = Tm diag(beta) V
 *   hc    [Nc, H, d_k, d_v] the state at the start of each chunk
 *   delta [T, H, d_v]       Delta = U - W hc
 * Nc = sum over sequences of ceil(len / 64).  Rows past a partial chunk's length are zero. */
gdn_status gdn_chunk_fwd_intermediates(const gdn_problem *p, const void *q, const void *k,
                                       const void *v, const float *g, const void *beta,
                                       const int32_t *cu_seqlens, const float *h0, void *o,
                                       float *ht, float *gamma, float *tmat, float *w, float *u,
                                       float *hc, float *delta, void *workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace gdn_chunk_bwd needs for *p: the recomputed per-chunk
 * intermediates ("How to Speed Up GDN Kernels for Qwen Models", section "Lever 2": the hidden
 * states are recomputed in one pass, not stored by the forward), the reverse chain's per-chunk
 * state gradients and, when the exact split runs, its per-unit maps.  The per-chunk arrays are
 * sized on the chunk bound ceil(T / 64) + N (fewer than N chunks above the exact count), which
 * covers every chunk index a device table can produce.  cu_seqlens_host (optional, N + 1 host
 * int32, checked like the forward's) sets the split's segment length and unit count exactly
 * (without it the unit bound is used); pass the same pointer (or NULL) to gdn_chunk_bwd.
 * Host only. */
gdn_status gdn_chunk_bwd_workspace_size(const gdn_problem *p, const int32_t *cu_seqlens_host,
                                        size_t *bytes);

/* Backward of the forward: given dout (dtype, [T, H, d_v])
 * and optionally dht ([N, H, d_k, d_v] fp32, NULL = zero), writes dq, dk (dtype, [T, Hk, d_k];
 * with grouped heads, the sums over each key head's value heads),
 * dv (dtype, [T, H, d_v]), dg (fp32, [T, H]) and dbeta (dtype, [T, H]).  dh0 (optional, fp32)
 * receives the gradient of the initial states: [N, H, d_k, d_v] per sequence, or [H, d_k, d_v]
 * summed over all sequences when h0_seq_stride is 0 (a state shared by every sequence collects
 * the sum of their gradients, "Musings on long-context fine-tuning", section "Backward
 * through P").  Hidden states are recomputed, not stored ("How to Speed Up GDN Kernels for
 * Qwen Models", section "Lever 2").  cu_seqlens_host is optional, as for the workspace query.
 * Mode: the exact backward (GDN_MODE_EXACT), split along the sequences for bf16 with d = 128
 * as the exact forward is.  GDN_MODE_TRUNCATE, where that split applies, gives each segment
 * warmup windows instead of the split's extra passes ("Lever 1"): the recompute's start state
 * from the chunks before the segment whose summed g reaches trunc_log_threshold, and the state
 * gradient at the segment's end from the chunks after it, by the same rule (the reverse chain's
 * maps are the forward maps transposed and decay alike); elsewhere it is the exact backward. */
gdn_status gdn_chunk_bwd(const gdn_problem *p, const void *q, const void *k, const void *v,
                         const float *g, const void *beta, const int32_t *cu_seqlens,
                         const int32_t *cu_seqlens_host, const float *h0, const void *dout,
                         const float *dht, void *dq, void *dk, void *dv, float *dg, void *dbeta,
                         float *dh0, void *workspace, size_t workspace_bytes, hipStream_t stream);

/* One decode step ("How to Speed Up GDN Kernels for Qwen Models", section "FAQ": decode is the
 * recurrent step on one token): every (sequence b, head h) state advances by one token of the
 * recurrence above, in place,
 *     S <- exp(g) (I - beta k k^T) S + beta k v^T,    o = scale * S^T q   (S after the update).
 * Layouts (sequence-major, contiguous): q, k [batch, Hk, head_dim] and v, o [batch, num_heads,
 * head_dim] in dtype (GDN_DTYPE_*), Hk = num_k_heads (0 = num_heads; otherwise a divisor of
 * num_heads, value head h reading key head h / (num_heads / Hk) as in gdn_problem); g
 * [batch, num_heads] fp32; beta [batch, num_heads] in dtype; state [batch, num_heads, head_dim,
 * head_dim] fp32, read and overwritten.  qk_l2norm = 1: q and k are L2-normalised first, as in
 * gdn_problem.  head_dim is 64 or 128 (d_k = d_v).  All tensors are caller-owned device
 * memory, 16-byte aligned; no workspace.  Arguments are validated before anything is enqueued
 * (batch, num_heads >= 1; num_k_heads; qk_l2norm in {0, 1}; pointers). */
gdn_status gdn_decode_step(int32_t batch, int32_t num_heads, int32_t num_k_heads, int32_t head_dim,
                           int32_t dtype, int32_t qk_l2norm, float scale, const void *q,
                           const void *k, const void *v, const float *g, const void *beta,
                           float *state, void *o, hipStream_t stream);

/* Checks a cu_seqlens table on the device ("Step 10 · Making it fast": packed documents whose
 * boundaries are wrong leak into each other; "How to Speed Up GDN Kernels for Qwen Models",
 * section "Using it, and the fine print": misuse is refused).  Reads cu_seqlens[0..num_seqs]
 * (device int32) and writes to *status (device int32, caller-owned) 0 when the table is valid,
 * else a bit mask: 1 cu[0] != 0, 2 a descending pair, 4 cu[N] != total_tokens, 8 an offset
 * outside [0, total_tokens].  Asynchronous on `stream`; read *status after the stream's work.
 * Validates num_seqs >= 1, total_tokens in [0, 2^31) and the pointers before launching. */
gdn_status gdn_validate_cu_seqlens(const int32_t *cu_seqlens, int32_t num_seqs,
                                   int64_t total_tokens, int32_t *status, hipStream_t stream);

/* Debug mode on (1) or off (0) for the whole process; its initial value comes from the
 * environment variable GDN_DEBUG (unset or "0": off).  In debug mode gdn_chunk_fwd,
 * gdn_chunk_fwd_intermediates, gdn_chunk_fwd_plan and gdn_chunk_bwd validate cu_seqlens on the
 * device (and compare it with cu_seqlens_host when one is given) before their first launch and
 * synchronise the stream (so they are not asynchronous,
 * and calls that overlap on one device share its check words).  No passage applies: a
 * diagnostic of this library. */
gdn_status gdn_set_debug(int32_t on);
int32_t gdn_get_debug(void);

/* The current device's fault flags: bit 1 means a forward launch's bounded wait between its
 * waves ran out (its results are not to be trusted).  Synchronises the device, then copies the
 * flags to *flags (host) and clears them when clear != 0.  No passage applies: a diagnostic of
 * this library's kernels. */
gdn_status gdn_device_faults(uint32_t *flags, int32_t clear);

/* Static description of a status code.  No passage applies (error reporting of this library;
 * the page's library "raises" on what it cannot run, "How to Speed Up GDN Kernels for Qwen
 * Models", section "Using it, and the fine print"). */
const char *gdn_status_string(gdn_status s);

/* Detail of the last error on the calling thread (empty string if none).  No passage applies,
 * as for gdn_status_string. */
const char *gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
