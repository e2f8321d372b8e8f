/*
 * Gated DeltaNet oracle: a plain, slow, fp64 CPU implementation of the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call this file:
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg use it.  It
 * shares no code, header, table or helper with the HIP library.
 *
 * Sources (web pages; cited by title and section):
 *   [GDN-K]  "How to Speed Up GDN Kernels for Qwen Models" (netraruntime.com)
 *            - section "What GDN actually computes": per-head state S (d_k x d_v), decay gate
 *              alpha_t = exp(g_t), write strength beta_t, the delta-rule factor (I - beta k k^T),
 *              64-token chunks, one lower-triangular 64x64 system per chunk per head.
 *            - section "Lever 1: the gate is also a license to parallelize": warmup windows
 *              found by scanning the gates until the summed g passes -10; the segment-length
 *              latency model (proportional to sqrt(HN/P), times 3, power of two, floor 4).
 *            - section "Lever 2": gate cumsum once per chunk, triangular inverse reused by the
 *              output path and the state update.
 *   [LCF]    "Musings on long-context fine-tuning" (hardikmeisheri.github.io)
 *            - section "Isolating the recurrent layers": the update first decays the memory,
 *              then corrects what it predicts for the current key; the query reads the updated
 *              matrix; initial_state carries a state in, cu_seqlens marks boundaries.
 *            - section "Backward through P": gradients of a shared state add up.
 *
 * Conventions (all arrays row-major, token-major):
 *   q, k: [T, H, dk]   v: [T, H, dv]   g, beta: [T, H]   cu: int32 [N+1], cu[0] = 0, cu[N] = T
 *   h0: state of sequence n at h0 + n*h0_seq_stride, each [H, dk, dv] (NULL => zeros;
 *       h0_seq_stride = 0 broadcasts one state to every sequence)
 *   o: [T, H, dv]   ht: [N, H, dk, dv] (NULL => not written)
 * Parallelism: OpenMP over independent (sequence, head) pairs only; every pair's arithmetic is
 * sequential and in fp64, so results do not depend on the thread count.
 *
 * Every public function returns 0 on success and a negative value on bad arguments.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX_TH(t, h, H) ((int64_t)(t) * (H) + (h))

static int check_common(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv,
                        const int32_t *cu) {
  if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || T < 0 || !cu) return -1;
  if (cu[0] != 0 || cu[N] != T) return -2;
  for (int32_t n = 0; n < N; ++n)
    if (cu[n + 1] < cu[n]) return -3;
  return 0;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

static void load_state(double *S, const double *h0, int64_t h0_seq_stride, int32_t n, int32_t h,
                       int32_t dk, int32_t dv) {
  if (h0) {
    const double *src = h0 + (int64_t)n * h0_seq_stride + (int64_t)h * dk * dv;
    memcpy(S, src, sizeof(double) * (size_t)dk * dv);
  } else {
    memset(S, 0, sizeof(double) * (size_t)dk * dv);
  }
}

/* One token of the gated delta rule on state S (dk x dv), [GDN-K] "What GDN actually computes",
 * [LCF] "Isolating the recurrent layers":
 *     S <- alpha (I - beta k k^T) S + beta k v^T,   alpha = exp(g)
 * written as: decay first, predict from the decayed memory, write the correction along k:
 *     p = (alpha S)^T k ;  S <- alpha S + beta k (v - p)^T
 * and then the query reads the updated state:  o = scale * S^T q.                          */
static void token_step(double *S, const double *q, const double *k, const double *v, double g,
                       double beta, double scale, int32_t dk, int32_t dv, double *o,
                       double *tmp) {
  const double alpha = exp(g);
  for (int32_t j = 0; j < dv; ++j) {
    double p = 0.0;
    for (int32_t i = 0; i < dk; ++i) p += S[(int64_t)i * dv + j] * k[i];
    tmp[j] = beta * (v[j] - alpha * p); /* written correction */
  }
  for (int32_t i = 0; i < dk; ++i)
    for (int32_t j = 0; j < dv; ++j)
      S[(int64_t)i * dv + j] = alpha * S[(int64_t)i * dv + j] + k[i] * tmp[j];
  if (o) {
    for (int32_t j = 0; j < dv; ++j) {
      double acc = 0.0;
      for (int32_t i = 0; i < dk; ++i) acc += S[(int64_t)i * dv + j] * q[i];
      o[j] = scale * acc;
    }
  }
}

/* Token-by-token forward: the plain definition of the operation. */
int gdn_oracle_fwd_recurrent(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv,
                             const int32_t *cu, const double *q, const double *k,
                             const double *v, const double *g, const double *beta,
                             const double *h0, int64_t h0_seq_stride, double scale, double *o,
                             double *ht, int nthreads) {
  int rc = check_common(T, N, H, dk, dv, cu);
  if (rc) return rc;
  if (!q || !k || !v || !g || !beta || !o) return -1;
  set_threads(nthreads);
  int64_t units = (int64_t)N * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u) {
    int32_t n = (int32_t)(u / H), h = (int32_t)(u % H);
    double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
    double *tmp = (double *)malloc(sizeof(double) * (size_t)dv);
    load_state(S, h0, h0_seq_stride, n, h, dk, dv);
    for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
      int64_t th = IDX_TH(t, h, H);
      token_step(S, q + th * dk, k + th * dk, v + th * dv, g[th], beta[th], scale, dk, dv,
                 o + th * dv, tmp);
    }
    if (ht) memcpy(ht + u * dk * dv, S, sizeof(double) * (size_t)dk * dv);
    free(S);
    free(tmp);
  }
  return 0;
}

/* ---------------------------------------------------------------------------------------
 * Chunked form, written separately from the token form.  [GDN-K] "What GDN actually
 * computes" (chunks of C tokens, one triangular system per chunk per head) and "Lever 2"
 * (gate cumsum once per chunk; the inverse reused by output and state update), with the
 * chunked delta-rule algebra of the paper that section cites:
 *   gamma_r = sum_{s<=r} g_s                                  (within the chunk)
 *   A_ri    = beta_r exp(gamma_r - gamma_i) k_r.k_i   for i < r, else 0
 *   Tm      = (I + A)^{-1}                                    (unit lower triangular)
 *   W       = Tm diag(beta exp(gamma)) K ;  U = Tm diag(beta) V
 *   Delta   = U - W h                                         (h = state at chunk start)
 *   O       = diag(exp(gamma)) Q h + ((Q K^T) o D o [i<=r]) Delta,  D_ri = exp(gamma_r-gamma_i)
 *   h_next  = exp(gamma_last) h + (diag(exp(gamma_last - gamma)) K)^T Delta
 * Chunks start at each sequence's first token; a sequence's last chunk may be partial.
 *
 * Optional intermediates (any may be NULL); chunk index c counts chunks of all sequences in
 * order (sequence 0's chunks first):
 *   gamma_out [T, H]          tm_out [nc, H, C, C]    w_out [nc, H, C, dk]
 *   u_out [nc, H, C, dv]      hc_out [nc, H, dk, dv]  delta_out [T, H, dv]
 * Rows of tm/w/u past a partial chunk's length are left zero.
 * ------------------------------------------------------------------------------------- */
int64_t gdn_oracle_num_chunks(int32_t N, const int32_t *cu, int32_t C) {
  int64_t nc = 0;
  for (int32_t n = 0; n < N; ++n) nc += (cu[n + 1] - cu[n] + C - 1) / C;
  return nc;
}

int gdn_oracle_fwd_chunked(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv,
                           const int32_t *cu, int32_t C, const double *q, const double *k,
                           const double *v, const double *g, const double *beta,
                           const double *h0, int64_t h0_seq_stride, double scale, double *o,
                           double *ht, double *gamma_out, double *tm_out, double *w_out,
                           double *u_out, double *hc_out, double *delta_out, int nthreads) {
  int rc = check_common(T, N, H, dk, dv, cu);
  if (rc) return rc;
  if (C <= 0 || !q || !k || !v || !g || !beta || !o) return -1;
  set_threads(nthreads);
  /* first chunk index of every sequence */
  int64_t *chunk0 = (int64_t *)malloc(sizeof(int64_t) * (size_t)(N + 1));
  chunk0[0] = 0;
  for (int32_t n = 0; n < N; ++n) chunk0[n + 1] = chunk0[n] + (cu[n + 1] - cu[n] + C - 1) / C;

  int64_t units = (int64_t)N * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u) {
    int32_t n = (int32_t)(u / H), h = (int32_t)(u % H);
    size_t sz = (size_t)dk * dv;
    double *S = (double *)malloc(sizeof(double) * sz);
    double *Snew = (double *)malloc(sizeof(double) * sz);
    double *gam = (double *)malloc(sizeof(double) * C);
    double *A = (double *)calloc((size_t)C * C, sizeof(double));
    double *Tm = (double *)calloc((size_t)C * C, sizeof(double));
    double *W = (double *)calloc((size_t)C * dk, sizeof(double));
    double *U = (double *)calloc((size_t)C * dv, sizeof(double));
    double *Dl = (double *)calloc((size_t)C * dv, sizeof(double));
    load_state(S, h0, h0_seq_stride, n, h, dk, dv);

    int64_t t0 = cu[n], t1 = cu[n + 1];
    for (int64_t cs = t0, c = chunk0[n]; cs < t1; cs += C, ++c) {
      int32_t len = (int32_t)((t1 - cs) < C ? (t1 - cs) : C);
#define Q_(r, i) q[IDX_TH(cs + (r), h, H) * dk + (i)]
#define K_(r, i) k[IDX_TH(cs + (r), h, H) * dk + (i)]
#define V_(r, j) v[IDX_TH(cs + (r), h, H) * dv + (j)]
#define G_(r) g[IDX_TH(cs + (r), h, H)]
#define B_(r) beta[IDX_TH(cs + (r), h, H)]
      /* gate cumsum */
      double run = 0.0;
      for (int32_t r = 0; r < len; ++r) {
        run += G_(r);
        gam[r] = run;
      }
      double glast = gam[len - 1];
      /* A = strict_lower(diag(beta) (K K^T o D)) */
      for (int32_t r = 0; r < len; ++r)
        for (int32_t i = 0; i < len; ++i) {
          double a = 0.0;
          if (i < r) {
            double dot = 0.0;
            for (int32_t d = 0; d < dk; ++d) dot += K_(r, d) * K_(i, d);
            a = B_(r) * exp(gam[r] - gam[i]) * dot;
          }
          A[(int64_t)r * C + i] = a;
        }
      /* Tm = (I + A)^{-1} by forward substitution, one column at a time:
       * row r of (I + A) Tm = I gives Tm[r][j] = delta_rj - sum_{i<r} A[r][i] Tm[i][j]. */
      memset(Tm, 0, sizeof(double) * (size_t)C * C);
      for (int32_t j = 0; j < len; ++j) {
        Tm[(int64_t)j * C + j] = 1.0;
        for (int32_t r = j + 1; r < len; ++r) {
          double acc = 0.0;
          for (int32_t i = j; i < r; ++i) acc += A[(int64_t)r * C + i] * Tm[(int64_t)i * C + j];
          Tm[(int64_t)r * C + j] = -acc;
        }
      }
      /* W = Tm diag(beta e^gamma) K ; U = Tm diag(beta) V */
      memset(W, 0, sizeof(double) * (size_t)C * dk);
      memset(U, 0, sizeof(double) * (size_t)C * dv);
      for (int32_t r = 0; r < len; ++r) {
        for (int32_t d = 0; d < dk; ++d) {
          double acc = 0.0;
          for (int32_t i = 0; i <= r; ++i)
            acc += Tm[(int64_t)r * C + i] * B_(i) * exp(gam[i]) * K_(i, d);
          W[(int64_t)r * dk + d] = acc;
        }
        for (int32_t j = 0; j < dv; ++j) {
          double acc = 0.0;
          for (int32_t i = 0; i <= r; ++i) acc += Tm[(int64_t)r * C + i] * B_(i) * V_(i, j);
          U[(int64_t)r * dv + j] = acc;
        }
      }
      /* Delta = U - W h */
      for (int32_t r = 0; r < len; ++r)
        for (int32_t j = 0; j < dv; ++j) {
          double acc = 0.0;
          for (int32_t d = 0; d < dk; ++d) acc += W[(int64_t)r * dk + d] * S[(int64_t)d * dv + j];
          Dl[(int64_t)r * dv + j] = U[(int64_t)r * dv + j] - acc;
        }
      /* O = diag(e^gamma) Q h + ((Q K^T) o D o [i<=r]) Delta */
      for (int32_t r = 0; r < len; ++r)
        for (int32_t j = 0; j < dv; ++j) {
          double inter = 0.0;
          for (int32_t d = 0; d < dk; ++d) inter += Q_(r, d) * S[(int64_t)d * dv + j];
          double intra = 0.0;
          for (int32_t i = 0; i <= r; ++i) {
            double qk = 0.0;
            for (int32_t d = 0; d < dk; ++d) qk += Q_(r, d) * K_(i, d);
            intra += qk * exp(gam[r] - gam[i]) * Dl[(int64_t)i * dv + j];
          }
          o[IDX_TH(cs + r, h, H) * dv + j] = scale * (exp(gam[r]) * inter + intra);
        }
      /* intermediates */
      if (gamma_out)
        for (int32_t r = 0; r < len; ++r) gamma_out[IDX_TH(cs + r, h, H)] = gam[r];
      if (delta_out)
        for (int32_t r = 0; r < len; ++r)
          for (int32_t j = 0; j < dv; ++j)
            delta_out[IDX_TH(cs + r, h, H) * dv + j] = Dl[(int64_t)r * dv + j];
      int64_t ch = c * H + h;
      if (tm_out) memcpy(tm_out + ch * C * C, Tm, sizeof(double) * (size_t)C * C);
      if (w_out) memcpy(w_out + ch * C * dk, W, sizeof(double) * (size_t)C * dk);
      if (u_out) memcpy(u_out + ch * C * dv, U, sizeof(double) * (size_t)C * dv);
      if (hc_out) memcpy(hc_out + ch * (int64_t)sz, S, sizeof(double) * sz);
      /* h_next = e^{gamma_last} h + (diag(e^{gamma_last - gamma}) K)^T Delta */
      for (int32_t d = 0; d < dk; ++d)
        for (int32_t j = 0; j < dv; ++j) {
          double acc = exp(glast) * S[(int64_t)d * dv + j];
          for (int32_t r = 0; r < len; ++r)
            acc += exp(glast - gam[r]) * K_(r, d) * Dl[(int64_t)r * dv + j];
          Snew[(int64_t)d * dv + j] = acc;
        }
      memcpy(S, Snew, sizeof(double) * sz);
#undef Q_
#undef K_
#undef V_
#undef G_
#undef B_
    }
    if (ht) memcpy(ht + u * (int64_t)sz, S, sizeof(double) * sz);
    free(S); free(Snew); free(gam); free(A); free(Tm); free(W); free(U); free(Dl);
  }
  free(chunk0);
  return 0;
}

/* ---------------------------------------------------------------------------------------
 * Segment plan for history truncation, [GDN-K] "Lever 1".
 *
 * Segment length in chunks (the latency model): the optimum is proportional to
 * sqrt(H * Nc / P) with H heads, Nc total chunks and P compute units; it is scaled by 3,
 * rounded to the nearest power of two (in log2) and floored at 4 chunks.  The proportionality
 * constant is not printed on the page; 1 is taken.  A seg_chunks > 0 argument forces L.
 * Splitting applies only when N * H < P (the batch does not fill the machine); otherwise
 * each sequence is one segment.
 *
 * Warmup window: for a segment starting at chunk c0 of its sequence (c0 > the sequence's
 * first chunk), per head, whole preceding chunks are taken one by one (c0-1, c0-2, ...) and
 * their gates summed (in fp64) until the sum is strictly below log_threshold (-10 on the
 * page); the window starts at the last chunk taken.  A window that reaches the sequence's
 * first chunk without passing the threshold starts there, from the true initial state.
 *
 * Outputs (capacity max_segments): seg_seq, seg_c0, seg_c1 (chunk range [c0, c1) within the
 * sequence, counted from the sequence's first chunk), warm_c [S, H] (first chunk of the
 * window, in the same numbering).  Returns the number of segments, or < 0 on error.
 * ------------------------------------------------------------------------------------- */
int32_t gdn_oracle_segment_chunks(int32_t H, int64_t total_chunks, int32_t num_seqs, int32_t P,
                                  int32_t forced) {
  if (forced > 0) return forced;
  if ((int64_t)num_seqs * H >= P) return 0; /* 0 => no split */
  double lstar = 3.0 * sqrt((double)H * (double)total_chunks / (double)P);
  double e = floor(log2(lstar) + 0.5);
  int32_t L = (int32_t)ldexp(1.0, (int)e);
  if (L < 4) L = 4;
  return L;
}

int32_t gdn_oracle_plan(int64_t T, int32_t N, int32_t H, const int32_t *cu, const double *g,
                        int32_t C, int32_t P, int32_t seg_chunks, double log_threshold,
                        int32_t max_segments, int32_t *seg_seq, int32_t *seg_c0, int32_t *seg_c1,
                        int32_t *warm_c) {
  if (check_common(T, N, H, 1, 1, cu)) return -1;
  if (C <= 0 || !g || !seg_seq || !seg_c0 || !seg_c1 || !warm_c) return -1;
  int64_t nc = gdn_oracle_num_chunks(N, cu, C);
  int32_t L = gdn_oracle_segment_chunks(H, nc, N, P, seg_chunks);
  int32_t ns = 0;
  for (int32_t n = 0; n < N; ++n) {
    int32_t chunks = (cu[n + 1] - cu[n] + C - 1) / C;
    int32_t step = (L > 0) ? L : (chunks > 0 ? chunks : 1);
    for (int32_t c0 = 0; c0 < chunks; c0 += step) {
      if (ns >= max_segments) return -4;
      int32_t c1 = c0 + step < chunks ? c0 + step : chunks;
      seg_seq[ns] = n;
      seg_c0[ns] = c0;
      seg_c1[ns] = c1;
      for (int32_t h = 0; h < H; ++h) {
        int32_t w = c0;
        double acc = 0.0;
        while (w > 0 && !(acc < log_threshold)) {
          --w;
          int64_t a = cu[n] + (int64_t)w * C;
          int64_t b = a + C; /* whole chunk: w < c0 <= chunks-1, so it is full */
          for (int64_t t = a; t < b; ++t) acc += g[IDX_TH(t, h, H)];
        }
        warm_c[(int64_t)ns * H + h] = w;
      }
      ++ns;
    }
  }
  return ns;
}

/* Truncated-history forward: every (segment, head) runs the token recurrence from its warmup
 * window's first chunk, starting from zero (or from the true initial state when the window
 * begins at the sequence start), and emits outputs only for its own chunks.  The final state
 * of a sequence is taken from its last segment; a sequence with no tokens returns h0 (or 0). */
int gdn_oracle_fwd_truncated(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv,
                             const int32_t *cu, int32_t C, const double *q, const double *k,
                             const double *v, const double *g, const double *beta,
                             const double *h0, int64_t h0_seq_stride, double scale,
                             int32_t num_segments, const int32_t *seg_seq, const int32_t *seg_c0,
                             const int32_t *seg_c1, const int32_t *warm_c, double *o, double *ht,
                             int nthreads) {
  int rc = check_common(T, N, H, dk, dv, cu);
  if (rc) return rc;
  if (!q || !k || !v || !g || !beta || !o || num_segments < 0) return -1;
  set_threads(nthreads);
  if (ht) /* sequences with no tokens keep their initial state */
    for (int32_t n = 0; n < N; ++n)
      if (cu[n + 1] == cu[n])
        for (int32_t h = 0; h < H; ++h)
          load_state(ht + ((int64_t)n * H + h) * dk * dv, h0, h0_seq_stride, n, h, dk, dv);
  int64_t units = (int64_t)num_segments * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u) {
    int32_t s = (int32_t)(u / H), h = (int32_t)(u % H);
    int32_t n = seg_seq[s];
    int32_t w = warm_c[(int64_t)s * H + h];
    double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
    double *tmp = (double *)malloc(sizeof(double) * (size_t)dv);
    if (w == 0) load_state(S, h0, h0_seq_stride, n, h, dk, dv);
    else memset(S, 0, sizeof(double) * (size_t)dk * dv);
    int64_t tw = cu[n] + (int64_t)w * C;
    int64_t ta = cu[n] + (int64_t)seg_c0[s] * C;
    int64_t tb = cu[n] + (int64_t)seg_c1[s] * C;
    if (tb > cu[n + 1]) tb = cu[n + 1];
    for (int64_t t = tw; t < tb; ++t) {
      int64_t th = IDX_TH(t, h, H);
      token_step(S, q + th * dk, k + th * dk, v + th * dv, g[th], beta[th], scale, dk, dv,
                 t >= ta ? o + th * dv : NULL, tmp);
    }
    if (ht && tb == cu[n + 1])
      memcpy(ht + ((int64_t)n * H + h) * dk * dv, S, sizeof(double) * (size_t)dk * dv);
    free(S);
    free(tmp);
  }
  return 0;
}

/* ---------------------------------------------------------------------------------------
 * Backward of the token recurrence, derived by hand from token_step (reverse-mode chain rule).
 * With G = dL/dS_t (from later tokens), per token t in reverse:
 *     G   += scale q_t do_t^T                ; dq_t = scale S_t do_t
 *     p    = S_{t-1}^T k_t ; r = G^T k_t ; u = v_t - alpha_t p
 *     dv_t = beta_t r ; dbeta_t = r.u
 *     dg_t = alpha_t ( <G, S_{t-1}>_F - beta_t r.p )
 *     dk_t = beta_t G u - alpha_t beta_t S_{t-1} r
 *     G    = alpha_t (G - beta_t k_t (k_t^T G))
 * and dh0 is G after the sequence's first token.  G starts at dht (or 0).  States are
 * checkpointed every C tokens in a forward pass and recomputed inside each block.
 * Gradients of a shared initial state add up over the sequences that read it ([LCF]
 * "Backward through P"); this function returns dh0 per sequence, [N, H, dk, dv], and the
 * caller sums over sequences that share one state.
 * ------------------------------------------------------------------------------------- */
int gdn_oracle_bwd(int64_t T, int32_t N, int32_t H, int32_t dk, int32_t dv, const int32_t *cu,
                   const double *q, const double *k, const double *v, const double *g,
                   const double *beta, const double *h0, int64_t h0_seq_stride, double scale,
                   const double *dout, const double *dht, double *dq, double *dk_out,
                   double *dv_out, double *dg, double *dbeta, double *dh0, int nthreads) {
  const int32_t C = 64;
  int rc = check_common(T, N, H, dk, dv, cu);
  if (rc) return rc;
  if (!q || !k || !v || !g || !beta || !dout || !dq || !dk_out || !dv_out || !dg || !dbeta)
    return -1;
  set_threads(nthreads);
  int64_t units = (int64_t)N * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t u = 0; u < units; ++u) {
    int32_t n = (int32_t)(u / H), h = (int32_t)(u % H);
    size_t sz = (size_t)dk * dv;
    int64_t t0 = cu[n], t1 = cu[n + 1], len = t1 - t0;
    int64_t nblk = (len + C - 1) / C;
    double *ck = (double *)malloc(sizeof(double) * sz * (size_t)(nblk > 0 ? nblk : 1));
    double *St = (double *)malloc(sizeof(double) * sz * (C + 1)); /* states inside a block */
    double *G = (double *)malloc(sizeof(double) * sz);
    double *tmp = (double *)malloc(sizeof(double) * (size_t)dv);
    double *p = (double *)malloc(sizeof(double) * (size_t)dv);
    double *r = (double *)malloc(sizeof(double) * (size_t)dv);
    double *uu = (double *)malloc(sizeof(double) * (size_t)dv);
    double *kG = (double *)malloc(sizeof(double) * (size_t)dv);
    /* forward pass: checkpoint the state at the start of every block */
    double *S = St;
    load_state(S, h0, h0_seq_stride, n, h, dk, dv);
    for (int64_t b = 0; b < nblk; ++b) {
      memcpy(ck + b * sz, S, sizeof(double) * sz);
      int64_t e = t0 + (b + 1) * C < t1 ? t0 + (b + 1) * C : t1;
      for (int64_t t = t0 + b * C; t < e; ++t) {
        int64_t th = IDX_TH(t, h, H);
        token_step(S, NULL, k + th * dk, v + th * dv, g[th], beta[th], scale, dk, dv, NULL, tmp);
      }
    }
    if (dht) memcpy(G, dht + u * (int64_t)sz, sizeof(double) * sz);
    else memset(G, 0, sizeof(double) * sz);
    for (int64_t b = nblk - 1; b >= 0; --b) {
      int64_t a = t0 + b * C;
      int64_t e = a + C < t1 ? a + C : t1;
      int64_t m = e - a;
      memcpy(St, ck + b * sz, sizeof(double) * sz);
      for (int64_t i = 0; i < m; ++i) {
        int64_t th = IDX_TH(a + i, h, H);
        memcpy(St + (i + 1) * sz, St + i * sz, sizeof(double) * sz);
        token_step(St + (i + 1) * sz, NULL, k + th * dk, v + th * dv, g[th], beta[th], scale,
                   dk, dv, NULL, tmp);
      }
      for (int64_t i = m - 1; i >= 0; --i) {
        int64_t th = IDX_TH(a + i, h, H);
        const double *Sp = St + i * sz, *Sc = St + (i + 1) * sz;
        const double *qt = q + th * dk, *kt = k + th * dk, *vt = v + th * dv,
                     *dot = dout + th * dv;
        double alpha = exp(g[th]), bt = beta[th];
        /* output read: o = scale S_t^T q */
        for (int32_t d = 0; d < dk; ++d)
          for (int32_t j = 0; j < dv; ++j) G[(int64_t)d * dv + j] += scale * qt[d] * dot[j];
        for (int32_t d = 0; d < dk; ++d) {
          double acc = 0.0;
          for (int32_t j = 0; j < dv; ++j) acc += Sc[(int64_t)d * dv + j] * dot[j];
          dq[th * dk + d] = scale * acc;
        }
        for (int32_t j = 0; j < dv; ++j) {
          double pj = 0.0, rj = 0.0;
          for (int32_t d = 0; d < dk; ++d) {
            pj += Sp[(int64_t)d * dv + j] * kt[d];
            rj += G[(int64_t)d * dv + j] * kt[d];
          }
          p[j] = pj;
          r[j] = rj;
          uu[j] = vt[j] - alpha * pj;
        }
        double db = 0.0, rp = 0.0, gs = 0.0;
        for (int32_t j = 0; j < dv; ++j) {
          dv_out[th * dv + j] = bt * r[j];
          db += r[j] * uu[j];
          rp += r[j] * p[j];
        }
        for (int64_t e2 = 0; e2 < (int64_t)sz; ++e2) gs += G[e2] * Sp[e2];
        dbeta[th] = db;
        dg[th] = alpha * (gs - bt * rp);
        for (int32_t d = 0; d < dk; ++d) {
          double a1 = 0.0, a2 = 0.0;
          for (int32_t j = 0; j < dv; ++j) {
            a1 += G[(int64_t)d * dv + j] * uu[j];
            a2 += Sp[(int64_t)d * dv + j] * r[j];
          }
          dk_out[th * dk + d] = bt * a1 - alpha * bt * a2;
        }
        /* propagate to the previous state: G <- alpha (G - beta k (k^T G)) */
        for (int32_t j = 0; j < dv; ++j) kG[j] = r[j];
        for (int32_t d = 0; d < dk; ++d)
          for (int32_t j = 0; j < dv; ++j)
            G[(int64_t)d * dv + j] = alpha * (G[(int64_t)d * dv + j] - bt * kt[d] * kG[j]);
      }
    }
    if (dh0) memcpy(dh0 + u * (int64_t)sz, G, sizeof(double) * sz);
    free(ck); free(St); free(G); free(tmp); free(p); free(r); free(uu); free(kG);
  }
  return 0;
}

/* L2 normalisation of rows (the optional first step of the op on q and k): y = x / sqrt(|x|^2 +
 * eps) per row of d elements. */
int gdn_oracle_l2norm(int64_t rows, int32_t d, const double *x, double eps, double *y) {
  if (rows < 0 || d < 1 || !(eps >= 0.0) || (rows > 0 && (!x || !y))) return -1;
  for (int64_t r = 0; r < rows; ++r) {
    double s = 0.0;
    for (int32_t i = 0; i < d; ++i) s += x[r * d + i] * x[r * d + i];
    const double inv = 1.0 / sqrt(s + eps);
    for (int32_t i = 0; i < d; ++i) y[r * d + i] = x[r * d + i] * inv;
  }
  return 0;
}

/* Its backward: with r = (|x|^2 + eps)^(-1/2) and y = r x, dy_i/dx_j = r delta_ij - r^3 x_i x_j,
 * so dx = r (dy - y (y . dy)). */
int gdn_oracle_l2norm_bwd(int64_t rows, int32_t d, const double *x, const double *dy, double eps,
                          double *dx) {
  if (rows < 0 || d < 1 || !(eps >= 0.0) || (rows > 0 && (!x || !dy || !dx))) return -1;
  for (int64_t r = 0; r < rows; ++r) {
    double s = 0.0;
    for (int32_t i = 0; i < d; ++i) s += x[r * d + i] * x[r * d + i];
    const double inv = 1.0 / sqrt(s + eps);
    double ydy = 0.0;
    for (int32_t i = 0; i < d; ++i) ydy += inv * x[r * d + i] * dy[r * d + i];
    for (int32_t i = 0; i < d; ++i) dx[r * d + i] = inv * (dy[r * d + i] - inv * x[r * d + i] * ydy);
  }
  return 0;
}

int gdn_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
