// Forward of the chunked gated delta rule on gfx950.
//
// Method: "How to Speed Up GDN Kernels for Qwen Models", sections "What GDN actually computes"
// (64-token chunks, one 64x64 lower-triangular system per chunk and head, a sequential state
// hand-off between chunks), "Lever 1" (history truncation and sequence splitting) and
// "Lever 2" (gate cumsum once per chunk, folded into the matrix operands; the triangular
// inverse reused by the output path and the state update).  Per chunk of n <= 64 tokens with
// the state h at its start:
//   gamma = cumsum(g);  A_ri = beta_r exp(gamma_r - gamma_i) k_r.k_i (i < r);  Tm = (I + A)^-1
//   W = Tm diag(beta e^gamma) K;  U = Tm diag(beta) V;  Delta = U - W h
//   O = diag(e^gamma) Q h + (Q K^T o exp(gamma_r - gamma_i) [i <= r]) Delta
//   h <- e^{gamma_last} h + K^T diag(e^{gamma_last - gamma}) Delta
//
// Work decomposition (one workgroup of 4 waves per (unit, head)):
//   * the d_k x d_v fp32 state stays in registers for the whole unit; wave w owns state columns
//     [w d_v/4, (w+1) d_v/4) as 16x16 MFMA accumulator tiles, so the chain never touches LDS
//     or HBM for the state;
//   * Q, K, V of a chunk are staged token-major in LDS with coalesced 16-byte loads; products
//     that contract over tokens read K and V through the LDS transpose read, so no transposed
//     copy is made;
//   * state-side operands (the state as the B operand of W h and Q h, Delta as the B operand
//     of P Delta and of the state update) are converted from the accumulator layout in
//     registers: the contraction index is permuted the same way on both operands, which the
//     sum does not see;
//   * dense products run on v_mfma_f32_16x16x32_bf16 (bf16 inputs) or v_mfma_f32_16x16x4_f32
//     (fp32 inputs); the triangular solve's off-diagonal blocks always use fp32 MFMA.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_tiles.h"
#include "gdn_unit.h"

namespace gdn {

// ------------------------------------------------------------------------------ planning
// A unit is one (sequence, chunk range) pair; the forward runs one workgroup per (unit, head).
// With L == 0 every sequence is one unit; with L > 0 a sequence of c chunks is split into
// max(1, ceil(c / L)) units of L chunks (the last one shorter).  A sequence with no tokens
// still gets one (empty) unit so that its final state is written.

__global__ __launch_bounds__(64) void plan_export_kernel(const int32_t *__restrict__ cu, int N,
                                                         int64_t T, const float *__restrict__ g,
                                                         int H,
                                                         int L, float thr, int truncate,
                                                         int32_t *__restrict__ out,
                                                         int64_t capacity) {
  const int u = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  Unit un;
  const bool ok = find_unit(cu, N, T, L, u, false, lane, un);
  // the last workgroup that finds a unit also writes the header
  Unit nx;
  const bool next = find_unit(cu, N, T, L, u + 1, false, lane, nx);
  if (ok && !next && h == 0 && lane == 0 && capacity >= 2) {
    out[0] = u + 1;
    out[1] = L;
  }
  if (!ok) return;
  const int64_t base = 2 + (int64_t)u * (3 + H);
  if (base + 3 + H > capacity) return;
  int w = un.c0;
  if (truncate && un.c0 > 0) w = warm_window(g, cu[un.seq], un.c0, h, H, thr, lane);
  if (lane == 0) {
    if (h == 0) {
      out[base + 0] = un.seq;
      out[base + 1] = un.c0;
      out[base + 2] = un.c1;
    }
    out[base + 3 + h] = w;
  }
}

hipError_t launch_plan_export(const int32_t *cu, int32_t N, int64_t T, const float *g, int32_t H,
                              int32_t L, float log_thr, int32_t truncate, int64_t max_units,
                              int32_t *out, int64_t capacity, hipStream_t stream) {
  hipLaunchKernelGGL(plan_export_kernel, dim3((unsigned)max_units, H), dim3(64), 0, stream, cu,
                     N, T, g, H, L, log_thr, truncate, out, capacity);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ fused forward
template <int D, bool BF16>
struct FwdSmem {
  using E = typename std::conditional<BF16, bf16, float>::type;
  // Row strides (elements).  bf16 rows are padded by 32 bytes, fp32 rows by 16 bytes; every row
  // starts 16-byte aligned.
  static constexpr int LDE = D + (BF16 ? 16 : 4);
  static constexpr int LDT = 64 + 4;
  alignas(16) E q[64 * LDE];    // Q of the chunk, then O staged for the store
  alignas(16) E k[64 * LDE];    // K
  alignas(16) E vw[64 * LDE];   // V, then W
  alignas(16) float t[64 * LDT];   // Tm = (I + A)^-1
  alignas(16) float ap[64 * LDT];  // A, then P = (Q K^T) o decay o causal mask
  alignas(16) float gam[64];       // gamma (within-chunk cumsum of g)
  alignas(16) float beta[64];
  alignas(16) float eg[64];        // exp(gamma)
  alignas(16) float el[64];        // exp(gamma_last - gamma)
  alignas(16) float misc[4];
  alignas(16) int imisc[4];
};

// Tm_bc = -Tm_bb * sum_{j=c}^{b-1} A_bj Tm_jc for one 16x16 block below the diagonal (the
// blocked inverse of a unit lower-triangular matrix), fp32 MFMA.  One wave.
template <int LDT>
__device__ __forceinline__ void solve_offdiag_block(float *__restrict__ t,
                                                    const float *__restrict__ ap, int b, int c,
                                                    int gq, int cl) {
  f32x4 acc = zero4();
  for (int j = c; j < b; ++j) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float av = ap[(16 * b + cl) * LDT + 16 * j + 4 * s + gq];
      const float bv = t[(16 * j + 4 * s + gq) * LDT + 16 * c + cl];
      acc = mma_f32(av, bv, acc);
    }
  }
  f32x4 out = zero4();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float av = t[(16 * b + cl) * LDT + 16 * b + 4 * gq + i];
    out = mma_f32(av, acc[i], out);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) t[(16 * b + 4 * gq + i) * LDT + 16 * c + cl] = -out[i];
}

// The optional q/k L2 normalisation on a 64-row fp32 tile in LDS: row r / sqrt(|row r|^2 + eps),
// four threads per row (rows past a ragged chunk's end are zero and stay zero).
template <int D, int LDE>
__device__ __forceinline__ void normalize_rows(float *__restrict__ t, int tid) {
  const int r = tid >> 2, part = tid & 3;
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < D / 4; ++j) s += t[r * LDE + part + 4 * j] * t[r * LDE + part + 4 * j];
  s += __shfl_xor(s, 1, 64);
  s += __shfl_xor(s, 2, 64);
  const float inv = 1.f / sqrtf(s + kL2NormEps);
#pragma unroll
  for (int j = 0; j < D / 4; ++j) t[r * LDE + part + 4 * j] *= inv;
}

// The same on a bf16 tile: the scaled rows are rounded back to bf16 (the d = 64 bf16 path's
// reading of the normalisation, as a separate normalisation writing bf16 would give).
template <int D, int LDE>
__device__ __forceinline__ void normalize_rows(bf16 *__restrict__ t, int tid) {
  const int r = tid >> 2, part = tid & 3;
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < D / 4; ++j) {
    const float x = (float)t[r * LDE + part + 4 * j];
    s += x * x;
  }
  s += __shfl_xor(s, 1, 64);
  s += __shfl_xor(s, 2, 64);
  const float inv = 1.f / sqrtf(s + kL2NormEps);
#pragma unroll
  for (int j = 0; j < D / 4; ++j)
    t[r * LDE + part + 4 * j] = (bf16)(inv * (float)t[r * LDE + part + 4 * j]);
}

template <int D, bool BF16, bool DUMP>
__global__ __launch_bounds__(256) void fwd_kernel(FwdArgs a) {
  using SM = FwdSmem<D, BF16>;
  using E = typename SM::E;
  constexpr int LDE = SM::LDE, LDT = SM::LDT;
  constexpr int NT = D / 64;   // 16-column tiles of the state per wave
  constexpr int MTD = D / 16;  // 16-row tiles of the state (d_k)
  __shared__ SM sm;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, gq = lane >> 4, cl = lane & 15;
  const int unit = blockIdx.x, h = blockIdx.y, H = a.H;
  if (wave == 0) {
    Unit un;
    const bool ok = find_unit(a.cu, a.N, a.T, a.L, unit, DUMP, lane, un);
    if (lane == 0) {
      sm.imisc[0] = ok ? un.seq : -1;
      sm.imisc[1] = un.c0;
      sm.imisc[2] = un.c1;
      sm.imisc[3] = (int)un.chunk_base;
    }
  }
  __syncthreads();
  const int seq = sm.imisc[0];
  if (seq < 0) return;
  const int c0 = sm.imisc[1], c1 = sm.imisc[2];
  const int64_t chunk_base = sm.imisc[3];
  const int64_t ts0 = a.cu[seq], ts1 = a.cu[seq + 1];
  if (ts0 < 0 || ts1 < ts0 || ts1 > a.T) return;  // malformed cu_seqlens: touch nothing
  const int nchunks_seq = (int)((ts1 - ts0 + kChunk - 1) / kChunk);
  const int hk = h / (H / a.HK);  // this value head's key head
  const E *__restrict__ gq_ = static_cast<const E *>(a.q);
  const E *__restrict__ gk_ = static_cast<const E *>(a.k);
  const E *__restrict__ gv_ = static_cast<const E *>(a.v);
  const E *__restrict__ gb_ = static_cast<const E *>(a.beta);
  E *__restrict__ go_ = static_cast<E *>(a.o);

  // Blocks above the diagonal of Tm and of A/P are never written by the chunk loop: zero once.
  for (int i = tid; i < 64 * 64; i += 256) {
    const int r = i >> 6, c = i & 63;
    if ((c >> 4) > (r >> 4)) {
      sm.t[r * LDT + c] = 0.f;
      sm.ap[r * LDT + c] = 0.f;
    }
  }

  int cw = c0;
  if (a.truncate && c0 > 0) {
    __syncthreads();  // every wave has read the unit from imisc
    if (wave == 0) {
      const int w = warm_window(a.g, ts0, c0, h, H, a.log_thr, lane);
      if (lane == 0) sm.imisc[0] = w;
    }
    __syncthreads();
    cw = sm.imisc[0];
  }

  const int ncol0 = wave * (D / 4);
  f32x4 S[MTD][NT];
  // start state: the unit's true start state when the caller provides one per unit (the exact
  // split's composed states), else h0 at a sequence's start, else zero
  const float *hp = a.unit_h0 != nullptr ? a.unit_h0 + ((int64_t)unit * H + h) * D * D
                    : (cw == 0 && a.h0 != nullptr)
                        ? a.h0 + (int64_t)seq * a.h0_stride + (int64_t)h * D * D
                        : nullptr;
  if (hp != nullptr) {
#pragma unroll
    for (int mt = 0; mt < MTD; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          S[mt][nt][i] = hp[(16 * mt + 4 * gq + i) * D + ncol0 + 16 * nt + cl];
  } else {
#pragma unroll
    for (int mt = 0; mt < MTD; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) S[mt][nt] = zero4();
  }

  for (int c = cw; c < c1; ++c) {
    const bool emit = (c >= c0);
    const int64_t t0 = ts0 + (int64_t)c * kChunk;
    const int n = (int)min<int64_t>(kChunk, ts1 - t0);
    const int64_t cglob = chunk_base + c;
    __syncthreads();  // the previous chunk is done with LDS

    // ---- stage K, V (and Q) token-major in LDS
    load_tile<E, D, LDE>(sm.k, gk_, t0, n, hk, a.HK, tid);
    load_tile<E, D, LDE>(sm.vw, gv_, t0, n, h, H, tid);
    if (emit) load_tile<E, D, LDE>(sm.q, gq_, t0, n, hk, a.HK, tid);

    // ---- gate cumsum and folded decay factors (row a1)
    if (wave == 0) {
      const float gv = lane < n ? a.g[(t0 + lane) * H + h] : 0.f;
      const float bv = lane < n ? to_f32(gb_[(t0 + lane) * H + h]) : 0.f;
      const float gam = wave_inclusive_scan(gv, lane);
      const float glast = __shfl(gam, n - 1, 64);
      sm.gam[lane] = gam;
      sm.beta[lane] = bv;
      sm.eg[lane] = __expf(gam);
      sm.el[lane] = __expf(glast - gam);
      if (lane == 0) sm.misc[0] = glast;
      if (DUMP && a.dbg_gamma && lane < n) a.dbg_gamma[(t0 + lane) * H + h] = gam;
    }
    __syncthreads();
    if (a.l2norm) {  // q/k L2 normalisation of the staged tiles
      normalize_rows<D, LDE>(sm.k, tid);
      if (emit) normalize_rows<D, LDE>(sm.q, tid);
      __syncthreads();
    }

    // ---- K K^T -> A (row a2) and Q K^T (kept in registers until A is consumed)
    f32x4 qk[3];
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      const int tau = wave + 4 * s;
      qk[s] = zero4();
      if (tau >= 10) continue;
      const int bi = tile_bi(tau), bj = tile_bj(tau);
      f32x4 acck = zero4(), accq = zero4();
      if constexpr (BF16) {
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
          const bf16x8 kb = lds_bf16x8(&sm.k[(16 * bj + cl) * LDE + 32 * ks + 8 * gq]);
          const bf16x8 ka = lds_bf16x8(&sm.k[(16 * bi + cl) * LDE + 32 * ks + 8 * gq]);
          acck = mma_bf16(ka, kb, acck);
          if (emit) {
            const bf16x8 qa = lds_bf16x8(&sm.q[(16 * bi + cl) * LDE + 32 * ks + 8 * gq]);
            accq = mma_bf16(qa, kb, accq);
          }
        }
      } else {
#pragma unroll 8
        for (int s4 = 0; s4 < D / 4; ++s4) {
          const float kb = sm.k[(16 * bj + cl) * LDE + 4 * s4 + gq];
          const float ka = sm.k[(16 * bi + cl) * LDE + 4 * s4 + gq];
          acck = mma_f32(ka, kb, acck);
          if (emit) accq = mma_f32(sm.q[(16 * bi + cl) * LDE + 4 * s4 + gq], kb, accq);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * bi + 4 * gq + i, j = 16 * bj + cl;
        float val = 0.f;
        if (j < r) val = sm.beta[r] * __expf(sm.gam[r] - sm.gam[j]) * acck[i];
        sm.ap[r * LDT + j] = val;
      }
      qk[s] = accq;
    }
    __syncthreads();

    // ---- Tm = (I + A)^-1 (row a3): diagonal 16x16 blocks by forward substitution, one column
    //      per lane; then the blocks below the diagonal, one block diagonal at a time.
    if (wave == 0) {
      const int b = lane >> 4, j = lane & 15;
      const float *Ab = &sm.ap[(16 * b) * LDT + 16 * b];
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) acc += Ab[r * LDT + i] * x[i];
        x[r] = (r < j) ? 0.f : ((r == j) ? 1.f : -acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.t[(16 * b + r) * LDT + 16 * b + j] = x[r];
    }
    __syncthreads();
#pragma unroll
    for (int d = 1; d <= 3; ++d) {
      if (wave < 4 - d) solve_offdiag_block<LDT>(sm.t, sm.ap, wave + d, wave, gq, cl);
      __syncthreads();
    }
    if (DUMP && a.dbg_tmat) {
      float *dst = a.dbg_tmat + (cglob * H + h) * 64 * 64;
      for (int i = tid; i < 64 * 64; i += 256) {
        const int r = i >> 6, cc = i & 63;
        dst[i] = (r < n && cc < n) ? sm.t[r * LDT + cc] : 0.f;
      }
    }

    // ---- P = (Q K^T) o exp(gamma_r - gamma_i) o [i <= r]  (A is no longer needed)
    if (emit) {
#pragma unroll
      for (int s = 0; s < 3; ++s) {
        const int tau = wave + 4 * s;
        if (tau >= 10) continue;
        const int bi = tile_bi(tau), bj = tile_bj(tau);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * bi + 4 * gq + i, j = 16 * bj + cl;
          float val = 0.f;
          if (j <= r) val = __expf(sm.gam[r] - sm.gam[j]) * qk[s][i];
          sm.ap[r * LDT + j] = val;
        }
      }
    }

    // ---- WY form (row a4): U = Tm diag(beta) V (this wave's columns, kept in registers) and
    //      W = Tm diag(beta e^gamma) K (this wave's columns, then shared through LDS)
    f32x4 U[4][NT], Wr[4][NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n0 = ncol0 + 16 * nt;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 au = zero4(), aw = zero4();
        if constexpr (BF16) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            if (32 * ks > 16 * mt + 15) continue;  // Tm is lower triangular
            const float *tp = &sm.t[(16 * mt + cl) * LDT + 32 * ks + 8 * gq];
            const f32x4 t0v = lds_f32x4(tp), t1v = lds_f32x4(tp + 4);
            const f32x4 b0 = lds_f32x4(&sm.beta[32 * ks + 8 * gq]);
            const f32x4 b1 = lds_f32x4(&sm.beta[32 * ks + 8 * gq + 4]);
            const f32x4 e0 = lds_f32x4(&sm.eg[32 * ks + 8 * gq]);
            const f32x4 e1 = lds_f32x4(&sm.eg[32 * ks + 8 * gq + 4]);
            const f32x4 tb0 = t0v * b0, tb1 = t1v * b1;
            const bf16x8 tu = to_bf16x8(tb0, tb1);
            const bf16x8 tw = to_bf16x8(tb0 * e0, tb1 * e1);
            const int rr = 32 * ks + 8 * gq + (cl >> 2), cc = n0 + 4 * (cl & 3);
            const bf16x8 vf = cat8(lds_tr16(&sm.vw[rr * LDE + cc]),
                                   lds_tr16(&sm.vw[(rr + 4) * LDE + cc]));
            const bf16x8 kf = cat8(lds_tr16(&sm.k[rr * LDE + cc]),
                                   lds_tr16(&sm.k[(rr + 4) * LDE + cc]));
            au = mma_bf16(tu, vf, au);
            aw = mma_bf16(tw, kf, aw);
          }
        } else {
#pragma unroll
          for (int s4 = 0; s4 < 16; ++s4) {
            if (4 * s4 > 16 * mt + 15) continue;
            const float tv = sm.t[(16 * mt + cl) * LDT + 4 * s4 + gq];
            const float tb = tv * sm.beta[4 * s4 + gq];
            const float vv = sm.vw[(4 * s4 + gq) * LDE + n0 + cl];
            const float kk = sm.k[(4 * s4 + gq) * LDE + n0 + cl];
            au = mma_f32(tb, vv, au);
            aw = mma_f32(tb * sm.eg[4 * s4 + gq], kk, aw);
          }
        }
        U[mt][nt] = au;
        Wr[mt][nt] = aw;
      }
    }
    __syncthreads();  // every wave is done reading V
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sm.vw[(16 * mt + 4 * gq + i) * LDE + ncol0 + 16 * nt + cl] = from_f32<E>(Wr[mt][nt][i]);
    if (DUMP) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * mt + 4 * gq + i, col = ncol0 + 16 * nt + cl;
            const int64_t off = ((cglob * H + h) * 64 + r) * D + col;
            if (a.dbg_w) a.dbg_w[off] = r < n ? Wr[mt][nt][i] : 0.f;
            if (a.dbg_u) a.dbg_u[off] = r < n ? U[mt][nt][i] : 0.f;
          }
      if (a.dbg_hc) {
        float *dst = a.dbg_hc + (cglob * H + h) * D * D;
#pragma unroll
        for (int mt = 0; mt < MTD; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              dst[(16 * mt + 4 * gq + i) * D + ncol0 + 16 * nt + cl] = S[mt][nt][i];
      }
    }
    __syncthreads();  // W is complete in LDS

    // ---- chain (row a5, first half): Delta = U - W h;  and Q h for the output
    f32x4 Dl[4][NT], QS[4][NT];
    if constexpr (BF16) {
      bf16x8 sb[D / 32][NT];
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sb[ks][nt] = to_bf16x8(S[2 * ks][nt], S[2 * ks + 1][nt]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          f32x4 accw = zero4(), accq = zero4();
#pragma unroll
          for (int ks = 0; ks < D / 32; ++ks) {
            const bf16 *wp = &sm.vw[(16 * mt + cl) * LDE + 32 * ks + 4 * gq];
            accw = mma_bf16(cat8(lds_bf16x4(wp), lds_bf16x4(wp + 16)), sb[ks][nt], accw);
            if (emit) {
              const bf16 *qp = &sm.q[(16 * mt + cl) * LDE + 32 * ks + 4 * gq];
              accq = mma_bf16(cat8(lds_bf16x4(qp), lds_bf16x4(qp + 16)), sb[ks][nt], accq);
            }
          }
          Dl[mt][nt] = U[mt][nt] - accw;
          QS[mt][nt] = accq;
        }
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          f32x4 accw = zero4(), accq = zero4();
#pragma unroll
          for (int kt = 0; kt < MTD; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int col = 16 * kt + 4 * gq + i;
              accw = mma_f32(sm.vw[(16 * mt + cl) * LDE + col], S[kt][nt][i], accw);
              if (emit) accq = mma_f32(sm.q[(16 * mt + cl) * LDE + col], S[kt][nt][i], accq);
            }
          Dl[mt][nt] = U[mt][nt] - accw;
          QS[mt][nt] = accq;
        }
      }
    }
    if (DUMP && a.dbg_delta) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 16 * mt + 4 * gq + i;
            if (r < n) a.dbg_delta[((t0 + r) * H + h) * D + ncol0 + 16 * nt + cl] = Dl[mt][nt][i];
          }
    }

    // ---- output (row a6): O = diag(e^gamma) Q h + P Delta
    if (emit) {
      f32x4 O[4][NT];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 egr = lds_f32x4(&sm.eg[16 * mt + 4 * gq]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          f32x4 acc = egr * QS[mt][nt];
          if constexpr (BF16) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
              if (32 * ks > 16 * mt + 15) continue;  // P is lower triangular
              const float *pp = &sm.ap[(16 * mt + cl) * LDT + 32 * ks + 4 * gq];
              const bf16x8 pa = to_bf16x8(lds_f32x4(pp), lds_f32x4(pp + 16));
              const bf16x8 db = to_bf16x8(Dl[2 * ks][nt], Dl[2 * ks + 1][nt]);
              acc = mma_bf16(pa, db, acc);
            }
          } else {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
              if (kt > mt) continue;
#pragma unroll
              for (int i = 0; i < 4; ++i)
                acc = mma_f32(sm.ap[(16 * mt + cl) * LDT + 16 * kt + 4 * gq + i], Dl[kt][nt][i],
                              acc);
            }
          }
          O[mt][nt] = acc * a.scale;
        }
      }
      __syncthreads();  // every wave is done reading Q
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sm.q[(16 * mt + 4 * gq + i) * LDE + ncol0 + 16 * nt + cl] = from_f32<E>(O[mt][nt][i]);
      __syncthreads();
      store_tile<E, D, LDE>(go_, sm.q, t0, n, h, H, tid);
    }

    // ---- chain (row a5, second half): h <- e^{gamma_last} h + K^T diag(e^{gamma_last-gamma}) Delta
    const float egl = __expf(sm.misc[0]);
    if constexpr (BF16) {
      bf16x8 db2[2][NT];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const f32x4 e0 = lds_f32x4(&sm.el[32 * ks + 4 * gq]);
        const f32x4 e1 = lds_f32x4(&sm.el[32 * ks + 16 + 4 * gq]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          db2[ks][nt] = to_bf16x8(Dl[2 * ks][nt] * e0, Dl[2 * ks + 1][nt] * e1);
      }
#pragma unroll
      for (int mt = 0; mt < MTD; ++mt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          f32x4 acc = S[mt][nt] * egl;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const int rr = 32 * ks + 4 * gq + (cl >> 2), cc = 16 * mt + 4 * (cl & 3);
            const bf16x8 ka = cat8(lds_tr16(&sm.k[rr * LDE + cc]),
                                   lds_tr16(&sm.k[(rr + 16) * LDE + cc]));
            acc = mma_bf16(ka, db2[ks][nt], acc);
          }
          S[mt][nt] = acc;
        }
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < MTD; ++mt) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          f32x4 acc = S[mt][nt] * egl;
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 16 * kt + 4 * gq + i;
              acc = mma_f32(sm.k[r * LDE + 16 * mt + cl], Dl[kt][nt][i] * sm.el[r], acc);
            }
          S[mt][nt] = acc;
        }
      }
    }
  }

  if (a.ht != nullptr && c1 == nchunks_seq) {
    float *dst = a.ht + ((int64_t)seq * H + h) * D * D;
#pragma unroll
    for (int mt = 0; mt < MTD; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[(16 * mt + 4 * gq + i) * D + ncol0 + 16 * nt + cl] = S[mt][nt][i];
  }
}

template <int D, bool BF16, bool DUMP>
static hipError_t launch_fwd_t(const FwdArgs &a, int64_t max_units, hipStream_t stream) {
  if (max_units <= 0) return hipSuccess;
  hipLaunchKernelGGL((fwd_kernel<D, BF16, DUMP>), dim3((unsigned)max_units, a.H), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

int fwd_blocks_per_cu(int D, bool bf16) {
  int blocks = 0;
  hipError_t e;
  if (D == 128)
    e = bf16 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fwd_kernel<128, true, false>, 256, 0)
             : hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fwd_kernel<128, false, false>, 256, 0);
  else
    e = bf16 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fwd_kernel<64, true, false>, 256, 0)
             : hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fwd_kernel<64, false, false>, 256, 0);
  return (e == hipSuccess && blocks > 0) ? blocks : 1;
}

hipError_t launch_fwd(const FwdArgs &a, int D, bool bf16, bool dump, int64_t max_units,
                      hipStream_t stream) {
  if (D == 128) {
    if (bf16) return dump ? launch_fwd_t<128, true, true>(a, max_units, stream)
                          : launch_fwd_t<128, true, false>(a, max_units, stream);
    return dump ? launch_fwd_t<128, false, true>(a, max_units, stream)
                : launch_fwd_t<128, false, false>(a, max_units, stream);
  }
  if (bf16) return dump ? launch_fwd_t<64, true, true>(a, max_units, stream)
                        : launch_fwd_t<64, true, false>(a, max_units, stream);
  return dump ? launch_fwd_t<64, false, true>(a, max_units, stream)
              : launch_fwd_t<64, false, false>(a, max_units, stream);
}

}  // namespace gdn
