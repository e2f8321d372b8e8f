// Backward of the chunked gated delta rule on gfx950.
//
// Method: the hidden states are recomputed, not stored ("How to Speed Up GDN Kernels for Qwen
// Models", section "Lever 2"): a forward pass (the forward kernel with its per-chunk
// intermediates written out) gives, per chunk, gamma, Tm = (I + A)^-1, W, the chunk-start state
// h and Delta.  Then, per chunk (n tokens, a = e^gamma, c = e^{gamma_last - gamma},
// lambda = e^{gamma_last}, Gm_ri = e^{gamma_r - gamma_i} for i <= r, dO scaled by `scale`):
//
//   reverse state chain (sequential over chunks, dh' = gradient of the state after the chunk):
//     dDelta = P^T dO + diag(c) K dh',  P = (Q K^T) o Gm
//     dh     = lambda dh' + Q^T diag(a) dO - W^T dDelta          (dh0 = dh of the first chunk)
//   local gradients (all chunks in parallel):
//     dP = dO Delta^T;  dPm = dP o Gm;  dW = -dDelta h^T;  Y1 = dO h^T;  Y2 = Delta dh'^T
//     dT = dDelta (diag(beta) V)^T + dW (diag(beta a) K)^T;  dA = strict_lower(-Tm^T dT Tm^T)
//     E  = dA o Gm o beta_row
//     dQ = diag(a) Y1 + dPm K
//     dK = dPm^T Q + diag(c) Y2 + diag(beta a) Tm^T dW + E K + E^T K
//     dV = diag(beta) Tm^T dDelta
//     dbeta_r  = (Tm^T dDelta . V)_r + a_r (Tm^T dW . K)_r + sum_i dA_ri Gm_ri (k_r . k_i)
//     dgamma_r = a_r (Y1 . Q)_r + beta_r a_r (Tm^T dW . K)_r - c_r (Y2 . K)_r
//                + rowsum_r - colsum_r of (dPm o Q K^T) and of (dA o A)
//     dgamma_last += sum_r c_r (Y2 . K)_r + lambda <dh', h>;   dg = reverse cumsum of dgamma
// (x . y)_r is the dot product of row r of x and y.  This is the reverse-mode derivative of the
// chunked form, which equals the derivative of the token recurrence.
//
// Both kernels use fp32 MFMA (v_mfma_f32_16x16x4_f32) on fp32 LDS tiles.  Every reduction has a
// fixed owner and order, so results are bitwise reproducible.  They serve fp32 inputs and d = 64;
// bf16 inputs with d = 128 run the bf16-MFMA kernels of gdn_bwd_chain.hip and gdn_bwd_grad.hip.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_unit.h"

namespace gdn {


namespace {

constexpr int LDF = 64 + 4;  // row stride of 64-wide fp32 LDS tiles

// One 16x16 output tile of A B with fp32 MFMA, K a multiple of 4.  A[m][k] is read at
// A + m * ars + k * acs and B[k][n] at B + k * brs + n * bcs (fp32 LDS), so transposed operands
// cost nothing.  Lane (gq, cl) receives rows 4 gq + i, column cl.
__device__ __forceinline__ f32x4 tile_mma(const float *A, int ars, int acs, const float *B,
                                          int brs, int bcs, int K, int gq, int cl, f32x4 acc) {
  const float *a = A + cl * ars + gq * acs;
  const float *b = B + gq * brs + cl * bcs;
#pragma unroll 4
  for (int k = 0; k < K; k += 4) acc = mma_f32(a[k * acs], b[k * brs], acc);
  return acc;
}

// Rows [0, 64) x columns [c0, c0 + 64) of a token-major [T, H, D] tensor times `mul`, rows past
// n zero, into a 64 x LDF fp32 LDS tile.
template <class E>
__device__ __forceinline__ void load_rows64(float *dst, const E *src, int64_t t0, int n, int h,
                                            int H, int D, int c0, float mul, int tid,
                                            const float *rs = nullptr) {
  // rs (optional): per-row factors [T, H] (the q/k L2 normalisation's inverse norms)
  for (int i = tid; i < 64 * 64; i += 256) {
    const int r = i >> 6, c = i & 63;
    const float x = r < n ? to_f32(src[((t0 + r) * H + h) * D + c0 + c]) : 0.f;
    // normalised rows are rounded to the input dtype, as the forward kernels use them
    dst[r * LDF + c] = rs != nullptr && r < n ? mul * to_f32(from_f32<E>(rs[(t0 + r) * H + h] * x))
                                              : mul * x;
  }
}

// A 64 x 64 block of a row-major fp32 matrix (leading dimension ld) into an LDS tile.
__device__ __forceinline__ void load_block64(float *dst, const float *src, int ld, int tid) {
  for (int i = tid; i < 64 * 64; i += 256) {
    const int r = i >> 6, c = i & 63;
    dst[r * LDF + c] = src[(int64_t)r * ld + c];
  }
}

}  // namespace

// ------------------------------------------------------------------------- reverse chain
// One workgroup per (sequence, head); wave w keeps columns [w D/4, (w+1) D/4) of the state
// gradient in MFMA accumulator registers and walks the sequence's chunks backwards.
template <int D>
struct ChainSmem {
  static constexpr int LD = D + 4;
  alignas(16) float q[64 * LD];
  alignas(16) float k[64 * LD];
  alignas(16) float dout[64 * LD];
  alignas(16) float w[64 * LD];
  alignas(16) float p[64 * LDF];
  alignas(16) float gam[64];
  alignas(16) float a[64];
  alignas(16) float c[64];
  alignas(16) int imisc[4];
};

template <int D, class E>
__global__ __launch_bounds__(256) void bwd_chain_kernel(BwdArgs b) {
  using SM = ChainSmem<D>;
  constexpr int LD = SM::LD;
  constexpr int NT = D / 64, MTD = D / 16;
  __shared__ SM sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, gq = lane >> 4, cl = lane & 15;
  const int seq = blockIdx.x, h = blockIdx.y, H = b.H, hk = h / (H / b.HK);
  if (wave == 0) {
    Unit un;
    const bool ok = find_unit(b.cu, b.N, b.T, 0, seq, true, lane, un);
    if (lane == 0) {
      sm.imisc[0] = ok ? (int)un.chunk_base : -1;
      sm.imisc[1] = un.c1;
    }
  }
  __syncthreads();
  if (sm.imisc[0] < 0) return;
  const int64_t chunk_base = sm.imisc[0];
  const int nch = sm.imisc[1];
  const int64_t ts0 = b.cu[seq], ts1 = b.cu[seq + 1];
  if (ts0 < 0 || ts1 < ts0 || ts1 > b.T) return;
  const E *gq_ = static_cast<const E *>(b.q);
  const E *gk_ = static_cast<const E *>(b.k);
  const E *gdo = static_cast<const E *>(b.dout);
  const int ncol0 = wave * (D / 4);

  f32x4 G[MTD][NT];  // dh' of the current chunk: starts at dht (or zero)
#pragma unroll
  for (int mt = 0; mt < MTD; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        G[mt][nt][i] = b.dht ? b.dht[(((int64_t)seq * H + h) * D + 16 * mt + 4 * gq + i) * D +
                                     ncol0 + 16 * nt + cl]
                             : 0.f;

  for (int c = nch - 1; c >= 0; --c) {
    const int64_t t0 = ts0 + (int64_t)c * kChunk;
    const int n = (int)min<int64_t>(kChunk, ts1 - t0);
    const int64_t cg = chunk_base + c;
    __syncthreads();  // the previous chunk is done with LDS
    for (int i = tid; i < 64 * D; i += 256) {
      const int r = i / D, col = i % D;
      const bool ok = r < n;
      const int64_t gi = ((t0 + r) * H + h) * D + col;
      const int64_t gik = ((t0 + r) * b.HK + hk) * D + col;  // q and k: the key head
      const int64_t rk_i = (t0 + r) * b.HK + hk;  // q/k L2 normalisation: the rows' factors
      // normalised rows are rounded to the input dtype, as the forward kernels use them
      sm.q[r * LD + col] = !ok ? 0.f : b.rq ? to_f32(from_f32<E>(b.rq[rk_i] * to_f32(gq_[gik])))
                                            : to_f32(gq_[gik]);
      sm.k[r * LD + col] = !ok ? 0.f : b.rk ? to_f32(from_f32<E>(b.rk[rk_i] * to_f32(gk_[gik])))
                                            : to_f32(gk_[gik]);
      sm.dout[r * LD + col] = ok ? b.scale * to_f32(gdo[gi]) : 0.f;
      sm.w[r * LD + col] = b.w[((cg * H + h) * 64 + r) * D + col];
    }
    if (wave == 0) {
      const float gam = lane < n ? b.gamma[(t0 + lane) * H + h] : 0.f;
      const float glast = __shfl(gam, n - 1, 64);
      sm.gam[lane] = lane < n ? gam : glast;
      sm.a[lane] = lane < n ? __expf(gam) : 0.f;
      sm.c[lane] = lane < n ? __expf(glast - gam) : 0.f;
    }
    __syncthreads();
    // P = (Q K^T) o Gm, lower triangle including the diagonal
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int bi = s, bj = wave;
      f32x4 acc = zero4();
      if (bj <= bi)
        acc = tile_mma(&sm.q[16 * bi * LD], LD, 1, &sm.k[16 * bj * LD], 1, LD, D, gq, cl, acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * bi + 4 * gq + i, j = 16 * bj + cl;
        sm.p[r * LDF + j] = (j <= r) ? __expf(sm.gam[r] - sm.gam[j]) * acc[i] : 0.f;
      }
    }
    __syncthreads();
    const float lam = __expf(sm.gam[63]);
    // the state gradient after this chunk, for the per-chunk gradient kernel
#pragma unroll
    for (int mt = 0; mt < MTD; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          b.dhn[((cg * H + h) * D + 16 * mt + 4 * gq + i) * D + ncol0 + 16 * nt + cl] =
              G[mt][nt][i];
    // dDelta = P^T dO + diag(c) K dh'
    f32x4 dD[4][NT];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int n0 = ncol0 + 16 * nt;
        f32x4 kd = zero4();
#pragma unroll
        for (int kt = 0; kt < MTD; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            kd = mma_f32(sm.k[(16 * mt + cl) * LD + 16 * kt + 4 * gq + i], G[kt][nt][i], kd);
        f32x4 acc = tile_mma(&sm.p[16 * mt], 1, LDF, &sm.dout[n0], LD, 1, 64, gq, cl, zero4());
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * mt + 4 * gq + i;
          acc[i] += sm.c[r] * kd[i];
          if (r < n) b.ddelta[((t0 + r) * H + h) * D + n0 + cl] = acc[i];
        }
        dD[mt][nt] = acc;
      }
    // dh = lambda dh' + Q^T diag(a) dO - W^T dDelta
#pragma unroll
    for (int mt = 0; mt < MTD; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int n0 = ncol0 + 16 * nt;
        f32x4 acc = G[mt][nt] * lam;
#pragma unroll 4
        for (int s = 0; s < 16; ++s) {
          const int r = 4 * s + gq;
          acc = mma_f32(sm.q[r * LD + 16 * mt + cl], sm.a[r] * sm.dout[r * LD + n0 + cl], acc);
        }
        f32x4 acc2 = zero4();
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc2 = mma_f32(sm.w[(16 * kt + 4 * gq + i) * LD + 16 * mt + cl], dD[kt][nt][i], acc2);
        G[mt][nt] = acc - acc2;
      }
  }
  if (b.dh0_seq != nullptr) {
    float *dst = b.dh0_seq + ((int64_t)seq * H + h) * D * D;
#pragma unroll
    for (int mt = 0; mt < MTD; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[(16 * mt + 4 * gq + i) * D + ncol0 + 16 * nt + cl] = G[mt][nt][i];
  }
}

// ------------------------------------------------------------------------- local gradients
// One workgroup per (chunk, head).  Matrices are held as 64 x 64 fp32 LDS tiles; D is
// processed in 64-column blocks.  Wave w owns the 16-column strip w of every 64 x 64 result
// (rows 0..63), so each row total is the sum of four per-wave partials in wave order and each
// column total has one owner.
struct GradSmem {
  alignas(16) float tm[64 * LDF];  // Tm
  alignas(16) float dp[64 * LDF];  // dP, then dPm = dP o Gm
  alignas(16) float qk[64 * LDF];  // Q K^T, then an operand tile
  alignas(16) float kk[64 * LDF];  // K K^T, then an operand tile
  alignas(16) float dt[64 * LDF];  // dT, then Tm^T dT, then E
  alignas(16) float x0[64 * LDF];  // operand tiles
  alignas(16) float x1[64 * LDF];
  alignas(16) float gam[64], a[64], c[64], beta[64];
  alignas(16) float rg[4][64];  // per-wave partial row terms of dgamma
  alignas(16) float rb[4][64];  // per-wave partial row terms of dbeta
  alignas(16) float rc[4][64];  // per-wave partial c_r (Y2 . K)_r
  alignas(16) float colg[64];   // column terms of dgamma (subtracted)
  alignas(16) float red[4];
  alignas(16) int imisc[4];
};

template <int D, class E>
__global__ __launch_bounds__(256) void bwd_grad_kernel(BwdArgs b) {
  constexpr int NB = D / 64;  // 64-column blocks
  __shared__ GradSmem sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, gq = lane >> 4, cl = lane & 15;
  const int cg = blockIdx.x, h = blockIdx.y, H = b.H, hk = h / (H / b.HK);
  // locate the chunk: its sequence and its index within that sequence
  if (wave == 0) {
    int64_t before = 0;
    int seq = -1, cidx = 0;
    for (int base = 0; base < b.N; base += 64) {
      const int nn = base + lane;
      const int ch = nn < b.N ? max(0, (b.cu[nn + 1] - b.cu[nn] + kChunk - 1) / kChunk) : 0;
      int sc = ch;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(sc, off, 64);
        if (lane >= off) sc += y;
      }
      const uint64_t hit = __ballot(nn < b.N && before + sc > cg);
      if (hit) {
        const int l = __builtin_ctzll(hit);
        seq = base + l;
        cidx = (int)(cg - before - __shfl(sc - ch, l, 64));
        break;
      }
      before += __shfl(sc, 63, 64);
    }
    if (lane == 0) {
      sm.imisc[0] = seq;
      sm.imisc[1] = cidx;
    }
  }
  __syncthreads();
  const int seq = sm.imisc[0];
  if (seq < 0) return;
  const int64_t ts0 = b.cu[seq], ts1 = b.cu[seq + 1];
  if (ts0 < 0 || ts1 < ts0 || ts1 > b.T) return;
  const int64_t t0 = ts0 + (int64_t)sm.imisc[1] * kChunk;
  const int n = (int)min<int64_t>(kChunk, ts1 - t0);
  const E *gq_ = static_cast<const E *>(b.q);
  const E *gk_ = static_cast<const E *>(b.k);
  const E *gv_ = static_cast<const E *>(b.v);
  const E *gdo = static_cast<const E *>(b.dout);
  const E *gb_ = static_cast<const E *>(b.beta);
  const float *hS = b.hc + ((int64_t)cg * H + h) * D * D;
  const float *dhn = b.dhn + ((int64_t)cg * H + h) * D * D;
  const float dsc = b.scale;
  const int bj = wave;  // this wave's column strip

  if (wave == 0) {
    const float gam = lane < n ? b.gamma[(t0 + lane) * H + h] : 0.f;
    const float glast = __shfl(gam, n - 1, 64);
    sm.gam[lane] = lane < n ? gam : glast;
    sm.a[lane] = lane < n ? __expf(gam) : 0.f;
    sm.c[lane] = lane < n ? __expf(glast - gam) : 0.f;
    sm.beta[lane] = lane < n ? to_f32(gb_[(t0 + lane) * H + h]) : 0.f;
  }
  load_block64(sm.tm, b.tmat + ((int64_t)cg * H + h) * 64 * 64, 64, tid);

  // ---- stage 1: dP = dO Delta^T, QK = Q K^T, KK = K K^T, X = dDelta (diag(beta) V)^T
  f32x4 acc_dp[4], acc_qk[4], acc_kk[4], acc_x[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) acc_dp[s] = acc_qk[s] = acc_kk[s] = acc_x[s] = zero4();
  for (int cb = 0; cb < NB; ++cb) {
    __syncthreads();
    load_rows64(sm.x0, gdo, t0, n, h, H, D, 64 * cb, dsc, tid);
    load_rows64(sm.x1, b.delta, t0, n, h, H, D, 64 * cb, 1.f, tid);
    load_rows64(sm.qk, gq_, t0, n, hk, b.HK, D, 64 * cb, 1.f, tid, b.rq);
    load_rows64(sm.kk, gk_, t0, n, hk, b.HK, D, 64 * cb, 1.f, tid, b.rk);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      acc_dp[s] = tile_mma(&sm.x0[16 * s * LDF], LDF, 1, &sm.x1[16 * bj * LDF], 1, LDF, 64, gq, cl,
                           acc_dp[s]);
      acc_qk[s] = tile_mma(&sm.qk[16 * s * LDF], LDF, 1, &sm.kk[16 * bj * LDF], 1, LDF, 64, gq, cl,
                           acc_qk[s]);
      acc_kk[s] = tile_mma(&sm.kk[16 * s * LDF], LDF, 1, &sm.kk[16 * bj * LDF], 1, LDF, 64, gq, cl,
                           acc_kk[s]);
    }
    __syncthreads();
    load_rows64(sm.x0, b.ddelta, t0, n, h, H, D, 64 * cb, 1.f, tid);
    load_rows64(sm.x1, gv_, t0, n, h, H, D, 64 * cb, 1.f, tid);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // X[r][i] = sum_d dDelta[r][d] beta_i V[i][d]: beta_i scales the output column
      f32x4 t = tile_mma(&sm.x0[16 * s * LDF], LDF, 1, &sm.x1[16 * bj * LDF], 1, LDF, 64, gq, cl,
                         zero4());
      acc_x[s] += t * sm.beta[16 * bj + cl];
    }
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * s + 4 * gq + i, j = 16 * bj + cl;
      sm.dp[r * LDF + j] = acc_dp[s][i];
      sm.qk[r * LDF + j] = acc_qk[s][i];
      sm.kk[r * LDF + j] = acc_kk[s][i];
      sm.dt[r * LDF + j] = acc_x[s][i];
    }

  // ---- stage 2: dT += dW (diag(beta a) K)^T with dW = -dDelta h^T, column block kb at a time
  f32x4 acc_t[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) acc_t[s] = zero4();
  for (int kb = 0; kb < NB; ++kb) {
    f32x4 dw[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) dw[s] = zero4();
    for (int vb = 0; vb < NB; ++vb) {
      __syncthreads();
      load_rows64(sm.x0, b.ddelta, t0, n, h, H, D, 64 * vb, 1.f, tid);
      load_block64(sm.x1, hS + (int64_t)(64 * kb) * D + 64 * vb, D, tid);  // h[kb rows][vb cols]
      __syncthreads();
#pragma unroll
      for (int s = 0; s < 4; ++s)  // dW[r][d] = -sum_j dDelta[r][j] h[d][j]
        dw[s] = tile_mma(&sm.x0[16 * s * LDF], LDF, 1, &sm.x1[16 * bj * LDF], 1, LDF, 64, gq, cl,
                         dw[s]);
    }
    __syncthreads();
    load_rows64(sm.x1, gk_, t0, n, hk, b.HK, D, 64 * kb, 1.f, tid, b.rk);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.x0[(16 * s + 4 * gq + i) * LDF + 16 * bj + cl] = -dw[s][i];
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // dT[r][i] += sum_d dW[r][d] beta_i a_i K[i][d]
      f32x4 t = tile_mma(&sm.x0[16 * s * LDF], LDF, 1, &sm.x1[16 * bj * LDF], 1, LDF, 64, gq, cl,
                         zero4());
      acc_t[s] += t * (sm.beta[16 * bj + cl] * sm.a[16 * bj + cl]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.dt[(16 * s + 4 * gq + i) * LDF + 16 * bj + cl] += acc_t[s][i];
  __syncthreads();

  // ---- stage 3: dA = strict_lower(-Tm^T dT Tm^T), E = dA o Gm o beta_row, dPm = dP o Gm and
  //      the row / column terms of dgamma and dbeta that come from A and P
  f32x4 y[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)  // Y[r][j] = sum_i Tm[i][r] dT[i][j]
    y[s] = tile_mma(&sm.tm[16 * s], 1, LDF, &sm.dt[16 * bj], LDF, 1, 64, gq, cl, zero4());
  __syncthreads();
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.dt[(16 * s + 4 * gq + i) * LDF + 16 * bj + cl] = y[s][i];
  __syncthreads();
#pragma unroll
  for (int s = 0; s < 4; ++s)  // Z[r][j] = sum_i Y[r][i] Tm[j][i];  dA = -Z below the diagonal
    y[s] = tile_mma(&sm.dt[16 * s * LDF], LDF, 1, &sm.tm[16 * bj * LDF], 1, LDF, 64, gq, cl,
                    zero4());
  __syncthreads();
  float colsum = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    float rg[4], rb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * s + 4 * gq + i, j = 16 * bj + cl;
      float e = 0.f, pm = 0.f, tg = 0.f, tb = 0.f;
      if (j <= r) {
        const float gm = __expf(sm.gam[r] - sm.gam[j]);
        if (j < r) {
          const float da = -y[s][i];
          const float gk = gm * sm.kk[r * LDF + j];
          e = da * gm * sm.beta[r];
          tb = da * gk;
          tg = da * sm.beta[r] * gk;
        }
        pm = sm.dp[r * LDF + j] * gm;
        tg += pm * sm.qk[r * LDF + j];
      }
      sm.dt[r * LDF + j] = e;
      sm.dp[r * LDF + j] = pm;
      rg[i] = tg;
      rb[i] = tb;
      colsum += tg;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) {
        rg[i] += __shfl_xor(rg[i], off, 64);
        rb[i] += __shfl_xor(rb[i], off, 64);
      }
      if (cl == 0) {
        sm.rg[wave][16 * s + 4 * gq + i] = rg[i];
        sm.rb[wave][16 * s + 4 * gq + i] = rb[i];
      }
    }
  }
  colsum += __shfl_xor(colsum, 16, 64);
  colsum += __shfl_xor(colsum, 32, 64);
  if (gq == 0) sm.colg[16 * bj + cl] = colsum;
  __syncthreads();

  // ---- stage 4: per output column block kb: dQ, dK, dV and the remaining row terms
  float prg[4][4], prb[4][4], prc[4][4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) prg[s][i] = prb[s][i] = prc[s][i] = 0.f;
  for (int kb = 0; kb < NB; ++kb) {
    f32x4 y1[4], y2[4], dw[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) y1[s] = y2[s] = dw[s] = zero4();
    for (int vb = 0; vb < NB; ++vb) {
      __syncthreads();
      load_rows64(sm.x0, gdo, t0, n, h, H, D, 64 * vb, dsc, tid);
      load_rows64(sm.x1, b.delta, t0, n, h, H, D, 64 * vb, 1.f, tid);
      load_block64(sm.qk, hS + (int64_t)(64 * kb) * D + 64 * vb, D, tid);
      load_block64(sm.kk, dhn + (int64_t)(64 * kb) * D + 64 * vb, D, tid);
      __syncthreads();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        y1[s] = tile_mma(&sm.x0[16 * s * LDF], LDF, 1, &sm.qk[16 * bj * LDF], 1, LDF, 64, gq, cl,
                         y1[s]);
        y2[s] = tile_mma(&sm.x1[16 * s * LDF], LDF, 1, &sm.kk[16 * bj * LDF], 1, LDF, 64, gq, cl,
                         y2[s]);
      }
      __syncthreads();
      load_rows64(sm.x0, b.ddelta, t0, n, h, H, D, 64 * vb, 1.f, tid);
      __syncthreads();
#pragma unroll
      for (int s = 0; s < 4; ++s)
        dw[s] = tile_mma(&sm.x0[16 * s * LDF], LDF, 1, &sm.qk[16 * bj * LDF], 1, LDF, 64, gq, cl,
                         dw[s]);
    }
    __syncthreads();
    // operand tiles of this block: x0 = Q, x1 = K, qk = dW, kk = dDelta
    load_rows64(sm.x0, gq_, t0, n, hk, b.HK, D, 64 * kb, 1.f, tid, b.rq);
    load_rows64(sm.x1, gk_, t0, n, hk, b.HK, D, 64 * kb, 1.f, tid, b.rk);
    load_rows64(sm.kk, b.ddelta, t0, n, h, H, D, 64 * kb, 1.f, tid);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.qk[(16 * s + 4 * gq + i) * LDF + 16 * bj + cl] = -dw[s][i];
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const f32x4 pk = tile_mma(&sm.dp[16 * s * LDF], LDF, 1, &sm.x1[16 * bj], LDF, 1, 64, gq, cl,
                                zero4());  // dPm K
      const f32x4 tdw = tile_mma(&sm.tm[16 * s], 1, LDF, &sm.qk[16 * bj], LDF, 1, 64, gq, cl,
                                 zero4());  // Tm^T dW
      const f32x4 tdu = tile_mma(&sm.tm[16 * s], 1, LDF, &sm.kk[16 * bj], LDF, 1, 64, gq, cl,
                                 zero4());  // Tm^T dDelta
      f32x4 dk = tile_mma(&sm.dp[16 * s], 1, LDF, &sm.x0[16 * bj], LDF, 1, 64, gq, cl,
                          zero4());  // dPm^T Q
      dk = tile_mma(&sm.dt[16 * s * LDF], LDF, 1, &sm.x1[16 * bj], LDF, 1, 64, gq, cl, dk);  // E K
      dk = tile_mma(&sm.dt[16 * s], 1, LDF, &sm.x1[16 * bj], LDF, 1, 64, gq, cl, dk);  // E^T K
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * s + 4 * gq + i, cc = 16 * bj + cl, col = 64 * kb + cc;
        const float ar = sm.a[r], br = sm.beta[r], cr = sm.c[r];
        const float qv = sm.x0[r * LDF + cc], kv = sm.x1[r * LDF + cc];
        const float dq = ar * y1[s][i] + pk[i];
        const float dkv = dk[i] + cr * y2[s][i] + br * ar * tdw[i];
        float vv = 0.f;
        if (r < n) {
          const int64_t gi = ((t0 + r) * H + h) * D + col;
          vv = to_f32(gv_[gi]);
          if (b.dq_part != nullptr) {  // grouped heads or normalised q, k: finished afterwards
            const int64_t ri = (t0 + r) * b.HK + hk;
            b.dq_part[gi] = b.rq ? b.rq[ri] * dq : dq;
            b.dk_part[gi] = b.rk ? b.rk[ri] * dkv : dkv;
          } else {
            static_cast<E *>(b.dq)[gi] = from_f32<E>(dq);
            static_cast<E *>(b.dk)[gi] = from_f32<E>(dkv);
          }
          static_cast<E *>(b.dv)[gi] = from_f32<E>(br * tdu[i]);
        }
        prg[s][i] += ar * y1[s][i] * qv + br * ar * tdw[i] * kv - cr * y2[s][i] * kv;
        prb[s][i] += ar * tdw[i] * kv + tdu[i] * vv;
        prc[s][i] += cr * y2[s][i] * kv;
      }
    }
  }
  // row reductions of the stage-4 terms over this wave's 16 columns
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) {
        prg[s][i] += __shfl_xor(prg[s][i], off, 64);
        prb[s][i] += __shfl_xor(prb[s][i], off, 64);
        prc[s][i] += __shfl_xor(prc[s][i], off, 64);
      }
    }
  __syncthreads();
  if (cl == 0) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * s + 4 * gq + i;
        sm.rg[wave][r] += prg[s][i];
        sm.rb[wave][r] += prb[s][i];
        sm.rc[wave][r] = prc[s][i];
      }
  }
  // lambda <dh', h>: a fixed-order block reduction
  float hd = 0.f;
  for (int i = tid; i < D * D; i += 256) hd += dhn[i] * hS[i];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) hd += __shfl_xor(hd, off, 64);
  if (lane == 0) sm.red[wave] = hd;
  __syncthreads();
  if (wave == 0) {
    const int r = lane;
    float dgam = sm.rg[0][r] + sm.rg[1][r] + sm.rg[2][r] + sm.rg[3][r] - sm.colg[r];
    const float dbet = sm.rb[0][r] + sm.rb[1][r] + sm.rb[2][r] + sm.rb[3][r];
    float csum = sm.rc[0][r] + sm.rc[1][r] + sm.rc[2][r] + sm.rc[3][r];
    if (r >= n) {
      dgam = 0.f;
      csum = 0.f;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) csum += __shfl_xor(csum, off, 64);
    const float hdot = sm.red[0] + sm.red[1] + sm.red[2] + sm.red[3];
    if (r == n - 1) dgam += csum + __expf(sm.gam[n - 1]) * hdot;
    // dg_s = sum_{r >= s} dgamma_r (reverse inclusive scan)
    float x = dgam;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float yv = __shfl_down(x, off, 64);
      if (r + off < 64) x += yv;
    }
    if (r < n) {
      b.dg[(t0 + r) * H + h] = x;
      static_cast<E *>(b.dbeta)[(t0 + r) * H + h] = from_f32<E>(dbet);
    }
  }
}

__global__ __launch_bounds__(256) void sum_dh0_kernel(const float *__restrict__ src, int N,
                                                      int64_t per_seq, float *__restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= per_seq) return;
  float acc = 0.f;
  for (int n = 0; n < N; ++n) acc += src[(int64_t)n * per_seq + i];
  dst[i] = acc;
}

// dst[n] = src[n * src_stride] (or 0 without src) for the N states of per_seq floats each.
__global__ __launch_bounds__(256) void copy_states_kernel(const float *__restrict__ src,
                                                         int64_t src_stride, int64_t n_total,
                                                         int64_t per_seq,
                                                         float *__restrict__ dst) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_total;
       i += (int64_t)gridDim.x * 256)
    dst[i] = src ? src[i / per_seq * src_stride + i % per_seq] : 0.f;
}

__global__ __launch_bounds__(256) void group_sum_kernel(const float *__restrict__ part, int64_t T,
                                                       int H, int HK, int D, int is_bf16,
                                                       void *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // element of out [T, HK, D]
  if (i >= T * HK * D) return;
  const int64_t t = i / ((int64_t)HK * D);
  const int hk = (int)(i / D % HK), d = (int)(i % D), G = H / HK;
  float s = 0.f;
  for (int j = 0; j < G; ++j) s += part[(t * H + hk * G + j) * D + d];
  if (is_bf16) static_cast<bf16 *>(out)[i] = (bf16)s;
  else static_cast<float *>(out)[i] = s;
}

// 1 / sqrt(|row|^2 + eps) per row of x [rows, D]: each row read as 16-byte units by UPR
// consecutive lanes (64 / UPR rows per wave), summed by a butterfly within the lane group.
template <class E, int D>
__global__ __launch_bounds__(256) void row_rnorm_kernel(const E *__restrict__ x, int64_t rows,
                                                        float *__restrict__ r) {
  constexpr int EPU = 16 / (int)sizeof(E);  // elements per 16-byte unit
  constexpr int UPR = D / EPU;              // lanes per row: 8 .. 32
  constexpr int RPW = 64 / UPR;             // rows per wave
  const int lane = threadIdx.x & 63, sub = lane / UPR, part = lane % UPR;
  const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  const int64_t waves = (int64_t)gridDim.x * 4;
  for (int64_t row0 = wave * RPW; row0 < rows; row0 += waves * RPW) {  // wave-uniform
    const int64_t row = row0 + sub;
    float s = 0.f;
    if (row < rows) {
      const uint4 u = *reinterpret_cast<const uint4 *>(x + row * D + part * EPU);
      const unsigned wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (sizeof(E) == 2) {
          const float lo = __uint_as_float(wd[j] << 16), hi = __uint_as_float(wd[j] & 0xFFFF0000u);
          s += lo * lo + hi * hi;
        } else {
          const float v = __uint_as_float(wd[j]);
          s += v * v;
        }
      }
    }
#pragma unroll
    for (int off = UPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    if (part == 0 && row < rows) r[row] = 1.f / sqrtf(s + kL2NormEps);
  }
}

// One wave per row (t, hk) of x [T, HK, D]; lane holds elements D / 64 * lane .. + D / 64 - 1.
template <class E, int D>
__global__ __launch_bounds__(256) void l2norm_bwd_kernel(const float *__restrict__ part,
                                                         const E *__restrict__ x,
                                                         const float *__restrict__ r, int64_t T,
                                                         int H, int HK, E *__restrict__ out) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
  if (row >= T * HK) return;  // wave-uniform
  const int64_t t = row / HK;
  const int hk = (int)(row % HK), G = H / HK;
  float z[PER], xv[PER], s = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int d = PER * lane + e;
    float acc = 0.f;
    for (int j = 0; j < G; ++j) acc += part[(t * H + (int64_t)hk * G + j) * D + d];
    z[e] = acc;
    xv[e] = to_f32(x[row * D + d]);
    s += xv[e] * acc;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  const float rr = r[row], cf = rr * rr * s;
#pragma unroll
  for (int e = 0; e < PER; ++e) out[row * D + PER * lane + e] = from_f32<E>(z[e] - cf * xv[e]);
}

hipError_t launch_row_rnorm(const void *x, int64_t rows, int32_t D, bool is_bf16, float *r,
                            hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int upr = D * (is_bf16 ? 2 : 4) / 16, rpb = 4 * (64 / upr);
  int64_t blocks = (rows + rpb - 1) / rpb;
  if (blocks > 65536) blocks = 65536;
  const dim3 grid((unsigned)blocks), block(256);
  if (D == 128) {
    if (is_bf16) hipLaunchKernelGGL((row_rnorm_kernel<bf16, 128>), grid, block, 0, stream, static_cast<const bf16 *>(x), rows, r);
    else hipLaunchKernelGGL((row_rnorm_kernel<float, 128>), grid, block, 0, stream, static_cast<const float *>(x), rows, r);
  } else {
    if (is_bf16) hipLaunchKernelGGL((row_rnorm_kernel<bf16, 64>), grid, block, 0, stream, static_cast<const bf16 *>(x), rows, r);
    else hipLaunchKernelGGL((row_rnorm_kernel<float, 64>), grid, block, 0, stream, static_cast<const float *>(x), rows, r);
  }
  return hipGetLastError();
}

hipError_t launch_l2norm_bwd(const float *part, const void *x, const float *r, int64_t T,
                             int32_t H, int32_t HK, int32_t D, bool is_bf16, void *out,
                             hipStream_t stream) {
  const int64_t rows = T * HK;
  if (rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (D == 128) {
    if (is_bf16) hipLaunchKernelGGL((l2norm_bwd_kernel<bf16, 128>), grid, block, 0, stream, part, static_cast<const bf16 *>(x), r, T, H, HK, static_cast<bf16 *>(out));
    else hipLaunchKernelGGL((l2norm_bwd_kernel<float, 128>), grid, block, 0, stream, part, static_cast<const float *>(x), r, T, H, HK, static_cast<float *>(out));
  } else {
    if (is_bf16) hipLaunchKernelGGL((l2norm_bwd_kernel<bf16, 64>), grid, block, 0, stream, part, static_cast<const bf16 *>(x), r, T, H, HK, static_cast<bf16 *>(out));
    else hipLaunchKernelGGL((l2norm_bwd_kernel<float, 64>), grid, block, 0, stream, part, static_cast<const float *>(x), r, T, H, HK, static_cast<float *>(out));
  }
  return hipGetLastError();
}

hipError_t launch_group_sum(const float *part, int64_t T, int32_t H, int32_t HK, int32_t D,
                            bool bf16, void *out, hipStream_t stream) {
  const int64_t n = T * HK * D;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(group_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     part, T, H, HK, D, bf16 ? 1 : 0, out);
  return hipGetLastError();
}

hipError_t launch_bwd_chain(const BwdArgs &b, int D, bool is_bf16, hipStream_t stream) {
  const dim3 grid(b.N, b.H), block(256);
  if (D == 128) {
    if (is_bf16) return hipErrorNotSupported;  // bf16, d = 128 runs gdn_bwd_chain.hip
    else hipLaunchKernelGGL((bwd_chain_kernel<128, float>), grid, block, 0, stream, b);
  } else {
    if (is_bf16) hipLaunchKernelGGL((bwd_chain_kernel<64, bf16>), grid, block, 0, stream, b);
    else hipLaunchKernelGGL((bwd_chain_kernel<64, float>), grid, block, 0, stream, b);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_grad(const BwdArgs &b, int D, bool is_bf16, int64_t max_chunks,
                           hipStream_t stream) {
  if (max_chunks <= 0) return hipSuccess;
  const dim3 grid((unsigned)max_chunks, b.H), block(256);
  if (D == 128) {
    if (is_bf16) return hipErrorNotSupported;  // bf16, d = 128 runs gdn_bwd_grad.hip
    else hipLaunchKernelGGL((bwd_grad_kernel<128, float>), grid, block, 0, stream, b);
  } else {
    if (is_bf16) hipLaunchKernelGGL((bwd_grad_kernel<64, bf16>), grid, block, 0, stream, b);
    else hipLaunchKernelGGL((bwd_grad_kernel<64, float>), grid, block, 0, stream, b);
  }
  return hipGetLastError();
}

hipError_t launch_sum_dh0(const float *dh0_seq, int32_t N, int32_t H, int32_t D, float *dh0,
                          hipStream_t stream) {
  const int64_t per_seq = (int64_t)H * D * D;
  hipLaunchKernelGGL(sum_dh0_kernel, dim3((unsigned)((per_seq + 255) / 256)), dim3(256), 0,
                     stream, dh0_seq, N, per_seq, dh0);
  return hipGetLastError();
}

hipError_t launch_copy_states(const float *src, int64_t src_stride, int32_t N, int32_t H,
                              int32_t D, float *dst, hipStream_t stream) {
  const int64_t per_seq = (int64_t)H * D * D, n_total = per_seq * N;
  int64_t blocks = (n_total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(copy_states_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, src,
                     src_stride, n_total, per_seq, dst);
  return hipGetLastError();
}

}  // namespace gdn
