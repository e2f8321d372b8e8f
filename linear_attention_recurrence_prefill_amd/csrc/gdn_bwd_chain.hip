// Reverse state-gradient chain of the backward for bf16 inputs with d_k = d_v = 128 on gfx950.
//
// Per chunk (n <= 64 tokens, gamma = cumsum(g), a = e^gamma, c = e^{gamma_last - gamma},
// lambda = e^{gamma_last}, dO_s = scale dO, P = (Q K^T) o e^{gamma_r - gamma_i} on i <= r), walking
// each sequence backwards from dh' = dht (the gradient of the state after the chunk):
//     dDelta = P^T dO_s + diag(c) K dh'
//     dh     = lambda dh' + Q^T diag(a) dO_s - W^T dDelta,      W = Tm diag(beta a) K
// the reverse-mode derivative of the chunked form of "How to Speed Up GDN Kernels for Qwen
// Models" (section "What GDN actually computes"); the hidden states themselves are recomputed by
// a forward pass ("Lever 2").  dh' of every chunk and dDelta go to the workspace for the
// per-chunk gradient kernel.
//
// Products run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  q, k and dO are bf16 inputs
// and enter exactly.  Every other operand (dh', W, dDelta, P, a dO) is split into a bf16 head and
// a bf16 remainder, x = hi + lo, and the product is taken as hi * y + lo * y (y exact) or
// hi * hi' + hi * lo' + lo * hi' (both split): about 16 significant bits per operand, so the chain
// keeps close to fp32 accuracy over thousands of chunks.
//
// One workgroup of four waves per (sequence, head); wave w owns columns [32 w, 32 w + 32) of the
// state gradient as MFMA accumulator tiles (rows 16 md + 4 gq + i, column 32 w + 16 nt + cl).
// Per chunk the tiles (K, Q, dO, W split, P^T split) are staged in LDS; products that contract
// over tokens read the token-major tiles with the transposing LDS read.  The contraction index of
// a pair of accumulator tiles used as an MFMA operand is permuted (item j of lane group gq is
// index 32 ks + 16 (j / 4) + 4 gq + j % 4) and the LDS operand is read in the same order.
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_unit.h"

namespace gdn {
namespace {

constexpr int kD = 128;
constexpr int kRowB = kD * 2;  // bytes per row of a 64 x 128 bf16 tile

// 64 x 128 bf16 token-major tiles: the 16-byte unit c of row r is stored at unit c ^ sw(r), so
// that 16 lanes reading one 8-byte unit of 16 consecutive rows, and the transposing read of 4
// consecutive 8-byte units of 8 consecutive rows, each touch every bank pair once per half-wave.
__device__ __forceinline__ int sw(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
// byte offset of the 8-byte unit u (elements 4 u .. 4 u + 3) of row r
__device__ __forceinline__ int toff(int r, int u) {
  return r * kRowB + (((u >> 1) ^ sw(r)) << 4) + ((u & 1) << 3);
}
// 64 x 64 bf16 (P^T): rows of 128 bytes, the 8-byte unit u of row r at u ^ 2 ((r / 2) % 8)
__device__ __forceinline__ int poff(int r, int u) {
  return r * 128 + ((u ^ (((r >> 1) & 7) << 1)) << 3);
}

__device__ __forceinline__ bf16x4 ld8(const char *p) { return *reinterpret_cast<const bf16x4 *>(p); }
__device__ __forceinline__ bf16x4 ldtr(const char *p) {
  return lds_tr16(reinterpret_cast<const bf16 *>(p));
}
__device__ __forceinline__ f32x4 to_f32x4(bf16x4 x) { return __builtin_convertvector(x, f32x4); }

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi), for a pair of accumulator tiles (items
// 0..3 from x0, 4..7 from x1)
__device__ __forceinline__ void split8(f32x4 x0, f32x4 x1, bf16x8 &hi, bf16x8 &lo) {
  const bf16x4 h0 = to_bf16x4(x0), h1 = to_bf16x4(x1);
  hi = cat8(h0, h1);
  lo = cat8(to_bf16x4(x0 - to_f32x4(h0)), to_bf16x4(x1 - to_f32x4(h1)));
}

struct ChainSmem {
  alignas(16) char k[64 * kRowB];
  alignas(16) char q[64 * kRowB];
  alignas(16) char dout[64 * kRowB];
  alignas(16) char whi[64 * kRowB];  // W = hi + lo
  alignas(16) char wlo[64 * kRowB];
  alignas(16) char pthi[64 * 128];  // P^T = hi + lo (row i, column r)
  alignas(16) char ptlo[64 * 128];
  alignas(16) float gam[64];  // gamma, rows past n hold gamma_last
  alignas(16) float as[64];   // scale e^gamma, 0 past n
  alignas(16) float c[64];    // e^{gamma_last - gamma}, 0 past n
  alignas(16) int imisc[4];
};
static_assert(sizeof(ChainSmem) <= 160 * 1024, "LDS budget");

// P's 16 x 16 tiles on or below the diagonal: tile t is rows 16 tr[t] .. (tokens r), columns
// 16 ti[t] .. (tokens i)
__constant__ int kPtR[10] = {0, 1, 1, 2, 2, 2, 3, 3, 3, 3};
__constant__ int kPtI[10] = {0, 0, 1, 0, 1, 2, 0, 1, 2, 3};

}  // namespace

__global__ __launch_bounds__(256) void bwd_chain_bf16_kernel(BwdArgs b) {
  __shared__ ChainSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 4, cl = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int seq = blockIdx.x, h = blockIdx.y, H = b.H;
  if (w == 0) {
    Unit un;
    const bool ok = find_unit(b.cu, b.N, 0, seq, true, lane, un);
    if (lane == 0) {
      sm.imisc[0] = ok ? (int)un.chunk_base : -1;
      sm.imisc[1] = un.c1;
    }
  }
  // P^T above the diagonal (row block > column block) is read but never written: zero it once
  for (int i = tid; i < 6 * 64; i += 256) {
    const int t = i >> 6, rr = (i >> 2) & 15, u = i & 3;
    const int mi = t < 1 ? 1 : (t < 3 ? 2 : 3), mr = t < 1 ? 0 : (t < 3 ? t - 1 : t - 3);
    const int off = poff(16 * mi + rr, 4 * mr + u);
    *reinterpret_cast<uint2 *>(&sm.pthi[off]) = uint2{0u, 0u};
    *reinterpret_cast<uint2 *>(&sm.ptlo[off]) = uint2{0u, 0u};
  }
  __syncthreads();
  if (sm.imisc[0] < 0) return;
  const int64_t chunk_base = sm.imisc[0];
  const int nch = sm.imisc[1];
  const int64_t ts0 = b.cu[seq], ts1 = b.cu[seq + 1];
  if (ts0 < 0 || ts1 < ts0 || ts1 > b.T) return;  // malformed cu_seqlens: touch nothing
  const int64_t tok_bytes = (int64_t)H * kRowB;
  const char *__restrict__ gk = static_cast<const char *>(b.k) + (int64_t)h * kRowB;
  const char *__restrict__ gqp = static_cast<const char *>(b.q) + (int64_t)h * kRowB;
  const char *__restrict__ gdo = static_cast<const char *>(b.dout) + (int64_t)h * kRowB;
  const int col0 = 32 * w + cl;  // this lane's column in tile nt: col0 + 16 nt
  const int64_t dd = (int64_t)kD * kD;

  f32x4 G[8][2];  // dh' (starts at dht, or zero)
#pragma unroll
  for (int md = 0; md < 8; ++md)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        G[md][nt][i] = b.dht ? b.dht[((int64_t)seq * H + h) * dd +
                                     (16 * md + 4 * gq + i) * kD + col0 + 16 * nt]
                             : 0.f;

  // lane-constant LDS offsets
  int o_kf[4][2];  // A operand rows cl, contraction units 8 ks + 4 hf + gq
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) o_kf[ks][hf] = toff(cl, 8 * ks + 4 * hf + gq);
  auto kfrag = [&](const char *t, int m, int ks) {
    return cat8(ld8(t + m * 16 * kRowB + o_kf[ks][0]), ld8(t + m * 16 * kRowB + o_kf[ks][1]));
  };
  auto pfrag = [&](const char *t, int m, int ks) {
    const int r = 16 * m + cl;
    return cat8(ld8(t + poff(r, 8 * ks + gq)), ld8(t + poff(r, 8 * ks + 4 + gq)));
  };
  // transposing reads: lane (cl, gq) receives rows 32 ks + 16 hf + 4 gq .. + 3 of column
  // 4 u0 + cl, addressing row 32 ks + 16 hf + 4 gq + cl / 4, 8-byte unit u0 + cl % 4
  auto trfrag = [&](const char *t, int ks, int u0) {
    const int r = 32 * ks + 4 * gq + (cl >> 2), u = u0 + (cl & 3);
    return cat8(ldtr(t + toff(r, u)), ldtr(t + toff(r + 16, u)));
  };

  for (int c = nch - 1; c >= 0; --c) {
    const int64_t t0 = ts0 + (int64_t)c * kChunk;
    const int n = (int)min<int64_t>(kChunk, ts1 - t0);
    const int64_t cg = chunk_base + c;
    __syncthreads();  // the previous chunk is done with LDS
    // ---- stage K, Q, dO (bf16 as they are) and W (fp32, split) in LDS; rows past n are zero
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int u = tid + 256 * m, r = u >> 4, c16 = u & 15;
      uint4 kv{0u, 0u, 0u, 0u}, qv = kv, ov = kv;
      if (r < n) {
        const int64_t off = (t0 + r) * tok_bytes + c16 * 16;
        kv = *reinterpret_cast<const uint4 *>(gk + off);
        qv = *reinterpret_cast<const uint4 *>(gqp + off);
        ov = *reinterpret_cast<const uint4 *>(gdo + off);
      }
      const int lo = r * kRowB + ((c16 ^ sw(r)) << 4);
      *reinterpret_cast<uint4 *>(&sm.k[lo]) = kv;
      *reinterpret_cast<uint4 *>(&sm.q[lo]) = qv;
      *reinterpret_cast<uint4 *>(&sm.dout[lo]) = ov;
    }
    {
      const float *wsrc = b.w + (cg * H + h) * 64 * kD;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int u = tid + 256 * m, r = u >> 5, c4 = u & 31;
        const f32x4 x = r < n ? *reinterpret_cast<const f32x4 *>(wsrc + r * kD + 4 * c4) : zero4();
        const bf16x4 hi = to_bf16x4(x);
        *reinterpret_cast<bf16x4 *>(&sm.whi[toff(r, c4)]) = hi;
        *reinterpret_cast<bf16x4 *>(&sm.wlo[toff(r, c4)]) = to_bf16x4(x - to_f32x4(hi));
      }
    }
    if (w == 0) {
      const float gmv = lane < n ? b.gamma[(t0 + lane) * H + h] : 0.f;
      const float glast = __shfl(gmv, n - 1, 64);
      sm.gam[lane] = lane < n ? gmv : glast;
      sm.as[lane] = lane < n ? b.scale * __expf(gmv) : 0.f;
      sm.c[lane] = lane < n ? __expf(glast - gmv) : 0.f;
    }
    __syncthreads();
    // ---- P^T = ((Q K^T) o decay)^T on and below the diagonal, split into hi + lo
    for (int t = w; t < 10; t += 4) {
      const int mr = kPtR[t], mi = kPtI[t];
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mma_bf16(kfrag(sm.q, mr, ks), kfrag(sm.k, mi, ks), acc);
      // acc[j] = q_r . k_i for r = 16 mr + 4 gq + j, i = 16 mi + cl
      const int i = 16 * mi + cl;
      const float gi = sm.gam[i];
      f32x4 p;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * mr + 4 * gq + j;
        p[j] = (i <= r && r < n) ? __expf(sm.gam[r] - gi) * acc[j] : 0.f;
      }
      const bf16x4 hi = to_bf16x4(p);
      const int off = poff(i, 4 * mr + gq);
      *reinterpret_cast<bf16x4 *>(&sm.pthi[off]) = hi;
      *reinterpret_cast<bf16x4 *>(&sm.ptlo[off]) = to_bf16x4(p - to_f32x4(hi));
    }
    __syncthreads();
    const float lam = __expf(sm.gam[63]);

    // ---- dh' of this chunk to the workspace
    float *dhn = b.dhn + (cg * H + h) * dd;
#pragma unroll
    for (int md = 0; md < 8; ++md)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) dhn[(16 * md + 4 * gq + i) * kD + col0 + 16 * nt] = G[md][nt][i];

    // ---- dDelta = P^T dO_s + diag(c) K dh'
    f32x4 kd[4][2], x[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) kd[mt][nt] = x[mt][nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 gh[2], gl[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) split8(G[2 * ks][nt], G[2 * ks + 1][nt], gh[nt], gl[nt]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 a = kfrag(sm.k, mt, ks);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          kd[mt][nt] = mma_bf16(a, gh[nt], kd[mt][nt]);
          kd[mt][nt] = mma_bf16(a, gl[nt], kd[mt][nt]);
        }
      }
    }
    bf16x8 of[2][2];  // dO as the B operand over tokens, exact
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) of[ks][nt] = trfrag(sm.dout, ks, 8 * w + 4 * nt);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (2 * ks + 1 < mt) continue;  // P^T[i][r] = 0 for r < i: tokens 0..31 vs rows >= 32
        const bf16x8 ah = pfrag(sm.pthi, mt, ks), al = pfrag(sm.ptlo, mt, ks);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          x[mt][nt] = mma_bf16(ah, of[ks][nt], x[mt][nt]);
          x[mt][nt] = mma_bf16(al, of[ks][nt], x[mt][nt]);
        }
      }
    f32x4 dD[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const f32x4 cr = *reinterpret_cast<const f32x4 *>(&sm.c[16 * mt + 4 * gq]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        dD[mt][nt] = b.scale * x[mt][nt] + cr * kd[mt][nt];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * mt + 4 * gq + i;
          if (r < n) b.ddelta[((t0 + r) * H + h) * kD + col0 + 16 * nt] = dD[mt][nt][i];
        }
      }
    }

    // ---- dh = lambda dh' + Q^T (scale a o dO) - W^T dDelta
    bf16x8 yh[2][2], yl[2][2], nh[2][2], nl[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const f32x4 a0 = *reinterpret_cast<const f32x4 *>(&sm.as[32 * ks + 4 * gq]);
      const f32x4 a1 = *reinterpret_cast<const f32x4 *>(&sm.as[32 * ks + 16 + 4 * gq]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const bf16x8 o = of[ks][nt];
        const f32x4 o0 = to_f32x4(__builtin_shufflevector(o, o, 0, 1, 2, 3));
        const f32x4 o1 = to_f32x4(__builtin_shufflevector(o, o, 4, 5, 6, 7));
        split8(a0 * o0, a1 * o1, yh[ks][nt], yl[ks][nt]);
        split8(-dD[2 * ks][nt], -dD[2 * ks + 1][nt], nh[ks][nt], nl[ks][nt]);
      }
    }
#pragma unroll
    for (int md = 0; md < 8; ++md) {
      f32x4 acc[2] = {lam * G[md][0], lam * G[md][1]};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 aq = trfrag(sm.q, ks, 4 * md);
        const bf16x8 awh = trfrag(sm.whi, ks, 4 * md);
        const bf16x8 awl = trfrag(sm.wlo, ks, 4 * md);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          acc[nt] = mma_bf16(aq, yh[ks][nt], acc[nt]);
          acc[nt] = mma_bf16(aq, yl[ks][nt], acc[nt]);
          acc[nt] = mma_bf16(awh, nh[ks][nt], acc[nt]);
          acc[nt] = mma_bf16(awh, nl[ks][nt], acc[nt]);
          acc[nt] = mma_bf16(awl, nh[ks][nt], acc[nt]);
        }
      }
      G[md][0] = acc[0];
      G[md][1] = acc[1];
    }
  }
  if (b.dh0_seq != nullptr) {
    float *dst = b.dh0_seq + ((int64_t)seq * H + h) * dd;
#pragma unroll
    for (int md = 0; md < 8; ++md)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(16 * md + 4 * gq + i) * kD + col0 + 16 * nt] = G[md][nt][i];
  }
}

hipError_t launch_bwd_chain_bf16(const BwdArgs &b, hipStream_t stream) {
  hipLaunchKernelGGL(bwd_chain_bf16_kernel, dim3(b.N, b.H), dim3(256), 0, stream, b);
  return hipGetLastError();
}

}  // namespace gdn
