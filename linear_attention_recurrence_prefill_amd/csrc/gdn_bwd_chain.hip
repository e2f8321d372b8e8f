// Reverse state-gradient chain of the backward for bf16 inputs with d_k = d_v = 128 on gfx950.
//
// Per chunk (n <= 64 tokens, gamma = cumsum(g), a = e^gamma, c = e^{gamma_last - gamma},
// lambda = e^{gamma_last}, dO_s = scale dO, P = (Q K^T) o e^{gamma_r - gamma_i} on i <= r), walking
// each sequence backwards from dh' = dht (the gradient of the state after the chunk):
//     dDelta = P^T dO_s + diag(c) K dh'
//     dR     = Tm^T dDelta                     (dV = diag(beta) dR)
//     dh     = lambda dh' + Q^T diag(a) dO_s - K^T diag(a beta) dR
// (the last term is W^T dDelta with W = Tm diag(beta a) K), the reverse-mode derivative of the
// chunked form of "How to Speed Up GDN Kernels for Qwen Models" (section "What GDN actually
// computes"); the hidden states themselves are recomputed by a forward pass ("Lever 2").  dh' of
// every chunk (in bf16: the gradient kernel's products take it as a bf16 operand), dR and dV go
// out for the per-chunk gradient kernel.
//
// Products run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  q, k and dO are bf16 inputs
// and enter exactly.  Every other operand (dh', dDelta, dR, Tm, P, a dO) is split into a bf16
// head and a bf16 remainder, x = hi + lo, and the product is taken as hi * y + lo * y (y exact)
// or hi * hi' + hi * lo' + lo * hi' (both split): about 16 significant bits per operand, so the
// chain keeps close to fp32 accuracy over thousands of chunks.
//
// One workgroup of eight waves per (unit, head), a unit being a sequence or a segment of it;
// wave w owns columns [16 w, 16 w + 16) of the state gradient as MFMA accumulator tiles (rows
// 16 md + 4 gq + i, column 16 w + cl).  K, Q and dO of the next chunk stream from HBM
// into a second set of LDS tiles with direct global->LDS loads while the current chunk runs, and
// so does Tm^T (already split and laid out by bwd_tm_kernel); the gates of the next chunk are
// loaded into registers and moved to LDS at the chunk turn.
// Products that contract over tokens read the token-major tiles with the transposing LDS read.
// The contraction index of a pair of accumulator tiles used as an MFMA operand is permuted (item
// j of lane group gq is index 32 ks + 16 (j / 4) + 4 gq + j % 4) and the LDS operand is read in
// the same order.
//
// Exact split (as in the forward): the map from a unit's end gradient to its start gradient is
// affine, dh_start = M^T dh_end + B', with M the forward map of the same unit (the derivative of
// S_end = M S_start + B; the forward recompute computes M).  The transition pass runs each unit
// from a zero end gradient (B'); a reverse walk of the affine scan composes M^T and B' into every
// unit's true end gradient; the final pass reruns each unit from it with the per-chunk outputs.
#include "gdn_bwd_internal.h"
#include "gdn_device.h"
#include "gdn_tiles.h"
#include "gdn_unit.h"

namespace gdn {
namespace {

constexpr int kD = 128;
constexpr int kRowB = kD * 2;  // bytes per row of a 64 x 128 bf16 tile
// The 16-row blocks of every LDS tile sit 16 bytes further apart than their size: two reads at
// the same lane offset a whole number of 512-byte steps apart would otherwise be fused by the
// compiler into one ds_read2st64_b64, which the hardware serves as two passes over the same banks.
constexpr int kBlk = 16 * kRowB + 16;  // 64 x 128 tiles (K, Q, dO)
constexpr int kTile = 4 * kBlk;
constexpr int pBlk = 16 * 128 + 16;    // 64 x 64 tiles (P^T, Tm^T)
constexpr int pTile = 4 * pBlk;
// Eight waves of 16 state-gradient columns each (kNT = 1 column tile of 16 per wave): two waves
// per SIMD, so that one wave's MFMA, LDS and store latencies overlap the other's work.
constexpr int kWaves = 8;
constexpr int kNT = 8 / kWaves;
constexpr int kThreads = 64 * kWaves;

// 64 x 128 bf16 token-major tiles: the 16-byte unit c of row r is stored at unit c ^ sw(r), so
// that 16 lanes reading one 8-byte unit of 16 consecutive rows, and the transposing read of 4
// consecutive 8-byte units of 8 consecutive rows, each touch every bank pair once per half-wave.
__device__ __forceinline__ int sw(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
// byte offset of the 8-byte unit u (elements 4 u .. 4 u + 3) of row r
__device__ __forceinline__ int toff(int r, int u) {
  return (r >> 4) * kBlk + (r & 15) * kRowB + (((u >> 1) ^ sw(r)) << 4) + ((u & 1) << 3);
}
// 64 x 64 bf16 (P^T, Tm^T): rows of 128 bytes, the 8-byte unit u of row r at u ^ 2 ((r / 2) % 8)
__device__ __forceinline__ int poff0(int r, int u) {  // unpadded: Tm^T as bwd_tm_kernel stores it
  return r * 128 + ((u ^ (((r >> 1) & 7) << 1)) << 3);
}
__device__ __forceinline__ int poff(int r, int u) { return (r >> 4) * pBlk + poff0(r & 15, u); }

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

// next-chunk loads: untracked, waited for by wait_vm0 at the chunk turn
__device__ __forceinline__ void dma16(const char *g, char *l) { dma16_untracked(g, l); }
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

struct ChainSmem {
  alignas(16) char kqo[2][3][kTile];  // [set][K, Q, dO]: this chunk's and the next chunk's
  alignas(16) char tt[2][2][pTile];  // [set][hi, lo]: Tm^T = hi + lo (row r, column i)
  alignas(16) char pth[pTile];       // P^T = hi + lo (row i, column r)
  alignas(16) char ptl[pTile];
  // per-token gate vectors, [set] as the tiles: the next chunk's are written at the end of a step
  alignas(16) float gam[2][64];  // gamma, rows past n hold gamma_last
  alignas(16) float as[2][64];   // scale e^gamma, 0 past n
  alignas(16) float c[2][64];    // e^{gamma_last - gamma}, 0 past n
  alignas(16) float ab[2][64];   // e^gamma beta, 0 past n
  alignas(16) float beta[2][64];
  alignas(16) float rq[2][64], rk[2][64];  // q/k L2 normalisation: inverse row norms (1 without)
  alignas(16) int imisc[8];
};
static_assert(sizeof(ChainSmem) <= 160 * 1024, "LDS budget");


}  // namespace

template <bool kTransition>
__global__ __launch_bounds__(kThreads) void bwd_chain_bf16_kernel(BwdArgs b, BwdUnits us) {
  __shared__ ChainSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 4, cl = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int unit = blockIdx.x, h = blockIdx.y, H = b.H;
  if (w == 0) {
    Unit un;
    const bool ok = find_unit(b.cu, b.N, b.T, us.L, unit, true, lane, un);
    // the chain starts at chunk ce - 1: the unit's last chunk, or (truncate mode) the last of
    // its warmup window after it
    int ce = un.c1;
    if (!kTransition && us.truncate && ok) {
      const int64_t s0 = b.cu[un.seq], s1 = b.cu[un.seq + 1];  // checked by find_unit
      const int nc = (int)((s1 - s0 + kChunk - 1) / kChunk);
      if (un.c1 < nc) ce = warm_window_rev(b.g, s0, s1, un.c1, nc, h, H, us.log_thr, lane);
    }
    if (lane == 0) {
      sm.imisc[0] = ok ? un.seq : -1;
      sm.imisc[1] = un.c0;
      sm.imisc[2] = un.c1;
      sm.imisc[3] = (int)un.chunk_base;
      sm.imisc[4] = ce;
    }
  }
  // P^T's tiles below the diagonal (row block > column block) are read but never written: zero
  // them once (Tm^T is written whole every chunk)
  for (int i = tid; i < 6 * 64; i += kThreads) {
    const int t = i >> 6, rr = (i >> 2) & 15, u = i & 3;
    const int mi = t < 1 ? 1 : (t < 3 ? 2 : 3), mr = t < 1 ? 0 : (t < 3 ? t - 1 : t - 3);
    const int off = poff(16 * mi + rr, 4 * mr + u);
    *reinterpret_cast<uint2 *>(&sm.pth[off]) = uint2{0u, 0u};
    *reinterpret_cast<uint2 *>(&sm.ptl[off]) = uint2{0u, 0u};
  }
  __syncthreads();
  const int seq = __builtin_amdgcn_readfirstlane(sm.imisc[0]);
  if (seq < 0) return;
  const int c0 = __builtin_amdgcn_readfirstlane(sm.imisc[1]);
  const int c1 = __builtin_amdgcn_readfirstlane(sm.imisc[2]);
  const int ce = __builtin_amdgcn_readfirstlane(sm.imisc[4]);
  const int64_t chunk_base = __builtin_amdgcn_readfirstlane(sm.imisc[3]);
  const int64_t ts0 = b.cu[seq], ts1 = b.cu[seq + 1];
  if (ts0 < 0 || ts1 < ts0 || ts1 > b.T) return;  // malformed cu_seqlens: touch nothing
  if (kTransition && c0 == 0) return;  // a sequence's first unit has no predecessor
  const int64_t tok_bytes = (int64_t)H * kRowB;
  const int hk = h / (H / b.HK);                   // this value head's key head
  const int64_t tok_qk = (int64_t)b.HK * kRowB;    // stride of one token in q, k
  const char *__restrict__ gk = static_cast<const char *>(b.k) + (int64_t)hk * kRowB;
  const char *__restrict__ gqp = static_cast<const char *>(b.q) + (int64_t)hk * kRowB;
  const char *__restrict__ gdo = static_cast<const char *>(b.dout) + (int64_t)h * kRowB;
  const bf16 *__restrict__ gb = static_cast<const bf16 *>(b.beta);
  const int col0 = 16 * kNT * w + cl;  // this lane's column in tile nt: col0 + 16 nt
  const int64_t dd = (int64_t)kD * kD;
  const float xs = b.scale;

  f32x4 G[8][kNT];  // dh'
  {
    const float *src = nullptr;
    const int ncs = (int)((ts1 - ts0 + kChunk - 1) / kChunk);  // the sequence's chunks
    if (!kTransition)  // dht where the chain starts at the sequence's end
      src = us.unit_dend != nullptr            ? us.unit_dend + ((int64_t)unit * H + h) * dd
            : (b.dht != nullptr && ce == ncs) ? b.dht + ((int64_t)seq * H + h) * dd
                                              : nullptr;
#pragma unroll
    for (int md = 0; md < 8; ++md)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * md + 4 * gq + i, cc = col0 + 16 * nt;
          G[md][nt][i] = src != nullptr ? src[r * kD + cc] : 0.f;
        }
  }

  // lane-constant LDS offsets
  int o_kf[4][2];  // A operand rows cl, contraction units 8 ks + 4 hf + gq
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) o_kf[ks][hf] = toff(cl, 8 * ks + 4 * hf + gq);
  auto kfrag = [&](const char *t, int m, int ks) {
    return cat8(ld8(t + m * kBlk + o_kf[ks][0]), ld8(t + m * kBlk + o_kf[ks][1]));
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

  // store offsets (bytes): row 4 gq of a 128 x 128 bf16 matrix and token 4 gq of a [T, H, 128]
  // fp32 tensor, at this lane's column of tile nt
  int o_st[kNT], o_tk[kNT];
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    o_st[nt] = (4 * gq * kD + col0 + 16 * nt) * 2;
    o_tk[nt] = (4 * gq * H * kD + col0 + 16 * nt) * 4;
  }

  auto chunk_t0 = [&](int c) { return ts0 + (int64_t)c * kChunk; };
  auto chunk_n = [&](int c) { return (int)min<int64_t>(kChunk, ts1 - chunk_t0(c)); };
  // next-chunk loads: K, Q, dO by direct loads into tile set `set` (wave w: rows 16 w .. 16 w +
  // 15; lane l of load j writes physical unit l % 16 of row 16 w + 4 j + l / 16, which holds
  // logical unit (l % 16) ^ sw(row); rows past n repeat the chunk's last token); Tm (this
  // thread's 16 entries) and the gates into registers
  float g_r = 0.f, rq_r = 1.f, rk_r = 1.f;
  unsigned short b_r = 0;  // beta's bits: converted at the chunk turn, so that nothing waits
                           // for the next chunk's loads early
  auto issue = [&](int c, int set) {
    const int64_t t0 = chunk_t0(c);
    const int n = chunk_n(c);
#pragma unroll
    for (int j = 0; j < 16 / kWaves; ++j) {
      const int r = (64 / kWaves) * w + 4 * j + (lane >> 4);
      const int64_t t = t0 + min(r, n - 1);
      const int u = ((lane & 15) ^ sw(r)) << 4;
      const int row0 = (64 / kWaves) * w + 4 * j;  // 4 rows, within one 16-row block
      const int lo = (row0 >> 4) * kBlk + (row0 & 15) * kRowB;
      dma16(gk + t * tok_qk + u, sm.kqo[set][0] + lo);
      dma16(gqp + t * tok_qk + u, sm.kqo[set][1] + lo);
      dma16(gdo + t * tok_bytes + u, sm.kqo[set][2] + lo);
    }
    // Tm^T hi and lo: 16 KiB in the tiles' layout without the block padding (bwd_tm_kernel),
    // copied 1 KiB (half a 16-row block) at a time to its padded place
    const char *tm = reinterpret_cast<const char *>(b.tmat) + ((chunk_base + c) * H + h) * 16384;
#pragma unroll
    for (int j = 0; j < 16 / kWaves; ++j) {
      const int q = (16 / kWaves) * w + j;
      dma16(tm + q * 1024 + 16 * lane, &sm.tt[set][q >> 3][0] + ((q & 7) >> 1) * pBlk + (q & 1) * 1024);
    }
    if (w == 0) {
      const int64_t t = t0 + min(lane, n - 1);
      g_r = b.gamma[t * H + h];
      b_r = reinterpret_cast<const unsigned short *>(gb)[t * H + h];
      if (b.rq != nullptr) {
        rq_r = b.rq[t * b.HK + hk];
        rk_r = b.rk[t * b.HK + hk];
      }
    }
  };

  // wave 0: chunk c's gate vectors (its loads, from issue) into set gs
  auto put_gates = [&](int c, int gs) {
    const int n = chunk_n(c);
    const float glast = __shfl(g_r, n - 1, 64);
    const bool in = lane < n;
    const float ea = __expf(g_r);
    const float bt = __uint_as_float((unsigned)b_r << 16);
    // normalised q, k: the rows' inverse norms fold into the factors of Q and K below
    sm.gam[gs][lane] = in ? g_r : glast;
    sm.as[gs][lane] = in ? xs * ea * rq_r : 0.f;
    sm.c[gs][lane] = in ? __expf(glast - g_r) * rk_r : 0.f;
    sm.ab[gs][lane] = in ? ea * bt * rk_r : 0.f;
    sm.beta[gs][lane] = in ? bt : 0.f;
    sm.rq[gs][lane] = rq_r;
    sm.rk[gs][lane] = rk_r;
  };

  if (ce > c0) {
    issue(ce - 1, 0);
    if (w == 0) put_gates(ce - 1, 0);
  }
  for (int c = ce - 1, it = 0; c >= c0; --c, ++it) {
    const bool emit = !kTransition && c < c1;  // the unit's own chunks (not a warmup's)
    const int set = it & 1;
    const char *Kt = sm.kqo[set][0], *Qt = sm.kqo[set][1], *Ot = sm.kqo[set][2];
    const int64_t t0 = chunk_t0(c);
    const int n = chunk_n(c);
    const int64_t cg = chunk_base + c;
    wait_vm0();       // this chunk's loads have landed (and this wave's stores are done)
    __syncthreads();  // ... for every wave, and its gate vectors; every wave is done with the
                      // previous chunk's LDS
    // ---- the next chunk's loads (in flight through this chunk)
    if (c > c0) issue(c - 1, set ^ 1);
    // ---- P^T = ((Q K^T) o decay)^T on and below the diagonal, split into hi + lo
    for (int t = w; t < 10; t += kWaves) {
      int mr, mi;
      tri_tile(t, mr, mi);
      // the gates first, so that their LDS reads overlap the products
      const int i = 16 * mi + cl;
      const float gi = sm.gam[set][i], ki = sm.rk[set][i];
      const f32x4 gr = *reinterpret_cast<const f32x4 *>(&sm.gam[set][16 * mr + 4 * gq]);
      const f32x4 rr = *reinterpret_cast<const f32x4 *>(&sm.rq[set][16 * mr + 4 * gq]);
      bf16x8 fq[4], fk[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        fq[ks] = kfrag(Qt, mr, ks);
        fk[ks] = kfrag(Kt, mi, ks);
      }
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mma_bf16(fq[ks], fk[ks], acc);
      // acc[j] = q_r . k_i for r = 16 mr + 4 gq + j, i = 16 mi + cl; branch-free (above the
      // diagonal the exponential may overflow: the select drops it)
      f32x4 p;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * mr + 4 * gq + j;
        const float v = (rr[j] * ki) * __expf(gr[j] - gi) * acc[j];
        p[j] = (i <= r && r < n) ? v : 0.f;
      }
      const bf16x4 hi = to_bf16x4(p);
      const int off = poff(i, 4 * mr + gq);
      *reinterpret_cast<bf16x4 *>(&sm.pth[off]) = hi;
      *reinterpret_cast<bf16x4 *>(&sm.ptl[off]) = to_bf16x4(p - to_f32x4(hi));
    }
    lds_barrier();  // P^T
    const float lam = __expf(sm.gam[set][63]);

    // ---- dh' of this chunk to the workspace, in bf16 (the precision of the products that use it)
    if (emit) {  // row offsets as scalar operands
      const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(
          b.dhn_b16 + (cg * H + h) * dd, (short)0, (int)dd * 2, 0x00020000);
#pragma unroll
      for (int md = 0; md < 8; ++md)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt)
            __builtin_amdgcn_raw_buffer_store_b16(
                __builtin_bit_cast(unsigned short, (bf16)G[md][nt][i]), hr, o_st[nt],
                (16 * md + i) * kD * 2, 0);
    }

    // ---- dDelta = P^T dO_s + diag(c) K dh'
    f32x4 dD[4][kNT];
    {
      f32x4 kd[4][kNT], x[4][kNT];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) kd[mt][nt] = x[mt][nt] = zero4();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 gh[kNT], gl[kNT];
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) split8(G[2 * ks][nt], G[2 * ks + 1][nt], gh[nt], gl[nt]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const bf16x8 a = kfrag(Kt, mt, ks);
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt) {
            kd[mt][nt] = mma_bf16(a, gh[nt], kd[mt][nt]);
            kd[mt][nt] = mma_bf16(a, gl[nt], kd[mt][nt]);
          }
        }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 of[kNT];  // dO over tokens, exact
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) of[nt] = trfrag(Ot, ks, 4 * kNT * w + 4 * nt);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          if (2 * ks + 1 < mt) continue;  // P^T[i][r] = 0 for r < i: tokens 0..31 vs rows >= 32
          const bf16x8 ah = pfrag(sm.pth, mt, ks), al = pfrag(sm.ptl, mt, ks);
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt) {
            x[mt][nt] = mma_bf16(ah, of[nt], x[mt][nt]);
            x[mt][nt] = mma_bf16(al, of[nt], x[mt][nt]);
          }
        }
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 cr = *reinterpret_cast<const f32x4 *>(&sm.c[set][16 * mt + 4 * gq]);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) dD[mt][nt] = xs * x[mt][nt] + cr * kd[mt][nt];
      }
    }

    // ---- dR = Tm^T dDelta (Tm^T[r][i] = 0 for i < r); dV = diag(beta) dR
    f32x4 dR[4][kNT];
    {
      bf16x8 eh[2][kNT], el[2][kNT];  // dDelta over tokens: [ks][nt]
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) split8(dD[2 * ks][nt], dD[2 * ks + 1][nt], eh[ks][nt], el[ks][nt]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) dR[mt][nt] = zero4();
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (2 * ks + 1 < mt) continue;
          const bf16x8 th = pfrag(sm.tt[set][0], mt, ks), tl = pfrag(sm.tt[set][1], mt, ks);
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt) {
            dR[mt][nt] = mma_bf16(th, eh[ks][nt], dR[mt][nt]);
            dR[mt][nt] = mma_bf16(th, el[ks][nt], dR[mt][nt]);
            dR[mt][nt] = mma_bf16(tl, eh[ks][nt], dR[mt][nt]);
          }
        }
      }
    }
    if (emit) {  // rows at or past the chunk's end fall outside the buffer ranges
      const int64_t base = (t0 * H + h) * kD;
      const __amdgpu_buffer_rsrc_t rr =
          __builtin_amdgcn_make_buffer_rsrc(b.ddelta + base, (short)0, n * H * kD * 4, 0x00020000);
      const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
          static_cast<bf16 *>(b.dv) + base, (short)0, n * H * kD * 2, 0x00020000);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 br = *reinterpret_cast<const f32x4 *>(&sm.beta[set][16 * mt + 4 * gq]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = (16 * mt + i) * H * kD;  // + 4 gq rows in the lane-constant part
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt) {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dR[mt][nt][i]), rr,
                                                  o_tk[nt] + 4 * row, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b16(
                __builtin_bit_cast(unsigned short, (bf16)(br[i] * dR[mt][nt][i])), vr,
                o_tk[nt] / 2 + 2 * row, 0, 0);
          }
        }
      }
    }

    // ---- dh = lambda dh' + Q^T (scale a o dO) - K^T (a beta o dR)
    bf16x8 yh[2][kNT], yl[2][kNT], nh[2][kNT], nl[2][kNT];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const f32x4 a0 = *reinterpret_cast<const f32x4 *>(&sm.as[set][32 * ks + 4 * gq]);
      const f32x4 a1 = *reinterpret_cast<const f32x4 *>(&sm.as[set][32 * ks + 16 + 4 * gq]);
      const f32x4 b0 = *reinterpret_cast<const f32x4 *>(&sm.ab[set][32 * ks + 4 * gq]);
      const f32x4 b1 = *reinterpret_cast<const f32x4 *>(&sm.ab[set][32 * ks + 16 + 4 * gq]);
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const bf16x8 o = trfrag(Ot, ks, 4 * kNT * w + 4 * nt);
        const f32x4 o0 = to_f32x4(__builtin_shufflevector(o, o, 0, 1, 2, 3));
        const f32x4 o1 = to_f32x4(__builtin_shufflevector(o, o, 4, 5, 6, 7));
        split8(a0 * o0, a1 * o1, yh[ks][nt], yl[ks][nt]);
        split8(-(b0 * dR[2 * ks][nt]), -(b1 * dR[2 * ks + 1][nt]), nh[ks][nt], nl[ks][nt]);
      }
    }
#pragma unroll
    for (int md = 0; md < 8; ++md) {
      f32x4 acc[kNT];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) acc[nt] = lam * G[md][nt];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 ak = trfrag(Kt, ks, 4 * md);
        const bf16x8 aq = trfrag(Qt, ks, 4 * md);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          acc[nt] = mma_bf16(aq, yh[ks][nt], acc[nt]);
          acc[nt] = mma_bf16(aq, yl[ks][nt], acc[nt]);
        }
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          acc[nt] = mma_bf16(ak, nh[ks][nt], acc[nt]);
          acc[nt] = mma_bf16(ak, nl[ks][nt], acc[nt]);
        }
      }
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) G[md][nt] = acc[nt];
    }
    // the next chunk's gate vectors (its loads have had the whole chunk to land), visible after
    // the barrier that opens the next step
    if (w == 0 && c > c0) put_gates(c - 1, set ^ 1);
  }
  float *dst = nullptr;
  if (kTransition) {  // B' in the reverse walk's operand order (map_b_index)
    float *bo = us.unit_out + ((int64_t)unit * H + h) * dd;
#pragma unroll
    for (int md = 0; md < 8; ++md)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
        *reinterpret_cast<f32x4 *>(bo + map_b_index(16 * md + 4 * gq, col0 + 16 * nt)) = G[md][nt];
  } else if (c0 == 0 && b.dh0_seq != nullptr) {
    dst = b.dh0_seq + ((int64_t)seq * H + h) * dd;
  }
  if (dst != nullptr) {
#pragma unroll
    for (int md = 0; md < 8; ++md)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(16 * md + 4 * gq + i) * kD + col0 + 16 * nt] = G[md][nt][i];
  }
}

// Tm = (I + A)^-1 of every chunk, A_ri = beta_r e^{gamma_r - gamma_i} k_r . k_i for i < r < n
// ("How to Speed Up GDN Kernels for Qwen Models", section "What GDN actually computes"), zero
// outside [0, n)^2, by 16 x 16 blocks (block row and column indices below): the four diagonal
// blocks D_k = (I + A_kk)^-1 by forward substitution, lane 16 k + c holding column c of D_k;
// then the blocks below the diagonal in order of their distance from it,
//     T_ij = -D_i sum_{j <= k < i} A_ik T_kj,
// each 16 x 16 x 16 product on v_mfma_f32_16x16x16_bf16 with both operands split, x = hi + lo
// (hi hi' + hi lo' + lo hi': about 16 significant bits, the precision Tm is stored in).  One wave
// per (chunk, head).  K K^T on bf16 MFMA (exact products of the bf16 inputs): the blocks below
// the diagonal straight into A-operand registers, the diagonal ones into LDS.  Written for the
// reverse chain as Tm^T = hi + lo in two bf16 64 x 64 tiles laid out as the chain's LDS tiles
// without their block padding (poff0), 16 KiB per (chunk, head) of tmat.
namespace {
constexpr int kTb = 16 * 20;  // one 16 x 16 fp32 block in LDS, rows padded to 20 floats
// T's block (i, j), i >= j, at index i (i + 1) / 2 + j
__host__ __device__ constexpr int tblk(int i, int j) { return i * (i + 1) / 2 + j; }
__device__ __forceinline__ void split4(f32x4 x, bf16x4 &hi, bf16x4 &lo) {
  hi = to_bf16x4(x);
  lo = to_bf16x4(x - to_f32x4(hi));
}
__device__ __forceinline__ f32x4 mma3(bf16x4 ah, bf16x4 al, bf16x4 bh, bf16x4 bl, f32x4 c) {
  c = mma_bf16_k16(ah, bh, c);
  c = mma_bf16_k16(ah, bl, c);
  return mma_bf16_k16(al, bh, c);
}
}  // namespace

__global__ __launch_bounds__(64) void bwd_tm_kernel(BwdArgs b, float *__restrict__ tmat) {
  // tb: T's ten blocks on and below the diagonal, each transposed (tb[blk][c][r] = T_blk[r][c]);
  // dt: A's diagonal blocks transposed (dt[k][c][r] = A_kk[r][c]), then, in the same space (one
  // wave: its LDS accesses take effect in program order), dr: D_k row by row.  The output tiles
  // (16 KiB) take the whole space once every block has been read.
  __shared__ __attribute__((aligned(16))) float smem[14 * kTb];
  float *const tb = smem, *const dt = smem + 10 * kTb, *const dr = dt;
  static_assert(14 * kTb * 4 >= 16384, "output tiles fit");
  const int lane = threadIdx.x, gq = lane >> 4, cl = lane & 15;
  const int cg = blockIdx.x, h = blockIdx.y, H = b.H;
  // the chunk's sequence and index within it
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
  if (seq < 0) return;
  const int64_t ts0 = b.cu[seq], ts1 = b.cu[seq + 1];
  if (ts0 < 0 || ts1 < ts0 || ts1 > b.T) return;
  const int64_t t0 = ts0 + (int64_t)cidx * kChunk;
  const int n = (int)min<int64_t>(kChunk, ts1 - t0);
  __shared__ float sg[64], sb[64], srk[64];
  const int hk = h / (H / b.HK);  // this value head's key head
  sg[lane] = lane < n ? b.gamma[(t0 + lane) * H + h] : 0.f;
  sb[lane] = lane < n ? (float)static_cast<const bf16 *>(b.beta)[(t0 + lane) * H + h] : 0.f;
  // q/k L2 normalisation: k_r . k_i of the normalised rows = rk_r rk_i (k_r . k_i)
  srk[lane] = b.rk != nullptr && lane < n ? b.rk[(t0 + lane) * b.HK + hk] : 1.f;
  // K rows as MFMA operands straight from HBM: row 16 m + cl, elements 32 ks + 8 gq .. + 7 (rows
  // past n read the last token; A masks them)
  const bf16 *gk = static_cast<const bf16 *>(b.k) + (int64_t)hk * kD;
  bf16x8 kf[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int64_t t = t0 + min(16 * m + cl, n - 1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      kf[m][ks] = *reinterpret_cast<const bf16x8 *>(gk + t * b.HK * kD + 32 * ks + 8 * gq);
  }
  __syncthreads();
  // A_rc for rows r = 16 bi + cl and columns c = 16 bk + 4 gq + e: the MFMA with K's block bk as
  // its A operand and block bi as its B operand leaves k_c . k_r at this lane, which is the
  // k16 A-operand layout of block (bi, bk) (row cl, items 4 gq .. 4 gq + 3)
  auto ablock = [&](int bi, int bk) {
    f32x4 acc = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mma_bf16(kf[bk][ks], kf[bi][ks], acc);
    const int r = 16 * bi + cl;
    const float gr = sg[r], br = sb[r] * srk[r];
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = 16 * bk + 4 * gq + e;
      v[e] = (c < r && r < n) ? br * srk[c] * __expf(gr - sg[c]) * acc[e] : 0.f;
    }
    return v;
  };
  // the diagonal blocks, transposed into LDS: ablock(k, k) holds A_kk[cl][4 gq + e], which goes
  // to dt[k][4 gq + e][cl] (row c of dt[k] is column c of A_kk)
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f32x4 v = ablock(k, k);
#pragma unroll
    for (int e = 0; e < 4; ++e) dt[k * kTb + (4 * gq + e) * 20 + cl] = v[e];
  }
  // the blocks below the diagonal, split, in registers: a[i][k] for i > k
  bf16x4 ah[4][3], al[4][3];
#pragma unroll
  for (int i = 1; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < i; ++k) split4(ablock(i, k), ah[i][k], al[i][k]);
  __syncthreads();
  // D_k = (I + A_kk)^-1, lane 16 k + c: column c, right-looking (row r final, then taken out of
  // every later row: x_s -= A_kk[s][r] x_r, A_kk[s][r] = dt[k][r][s])
  {
    const int k = gq, c = cl;
    float x[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) x[s] = s == c ? 1.f : 0.f;
#pragma unroll
    for (int r = 0; r < 15; ++r) {
#pragma unroll
      for (int s4 = r / 4 * 4; s4 < 16; s4 += 4) {
        const f32x4 a4 = *reinterpret_cast<const f32x4 *>(&dt[k * kTb + r * 20 + s4]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (s4 + e > r) x[s4 + e] -= a4[e] * x[r];
      }
    }
    // T_kk = D_k: tb (transposed: row c of the block is column c of D_k) and dr (row by row)
#pragma unroll
    for (int s4 = 0; s4 < 16; s4 += 4)
      *reinterpret_cast<f32x4 *>(&tb[tblk(k, k) * kTb + c * 20 + s4]) =
          f32x4{x[s4], x[s4 + 1], x[s4 + 2], x[s4 + 3]};
#pragma unroll
    for (int s = 0; s < 16; ++s) dr[k * kTb + s * 20 + c] = x[s];
  }
  __syncthreads();
  // T_ij = -D_i sum_{j <= k < i} A_ik T_kj: Y = sum A_ik T_kj with T_kj as the B operand (column
  // cl, rows 4 gq ..: row cl of tb's block), then D_i Y with Y, a D-layout accumulator, as the B
  // operand as it stands; T_ij (column cl, rows 4 gq + e) to row cl of its tb block
  auto tblock = [&](int i, int j) {
    f32x4 y = zero4();
#pragma unroll
    for (int k = j; k < i; ++k) {
      bf16x4 th, tl;
      split4(*reinterpret_cast<const f32x4 *>(&tb[tblk(k, j) * kTb + cl * 20 + 4 * gq]), th, tl);
      y = mma3(ah[i][k], al[i][k], th, tl, y);
    }
    bf16x4 dh, dl, yh, yl;
    split4(*reinterpret_cast<const f32x4 *>(&dr[i * kTb + cl * 20 + 4 * gq]), dh, dl);
    split4(y, yh, yl);
    const f32x4 t = mma3(dh, dl, yh, yl, zero4());
    *reinterpret_cast<f32x4 *>(&tb[tblk(i, j) * kTb + cl * 20 + 4 * gq]) = -t;
  };
  tblock(1, 0);
  tblock(2, 1);
  tblock(3, 2);
  __syncthreads();
  tblock(2, 0);
  tblock(3, 1);
  __syncthreads();
  tblock(3, 0);
  __syncthreads();
  // column `lane` of Tm (row lane of Tm^T): rows 16 i .. 16 i + 15 from row lane % 16 of block
  // (i, lane / 16), zero above the diagonal blocks and outside [0, n)
  const int jb = lane >> 4, jc = lane & 15;
  const bool col_in = lane < n;
  float x[64];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int s4 = 0; s4 < 16; s4 += 4) {
      f32x4 v = zero4();
      if (i >= jb) v = *reinterpret_cast<const f32x4 *>(&tb[tblk(i, jb) * kTb + jc * 20 + s4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[16 * i + s4 + e] = (col_in && 16 * i + s4 + e < n) ? v[e] : 0.f;
    }
  __syncthreads();  // every block is read: the output tiles take the space
  // row `lane` of Tm^T = hi + lo, in the chain's LDS layout, then out with contiguous 16-byte
  // stores
  char *stage = reinterpret_cast<char *>(smem);
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const f32x4 v{x[4 * u], x[4 * u + 1], x[4 * u + 2], x[4 * u + 3]};
    const bf16x4 hi = to_bf16x4(v);
    *reinterpret_cast<bf16x4 *>(stage + poff0(lane, u)) = hi;
    *reinterpret_cast<bf16x4 *>(stage + 8192 + poff0(lane, u)) = to_bf16x4(v - to_f32x4(hi));
  }
  __syncthreads();
  char *dst = reinterpret_cast<char *>(tmat) + ((int64_t)cg * H + h) * 16384;
#pragma unroll
  for (int j = 0; j < 16; ++j)
    *reinterpret_cast<uint4 *>(dst + 1024 * j + 16 * lane) =
        *reinterpret_cast<const uint4 *>(stage + 1024 * j + 16 * lane);
}

hipError_t launch_bwd_tm(const BwdArgs &b, float *tmat, int64_t max_chunks, hipStream_t stream) {
  if (max_chunks <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_tm_kernel, dim3((unsigned)max_chunks, b.H), dim3(64), 0, stream, b, tmat);
  return hipGetLastError();
}

hipError_t launch_bwd_chain_bf16(const BwdArgs &b, const BwdUnits &u, hipStream_t stream) {
  const int64_t units = u.L > 0 ? u.units : b.N;
  if (units <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_chain_bf16_kernel<false>, dim3((unsigned)units, b.H), dim3(kThreads), 0,
                     stream, b, u);
  return hipGetLastError();
}

hipError_t launch_bwd_chain_bf16_transition(const BwdArgs &b, const BwdUnits &u,
                                            hipStream_t stream) {
  if (u.units <= 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_chain_bf16_kernel<true>, dim3((unsigned)u.units, b.H), dim3(kThreads), 0,
                     stream, b, u);
  return hipGetLastError();
}

}  // namespace gdn
