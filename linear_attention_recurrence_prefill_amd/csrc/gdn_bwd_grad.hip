// Per-chunk gradients of the backward for bf16 inputs with d_k = d_v = 128 on gfx950.
//
// Per chunk (n <= 64 tokens) and head, from the forward recompute (gamma, the chunk-start state
// h, Delta) and the reverse chain (dh' = gradient of the state after the chunk, dR = Tm^T dDelta
// = the gradient of R = diag(beta) (V - diag(a) K h), since Delta = Tm R; the chain also writes
// dV = diag(beta) dR), with a = e^gamma, c = e^{gamma_last - gamma}, Gm_ri = e^{gamma_r -
// gamma_i} (i <= r), dO_s = scale dO:
//   dA  = strict_lower(-dR Delta^T)         (gradient of A through Tm = (I + A)^-1)
//   dPm = (dO_s Delta^T) o Gm on i <= r;    E = dA o Gm o beta_row
//   Y1 = dO_s h^T,  Y2 = Delta dh'^T,  Rh = dR h^T
//   dQ = diag(a) Y1 + dPm K
//   dK = dPm^T Q + (E + E^T) K + diag(c) Y2 - diag(beta a) Rh
//   dbeta_r  = dR_r . V_r - a_r (Rh . K)_r + sum_i dA_ri Gm_ri (k_r . k_i)
//   dgamma_r = a_r (Y1 . Q)_r - beta_r a_r (Rh . K)_r - c_r (Y2 . K)_r
//              + row r minus column r sums of (dPm o Q K^T) and of (dA o A)
//   dgamma_last += sum_r c_r (Y2 . K)_r + e^{gamma_last} <dh', h>;  dg = reverse cumsum of dgamma
// ((x . y)_r is the dot product of row r of x and y.)  This is the reverse-mode derivative of the
// chunked form of "How to Speed Up GDN Kernels for Qwen Models" (section "What GDN actually
// computes"), with the hidden states recomputed ("Lever 2").
//
// One workgroup of eight waves per (chunk, head), the heads of a chunk in consecutive
// workgroups.  Products run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation; q, k, v and dO enter
// exactly, h and dh' as stored (bf16, as the forward takes h in its products), every other operand
// as a bf16 head plus a bf16 remainder (see the reverse chain).  Wave w owns feature columns [16 w,
// 16 w + 16) of every 64 x 128 result and takes its share of the 64 x 64 tiles; h and dh' go
// straight from HBM into the B operands of the wave that owns their rows.  Every reduction has a
// fixed owner and order, so results are bitwise reproducible.
#include "gdn_bwd_internal.h"
#include "gdn_device.h"

namespace gdn {
namespace {

constexpr int kD = 128;
constexpr int kRowB = kD * 2;
// Eight waves of 16 feature columns each (kNT = 1 column tile of 16 per wave): two waves per
// SIMD, so that one wave's latencies overlap the other's work.
constexpr int kWaves = 8;
constexpr int kNT = 8 / kWaves;
constexpr int kThreads = 64 * kWaves;

// 64 x 128 bf16 tiles, token-major, 16-byte unit c of row r at c ^ sw(r) (as in the chain)
__device__ __forceinline__ int sw(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
__device__ __forceinline__ int toff(int r, int u) {
  return r * kRowB + (((u >> 1) ^ sw(r)) << 4) + ((u & 1) << 3);
}
// 64 x 64 bf16 tiles (dPm, E): rows of 128 bytes, 8-byte unit u of row r at u ^ f(x), x =
// (r / 2) % 8 = (b2 b1 b0), f = 8 b1 + 4 (b0 ^ b2) + 2 b2.  Two rows of 128 bytes fill the 64
// banks.  Each access below then touches every bank pair once per half-wave: the row reads (16
// consecutive rows, one unit each: f's bits 3..1 differ over the 8 rows of one parity), the
// transposing reads (4 rows, 4 consecutive units each: f's bits 3..2 differ over the 4 rows of one
// parity, b2 being 0 there) and the 2-byte stores of a 16 x 16 block (4 rows two apart: bits 3..2
// differ over (b2, b1) with b0 fixed).
__device__ __forceinline__ int poff(int r, int u) {
  const int x = (r >> 1) & 7;
  const int f = ((x & 2) << 2) | (((x ^ (x >> 2)) & 1) << 2) | ((x >> 2) << 1);
  return r * 128 + ((u ^ f) << 3);
}

__device__ __forceinline__ bf16x4 ld8(const char *p) { return *reinterpret_cast<const bf16x4 *>(p); }
__device__ __forceinline__ bf16x8 ld16(const char *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ bf16x4 ldtr(const char *p) {
  return lds_tr16(reinterpret_cast<const bf16 *>(p));
}
__device__ __forceinline__ f32x4 to_f32x4(bf16x4 x) { return __builtin_convertvector(x, f32x4); }
// the four rows' totals of a value that row16_sum_dpp made uniform within each row, added in
// row order (a wave-uniform result).  Call it where every lane is active: it reads lanes 16, 32
// and 48 whatever the branch, and the compiler may sink the row sums' last adds into a branch
// taken by lane 0 alone.
__device__ __forceinline__ float wave_sum_rows(float x) {
  const int b = __float_as_int(x);
  return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) +
          __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(b, 32)) +
          __int_as_float(__builtin_amdgcn_readlane(b, 48)));
}
__device__ __forceinline__ void st_split(char *hi, char *lo, int off, float x) {
  const bf16 h = (bf16)x;
  *reinterpret_cast<bf16 *>(hi + off) = h;
  *reinterpret_cast<bf16 *>(lo + off) = (bf16)(x - (float)h);
}

struct GradSmem {
  alignas(16) char dout[64 * kRowB];
  alignas(16) char q[64 * kRowB];
  alignas(16) char k[64 * kRowB];
  // V; from the tile phase on, E hi and lo (lo 16 bytes past hi's end, so that reads of the two
  // at the same lane offset are not fused into one two-address read over the same banks)
  alignas(16) char v[64 * kRowB + 16];
  alignas(16) char dh[64 * kRowB];  // Delta = hi + lo
  alignas(16) char dl[64 * kRowB];
  alignas(16) char eh[64 * kRowB];  // dR = hi + lo
  alignas(16) char el[64 * kRowB];
  alignas(16) char tth[64 * 128];   // dPm = hi + lo
  alignas(16) char ttl[64 * 128];
  alignas(16) float gam[64], a[64], c[64], beta[64];
  alignas(16) float rq[64], rk[64];  // q/k L2 normalisation: inverse row norms (1 without)
  alignas(16) float prg[kWaves][64];  // per-wave partial row terms of dgamma (tiles)
  alignas(16) float pcg[kWaves][64];  // per-wave partial column terms of dgamma (tiles, subtracted)
  alignas(16) float prb[kWaves][64];  // per-wave partial row terms of dbeta (tiles)
  alignas(16) float frg[kWaves][64];  // per-wave row terms of dgamma over the wave's columns
  alignas(16) float frb[kWaves][64];  // per-wave row terms of dbeta over the wave's columns
  alignas(16) float fc[kWaves][64];   // per-wave c_r (Y2 . K)_r
  alignas(16) float hd[kWaves];
  alignas(16) int imisc[4];
};
static_assert(sizeof(GradSmem) <= 160 * 1024, "LDS budget");


}  // namespace

// kNorm: q and k were L2-normalised in the forward (b.rq, b.rk hold the inverse row norms).
template <bool kNorm>
__global__ __launch_bounds__(kThreads) void bwd_grad_bf16_kernel(BwdArgs b) {
  __shared__ GradSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 4, cl = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroup x = cg * H + h: the heads of a chunk are consecutive (their rows of the [T, H, d]
  // tensors interleave in memory and are read close together)
  const int H = b.H, h = (int)(blockIdx.x % (unsigned)H), cg = (int)(blockIdx.x / (unsigned)H);
  // locate the chunk: its sequence and its index within that sequence
  if (w == 0) {
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
  for (int i = tid; i < 6 * kWaves * 64; i += kThreads) (&sm.prg[0][0])[i] = 0.f;
  __syncthreads();
  // wave-uniform (read from LDS, which the compiler cannot tell): the addresses built from them
  // stay scalar, and the buffer resources of the stores below need no per-lane loop
  const int seq = __builtin_amdgcn_readfirstlane(sm.imisc[0]);
  if (seq < 0) return;
  const int64_t ts0 = b.cu[seq], ts1 = b.cu[seq + 1];
  if (ts0 < 0 || ts1 < ts0 || ts1 > b.T) return;
  const int64_t t0 = ts0 + (int64_t)__builtin_amdgcn_readfirstlane(sm.imisc[1]) * kChunk;
  const int n = (int)min<int64_t>(kChunk, ts1 - t0);
  const int64_t tok_bytes = (int64_t)H * kRowB;
  const int hk = h / (H / b.HK);                  // this value head's key head
  const int64_t tok_qk = (int64_t)b.HK * kRowB;   // stride of one token in q, k
  const int64_t dd = (int64_t)kD * kD;
  const float scale = b.scale;
  const bf16 *hS = reinterpret_cast<const bf16 *>(b.hc_b16) + ((int64_t)cg * H + h) * dd;
  const bf16 *dhn = reinterpret_cast<const bf16 *>(b.dhn_b16) + ((int64_t)cg * H + h) * dd;

  // ---- stage.  Every load is issued before any is waited for, h and dh' last: dO, Q, K, V into
  //      LDS through registers (rows past n repeat the chunk's last token, which every use
  //      masks), Delta and dR split into LDS (rows past n zero), and each wave's rows of h and
  //      dh' into registers for its B operands, where they stay in flight through the tile phase.
  const int fcol = 16 * kNT * w + cl;  // this lane's feature column in tile nt: fcol + 16 nt
  bf16x8 hh[kNT][4], gh[kNT][4];  // h and dh' rows fcol + 16 nt, elements 32 ks + 8 gq .. + 7
  {
    const char *src[4] = {static_cast<const char *>(b.dout), static_cast<const char *>(b.q),
                          static_cast<const char *>(b.k), static_cast<const char *>(b.v)};
    char *dst[4] = {sm.dout, sm.q, sm.k, sm.v};
    // wave w fills rows 8 w .. 8 w + 7; lane l of load j writes physical unit l % 16 of row
    // 8 w + 4 j + l / 16, which holds logical unit (l % 16) ^ sw(row).  Staged through registers,
    // not by direct global->LDS loads: with those outstanding the compiler waits for every load
    // before the first use of any, which would hold h and dh' (issued last) up at the barrier.
    f32x4 tv[4][16 / kWaves];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int j = 0; j < 16 / kWaves; ++j) {
        const int r = (64 / kWaves) * w + 4 * j + (lane >> 4);
        const bool qk = s == 1 || s == 2;  // q and k: the key head's rows
        tv[s][j] = *reinterpret_cast<const f32x4 *>(
            src[s] + (t0 + min(r, n - 1)) * (qk ? tok_qk : tok_bytes) +
            (int64_t)(qk ? hk : h) * kRowB + (((lane & 15) ^ sw(r)) << 4));
      }
    f32x4 xr[2][8 * 4 / kWaves];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float *g = s == 0 ? b.delta : b.ddelta;  // Delta, dR
#pragma unroll
      for (int m = 0; m < 8 * 4 / kWaves; ++m) {
        // branch-free: rows past n load the last row and are zeroed once they land (a load
        // under a branch would make the compiler wait for every load at the join)
        const int u = tid + kThreads * m, r = u >> 5, c4 = u & 31;
        xr[s][m] = *reinterpret_cast<const f32x4 *>(g + ((t0 + min(r, n - 1)) * H + h) * kD + 4 * c4);
      }
    }
    // the gates (every wave loads them, so that no load sits under a branch; wave 0 stores
    // them); lanes past n read the last token and are replaced below
    float rqv = 1.f, rkv = 1.f;
    const int64_t tl = t0 + min(lane, n - 1);
    const float gmv = b.gamma[tl * H + h];
    const unsigned short bbits = static_cast<const unsigned short *>(b.beta)[tl * H + h];
    if (kNorm) {
      rqv = b.rq[tl * b.HK + hk];
      rkv = b.rk[tl * b.HK + hk];
    }
    // h and dh' rows of this wave into registers, issued after every other load so that the
    // wait before the barrier below leaves them in flight: first used after the tile phase
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    sched_fence();
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int64_t off = (int64_t)(fcol + 16 * nt) * kD + 32 * ks + 8 * gq;
        hh[nt][ks] = *reinterpret_cast<const bf16x8 *>(hS + off);
        gh[nt][ks] = *reinterpret_cast<const bf16x8 *>(dhn + off);
      }
    sched_fence();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int j = 0; j < 16 / kWaves; ++j)
        *reinterpret_cast<f32x4 *>(dst[s] + ((64 / kWaves) * w + 4 * j) * kRowB + 16 * lane) =
            tv[s][j];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      char *hi = s == 0 ? sm.dh : sm.eh;
      char *lo = s == 0 ? sm.dl : sm.el;
#pragma unroll
      for (int m = 0; m < 8 * 4 / kWaves; ++m) {
        const int u = tid + kThreads * m, r = u >> 5, c4 = u & 31;
        const f32x4 x = r < n ? xr[s][m] : zero4();
        const bf16x4 xh = to_bf16x4(x);
        *reinterpret_cast<bf16x4 *>(hi + toff(r, c4)) = xh;
        *reinterpret_cast<bf16x4 *>(lo + toff(r, c4)) = to_bf16x4(x - to_f32x4(xh));
      }
    }
    if (w == 0) {  // lane n - 1 holds gamma_last
      const float glast = __shfl(gmv, n - 1, 64);
      const bool in = lane < n;
      sm.gam[lane] = in ? gmv : glast;
      sm.a[lane] = in ? __expf(gmv) : 0.f;
      sm.c[lane] = in ? __expf(glast - gmv) : 0.f;
      sm.beta[lane] = in ? __uint_as_float((unsigned)bbits << 16) : 0.f;
      sm.rq[lane] = in ? rqv : 1.f;
      sm.rk[lane] = in ? rkv : 1.f;
    }
  }
  __syncthreads();  // the loads of h and dh' may still be in flight

  // fragment readers
  // A or B operand over features, natural order: row r, elements 32 ks + 8 gq .. + 7
  auto rowf = [&](const char *t, int r, int ks) { return ld16(t + toff(r, 8 * ks + 2 * gq)); };
  // A operand over tokens from a 64 x 64 tile, rows 16 m + cl, tokens in the permuted order
  auto pfrag = [&](const char *t, int m, int ks) {
    const int r = 16 * m + cl;
    return cat8(ld8(t + poff(r, 8 * ks + gq)), ld8(t + poff(r, 8 * ks + 4 + gq)));
  };
  // the same from the transpose of a 64 x 64 tile (A[r][i] = t[i][r])
  auto ptfrag = [&](const char *t, int m, int ks) {
    const int i = 32 * ks + 4 * gq + (cl >> 2), u = 4 * m + (cl & 3);
    return cat8(ldtr(t + poff(i, u)), ldtr(t + poff(i + 16, u)));
  };
  // B operand over tokens from a 64 x 128 tile, column 4 u0 + cl, tokens in the permuted order
  auto trfrag = [&](const char *t, int ks, int u0) {
    const int r = 32 * ks + 4 * gq + (cl >> 2), u = u0 + (cl & 3);
    return cat8(ldtr(t + toff(r, u)), ldtr(t + toff(r + 16, u)));
  };
  // rows 16 m + 4 gq .. + 3 of column 4 u0 + cl of a 64 x 128 tile
  auto colv = [&](const char *t, int m, int u0) {
    return to_f32x4(ldtr(t + toff(16 * m + 4 * gq + (cl >> 2), u0 + (cl & 3))));
  };

  // ---- dR_r . V_r over this wave's columns (v)
  float rb[4][4];  // row terms of dbeta over this wave's columns: [mt][i]
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) rb[mt][i] = 0.f;
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const f32x4 vv = colv(sm.v, mt, 4 * kNT * w + 4 * nt);
      const f32x4 rr = colv(sm.eh, mt, 4 * kNT * w + 4 * nt) + colv(sm.el, mt, 4 * kNT * w + 4 * nt);
#pragma unroll
      for (int i = 0; i < 4; ++i) rb[mt][i] += rr[i] * vv[i];
    }
  }
  __syncthreads();  // every wave is done with V
  char *eth = sm.v, *etl = sm.v + 64 * 128 + 16;  // E = hi + lo
  // zero the tiles above the diagonal of dPm (tth, ttl) and E (v region)
  for (int i = tid; i < 6 * 64; i += kThreads) {
    const int t = i >> 6, rr = (i >> 2) & 15, u = i & 3;
    // (mi, mr) = (0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3): column block > row block
    const int mi = t < 3 ? 0 : (t < 5 ? 1 : 2);
    const int mr = t < 3 ? t + 1 : (t < 5 ? t - 1 : 3);
    const int off = poff(16 * mi + rr, 4 * mr + u);
    *reinterpret_cast<uint2 *>(&sm.tth[off]) = uint2{0u, 0u};
    *reinterpret_cast<uint2 *>(&sm.ttl[off]) = uint2{0u, 0u};
    *reinterpret_cast<uint2 *>(&sm.v[off]) = uint2{0u, 0u};
    *reinterpret_cast<uint2 *>(&etl[off]) = uint2{0u, 0u};
  }
  __syncthreads();

  // ---- 64 x 64 tiles on and below the diagonal: dP, dR Delta^T, Q K^T, K K^T
  for (int t = w; t < 10; t += kWaves) {
    int tr, ti;
    tri_tile(t, tr, ti);
    // the gates first, so that their LDS reads overlap the products
    const int i = 16 * ti + cl;
    const float gi = sm.gam[i], ki = sm.rk[i];
    const f32x4 gr = *reinterpret_cast<const f32x4 *>(&sm.gam[16 * tr + 4 * gq]);
    const f32x4 rqr = *reinterpret_cast<const f32x4 *>(&sm.rq[16 * tr + 4 * gq]);
    const f32x4 rkr = *reinterpret_cast<const f32x4 *>(&sm.rk[16 * tr + 4 * gq]);
    const f32x4 btr = *reinterpret_cast<const f32x4 *>(&sm.beta[16 * tr + 4 * gq]);
    f32x4 dp = zero4(), da = zero4(), qk = zero4(), kk = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int ra = 16 * tr + cl, rb_ = 16 * ti + cl;
      const bf16x8 ao = rowf(sm.dout, ra, ks), aq = rowf(sm.q, ra, ks), ak = rowf(sm.k, ra, ks);
      const bf16x8 arh = rowf(sm.eh, ra, ks), arl = rowf(sm.el, ra, ks);
      const bf16x8 bdh = rowf(sm.dh, rb_, ks), bdl = rowf(sm.dl, rb_, ks), bk = rowf(sm.k, rb_, ks);
      dp = mma_bf16(ao, bdh, dp);
      dp = mma_bf16(ao, bdl, dp);
      da = mma_bf16(arh, bdh, da);
      da = mma_bf16(arh, bdl, da);
      da = mma_bf16(arl, bdh, da);
      qk = mma_bf16(aq, bk, qk);
      kk = mma_bf16(ak, bk, kk);
    }
    float rg4[4], rb4[4], csc = 0.f;  // csc: this column's sum
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * tr + 4 * gq + j;
      // normalised q, k (factors 1 without): qk and kk of the normalised rows are rq_r rk_i qk
      // and rk_r rk_i kk; the stored tiles carry rq_r dPm rk_i and rk_r E rk_i, so that the
      // products below give rq dQ and rk dK of the normalised rows
      const float qs = rqr[j] * ki, ks2 = rkr[j] * ki;
      // branch-free: every term is formed and the masks select (above the diagonal the
      // exponential may overflow; the selects drop it)
      const bool on = i <= r && r < n, below = on && i < r;
      const float gm = __expf(gr[j] - gi);
      const float pm0 = scale * dp[j] * gm;
      const float dA = -da[j];
      const float gk = gm * (ks2 * kk[j]);
      const float pm = on ? pm0 : 0.f;
      const float e = below ? dA * gm * btr[j] : 0.f;
      const float tb = below ? dA * gk : 0.f;
      const float tg = (on ? pm0 * (qs * qk[j]) : 0.f) + (below ? dA * btr[j] * gk : 0.f);
      const int off = poff(r, i >> 2) + 2 * (i & 3);
      st_split(sm.tth, sm.ttl, off, qs * pm);
      st_split(eth, etl, off, ks2 * e);
      rg4[j] = tg;
      rb4[j] = tb;
      csc += tg;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      rg4[j] = row16_sum_dpp(rg4[j]);
      rb4[j] = row16_sum_dpp(rb4[j]);
    }
    csc += __shfl_xor(csc, 16, 64);
    csc += __shfl_xor(csc, 32, 64);
    if (cl == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sm.prg[w][16 * tr + 4 * gq + j] = rg4[j];
        sm.prb[w][16 * tr + 4 * gq + j] = rb4[j];
      }
    }
    if (gq == 0) sm.pcg[w][i] = csc;
  }
  // ---- h and dh' rows of this wave (bf16 B operands over features), <dh', h>
  f32x4 Y1[4][kNT], Y2[4][kNT];
  float hdot = 0.f;
  {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f32x4 h0 = to_f32x4(lo4(hh[nt][ks])), h1 = to_f32x4(hi4(hh[nt][ks]));
        const f32x4 d0 = to_f32x4(lo4(gh[nt][ks])), d1 = to_f32x4(hi4(gh[nt][ks]));
#pragma unroll
        for (int j = 0; j < 4; ++j) hdot += h0[j] * d0[j] + h1[j] * d1[j];
      }
    // Y1 = dO h^T (scale applied later), Y2 = Delta dh'^T
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) Y1[mt][nt] = Y2[mt][nt] = zero4();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 ao = rowf(sm.dout, 16 * mt + cl, ks);
        const bf16x8 ah = rowf(sm.dh, 16 * mt + cl, ks), al = rowf(sm.dl, 16 * mt + cl, ks);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          Y1[mt][nt] = mma_bf16(ao, hh[nt][ks], Y1[mt][nt]);
          Y2[mt][nt] = mma_bf16(ah, gh[nt][ks], Y2[mt][nt]);
          Y2[mt][nt] = mma_bf16(al, gh[nt][ks], Y2[mt][nt]);
        }
      }
    }
  }
  hdot = wave_sum_rows(row16_sum_dpp(hdot));  // at full exec: every lane's partial is formed
  if (lane == 0) sm.hd[w] = hdot;

  // ---- Rh = dR h^T over this wave's columns (d)
  f32x4 Rh[4][kNT];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) Rh[mt][nt] = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 ah = rowf(sm.eh, 16 * mt + cl, ks), al = rowf(sm.el, 16 * mt + cl, ks);
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        Rh[mt][nt] = mma_bf16(ah, hh[nt][ks], Rh[mt][nt]);
        Rh[mt][nt] = mma_bf16(al, hh[nt][ks], Rh[mt][nt]);
      }
    }
  }

  __syncthreads();

  // dq, dk of row r (this lane's rows 4 gq + r - r % 16 .. , column fcol) through buffer
  // resources whose range ends at the chunk's last token: rows at or past n are dropped by the
  // hardware, the row offset is a scalar operand and the lane's offset is one register.  Grouped
  // heads write fp32 partials, summed per key head afterwards.
  const bool part = b.dq_part != nullptr;
  const int64_t row0 = (t0 * H + h) * kD;
  const int es = part ? 4 : 2;
  const int rb_bytes = H * kD * es;  // one token
  const __amdgpu_buffer_rsrc_t rq_ = __builtin_amdgcn_make_buffer_rsrc(
      part ? (void *)(b.dq_part + row0) : (void *)(static_cast<bf16 *>(b.dq) + row0), (short)0,
      n * rb_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rk_ = __builtin_amdgcn_make_buffer_rsrc(
      part ? (void *)(b.dk_part + row0) : (void *)(static_cast<bf16 *>(b.dk) + row0), (short)0,
      n * rb_bytes, 0x00020000);
  const int vo = 4 * gq * rb_bytes + fcol * es;
  auto store_qk = [&](int r16, float dqv, float dkv) {  // r16 = 16 mt + i: the row less 4 gq
    const int so = r16 * rb_bytes;
    if (part) {
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dqv), rq_, vo, so, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dkv), rk_, vo, so, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (bf16)dqv), rq_, vo,
                                            so, 0);
      __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (bf16)dkv), rk_, vo,
                                            so, 0);
    }
  };

  // ---- dQ = diag(a) Y1 + dPm K;  dK = dPm^T Q + (E + E^T) K + diag(c) Y2 - diag(beta a) Rh
  float rg[4][4], rc[4][4];
  // normalised q, k: Z = rq dQ and W = rk dK of the normalised rows, held until the row dots
  // q_r . Z_r and k_r . W_r over all columns are known; then dq = Z - rq^2 q (q . Z) (likewise
  // dk), the normalisation's backward
  static_assert(kNT == 1, "one column tile per wave");
  constexpr bool norm = kNorm;
  float zq[4][4], zk[4][4], pq[4][4], pk[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) rg[mt][i] = rc[mt][i] = zq[mt][i] = zk[mt][i] = pq[mt][i] = pk[mt][i] = 0.f;
  {
    bf16x8 kb[2][kNT], qb[2][kNT];  // K and Q over tokens: [ks][nt]
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        kb[ks][nt] = trfrag(sm.k, ks, 4 * kNT * w + 4 * nt);
        qb[ks][nt] = trfrag(sm.q, ks, 4 * kNT * w + 4 * nt);
      }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 dq[kNT], dk[kNT];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) dq[nt] = dk[nt] = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bool lower = 2 * ks <= mt;      // blocks with tokens i <= rows r exist
        const bool upper = 2 * ks + 1 >= mt;  // blocks with tokens i >= rows r exist
        if (lower) {
          const bf16x8 ph = pfrag(sm.tth, mt, ks), pl = pfrag(sm.ttl, mt, ks);
          const bf16x8 eh_ = pfrag(eth, mt, ks), el_ = pfrag(etl, mt, ks);
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt) {
            dq[nt] = mma_bf16(ph, kb[ks][nt], dq[nt]);
            dq[nt] = mma_bf16(pl, kb[ks][nt], dq[nt]);
            dk[nt] = mma_bf16(eh_, kb[ks][nt], dk[nt]);
            dk[nt] = mma_bf16(el_, kb[ks][nt], dk[nt]);
          }
        }
        if (upper) {
          const bf16x8 ph = ptfrag(sm.tth, mt, ks), pl = ptfrag(sm.ttl, mt, ks);
          const bf16x8 eh_ = ptfrag(eth, mt, ks), el_ = ptfrag(etl, mt, ks);
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt) {
            dk[nt] = mma_bf16(ph, qb[ks][nt], dk[nt]);
            dk[nt] = mma_bf16(pl, qb[ks][nt], dk[nt]);
            dk[nt] = mma_bf16(eh_, kb[ks][nt], dk[nt]);
            dk[nt] = mma_bf16(el_, kb[ks][nt], dk[nt]);
          }
        }
      }
      const f32x4 ar = *reinterpret_cast<const f32x4 *>(&sm.a[16 * mt + 4 * gq]);
      const f32x4 cr0 = *reinterpret_cast<const f32x4 *>(&sm.c[16 * mt + 4 * gq]);
      const f32x4 br = *reinterpret_cast<const f32x4 *>(&sm.beta[16 * mt + 4 * gq]);
      // normalised q, k: every term of row r that carries q_r (k_r) takes rq_r (rk_r)
      const f32x4 rqr = *reinterpret_cast<const f32x4 *>(&sm.rq[16 * mt + 4 * gq]);
      const f32x4 rkr = *reinterpret_cast<const f32x4 *>(&sm.rk[16 * mt + 4 * gq]);
      const f32x4 aq = ar * rqr, ak = ar * rkr, cr = cr0 * rkr;
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const f32x4 qv = colv(sm.q, mt, 4 * kNT * w + 4 * nt), kv = colv(sm.k, mt, 4 * kNT * w + 4 * nt);
        const f32x4 y1 = scale * Y1[mt][nt];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float dqv = aq[i] * y1[i] + dq[nt][i];
          const float dkv = dk[nt][i] + cr[i] * Y2[mt][nt][i] - br[i] * ak[i] * Rh[mt][nt][i];
          if constexpr (norm) {
            zq[mt][i] = dqv;
            zk[mt][i] = dkv;
            pq[mt][i] += qv[i] * dqv;
            pk[mt][i] += kv[i] * dkv;
          } else {
            store_qk(16 * mt + i, dqv, dkv);
          }
          rg[mt][i] += aq[i] * y1[i] * qv[i] - br[i] * ak[i] * Rh[mt][nt][i] * kv[i] -
                       cr[i] * Y2[mt][nt][i] * kv[i];
          rb[mt][i] -= ak[i] * Rh[mt][nt][i] * kv[i];
          rc[mt][i] += cr[i] * Y2[mt][nt][i] * kv[i];
        }
      }
    }
  }
  // row sums over this wave's 16 columns per tile (the row dots of the normalisation go to the
  // dO tile's space, free since the tile phase)
  float *fq = reinterpret_cast<float *>(sm.dout), *fk = fq + kWaves * 64;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rg[mt][i] = row16_sum_dpp(rg[mt][i]);
      rb[mt][i] = row16_sum_dpp(rb[mt][i]);
      rc[mt][i] = row16_sum_dpp(rc[mt][i]);
      if constexpr (norm) {
        pq[mt][i] = row16_sum_dpp(pq[mt][i]);
        pk[mt][i] = row16_sum_dpp(pk[mt][i]);
      }
      if (cl == 0) {
        const int r = 16 * mt + 4 * gq + i;
        sm.frg[w][r] = rg[mt][i];
        sm.frb[w][r] = rb[mt][i];
        sm.fc[w][r] = rc[mt][i];
        if constexpr (norm) {
          fq[w * 64 + r] = pq[mt][i];
          fk[w * 64 + r] = pk[mt][i];
        }
      }
    }
  __syncthreads();
  if constexpr (norm) {  // dq = Z - rq^2 q (q . Z), dk = W - rk^2 k (k . W), summed over waves in order
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 tq = zero4(), tk = zero4();
#pragma unroll
      for (int x = 0; x < kWaves; ++x) {
        tq += *reinterpret_cast<const f32x4 *>(&fq[x * 64 + 16 * mt + 4 * gq]);
        tk += *reinterpret_cast<const f32x4 *>(&fk[x * 64 + 16 * mt + 4 * gq]);
      }
      const f32x4 qv = colv(sm.q, mt, 4 * kNT * w), kv = colv(sm.k, mt, 4 * kNT * w);
      const f32x4 rqr = *reinterpret_cast<const f32x4 *>(&sm.rq[16 * mt + 4 * gq]);
      const f32x4 rkr = *reinterpret_cast<const f32x4 *>(&sm.rk[16 * mt + 4 * gq]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        store_qk(16 * mt + i, zq[mt][i] - rqr[i] * rqr[i] * qv[i] * tq[i],
                 zk[mt][i] - rkr[i] * rkr[i] * kv[i] * tk[i]);
      }
    }
  }
  if (w == 0) {
    const int r = lane;
    float dgam = 0.f, dbet = 0.f, csum = 0.f;
#pragma unroll
    for (int x = 0; x < kWaves; ++x) {
      dgam += sm.prg[x][r] - sm.pcg[x][r] + sm.frg[x][r];
      dbet += sm.prb[x][r] + sm.frb[x][r];
      csum += sm.fc[x][r];
    }
    if (r >= n) {
      dgam = 0.f;
      csum = 0.f;
    }
    csum = wave_sum_rows(row16_sum_dpp(csum));
    float hdot = 0.f;
#pragma unroll
    for (int x = 0; x < kWaves; ++x) hdot += sm.hd[x];
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
      static_cast<bf16 *>(b.dbeta)[(t0 + r) * H + h] = (bf16)dbet;
    }
  }
}

hipError_t launch_bwd_grad_bf16(const BwdArgs &b, int64_t max_chunks, hipStream_t stream) {
  if (max_chunks <= 0) return hipSuccess;
  const int64_t wgs = max_chunks * b.H;
  if (wgs > (int64_t)UINT32_MAX) return hipErrorInvalidConfiguration;
  if (b.rq != nullptr)
    hipLaunchKernelGGL(bwd_grad_bf16_kernel<true>, dim3((unsigned)wgs), dim3(kThreads), 0, stream,
                       b);
  else
    hipLaunchKernelGGL(bwd_grad_bf16_kernel<false>, dim3((unsigned)wgs), dim3(kThreads), 0, stream,
                       b);
  return hipGetLastError();
}

}  // namespace gdn
