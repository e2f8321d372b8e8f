// Forward of the chunked gated delta rule for bf16 inputs with d_k = d_v = 128 on gfx950: a
// warp-specialised pipeline.
//
// The method is the chunked form of "How to Speed Up GDN Kernels for Qwen Models" (sections
// "What GDN actually computes", "Lever 1", "Lever 2"): per 64-token chunk, gamma = cumsum(g),
// A = strict_lower(diag(beta) (K K^T o e^{gamma_r - gamma_i})), Tm = (I + A)^-1, the state chain
// and the output.  The residual form of Delta is used (same quantity as U - W h):
//     R = diag(beta) (V - diag(e^gamma) K h),   Delta = Tm R.
//
// Work split.  Everything that does not depend on the state (the gate vectors, A, the inverse,
// P = (Q K^T) o decay o mask) is "prep"; the rest (K h, Delta, the output, the state update) is
// the "chain".  A workgroup has eight waves: waves 0-3 run the chain, wave w owning state columns
// [32 w, 32 w + 32); waves 4-7 prep chunk c + 1 while the chain runs chunk c, and wave 7 streams
// chunk c + 2's K and Q from HBM into LDS with direct global->LDS loads.  One barrier per chunk
// hands the prepared chunk over; chain waves never wait for each other (each owns its columns of
// the state, of V and of the output).
//
// Delta by block forward substitution.  With Tm = [[T_TL, 0], [T_BL, T_BR]] over 32-token halves,
//     Delta_T = T_TL R_T,   Delta_B = T_BR (R_B - A_BL Delta_T),
// so prep only inverts the two 32x32 diagonal blocks (four 16x16 inverses by substitution on one
// wave, then Tm_10 = -T_11 A_10 T_00 and Tm_32 = -T_33 A_32 T_22 with fp32 MFMA) and never forms
// T_BL; the chain spends the same number of MFMAs as with the full Tm.
//
// The output is formed transposed, O^T = e^gamma-scaled (S^T Q^T) + Delta^T P^T, so each lane
// holds 4 consecutive state columns of one token and writes them with one 8-byte store.
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_tiles.h"
#include "gdn_unit.h"

namespace gdn {
namespace {

constexpr int kD = 128;

// 64 x 128 bf16 tiles (K, Q, V): rows of 256 bytes; the 16-byte unit c of row r is stored at unit
// c ^ sw(r).  For the reads below (16 lanes on one 8-byte unit of 16 consecutive rows, or
// transpose reads of 4 consecutive 8-byte units of 8 consecutive rows) each half-wave touches
// 32 distinct 8-byte bank pairs.
__device__ __forceinline__ int sw(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
// element offset of the 8-byte unit u (elements 4u .. 4u + 3) of row r
__device__ __forceinline__ int toff(int r, int u) {
  return r * kD + (((u >> 1) ^ sw(r)) << 3) + ((u & 1) << 2);
}
// 32 x 32 bf16 blocks (T_TL, T_BR, -A_BL): rows of 64 bytes, unit u of row r at u ^ 2 ((r/4) % 4)
__device__ __forceinline__ int boff(int r, int u) { return r * 32 + ((u ^ (((r >> 2) & 3) << 1)) << 2); }
// 64 x 64 bf16 P: rows of 128 bytes, unit u of row r at u ^ 2 ((r/2) % 8)
__device__ __forceinline__ int poff(int r, int u) { return r * 64 + ((u ^ (((r >> 1) & 7) << 1)) << 2); }

constexpr int LA = 20;        // fp32 row stride of the 16x16 solve blocks
constexpr int AB = 16 * LA + 16;  // fp32 stride between solve blocks (spreads blocks over banks)

struct WsSmem {
  struct Vec {
    alignas(16) float beta[64];
    alignas(16) float eg[64];   // e^gamma
    alignas(16) float edt[64];  // e^(gamma_last - gamma)
    alignas(16) float gam[64];
    alignas(16) float egl[4];   // e^gamma_last
  };
  alignas(16) bf16 kq[3][2][64 * kD];  // [set][K, Q], three chunks in flight
  alignas(16) bf16 v[64 * kD];         // V of the chunk on the chain (each chain wave its columns)
  alignas(16) bf16 tb[2][3][32 * 32];  // [set][T_TL, T_BR, -A_BL]
  alignas(16) bf16 p[2][64 * 64];      // [set] P
  Vec vec[2];
  alignas(16) float at[4 * AB];  // A_bb transposed (row i = column i of A_bb), wave 4 only
  alignas(16) float ao[2 * AB];  // A_10, A_32 row-major, wave 4 only
  alignas(16) float tt[4 * AB];  // T_bb row-major, wave 4 only
  alignas(16) int imisc[4];
};
static_assert(sizeof(WsSmem) <= 160 * 1024, "LDS budget");

__device__ __forceinline__ bf16x4 ld4(const bf16 *p) { return lds_bf16x4(p); }
__device__ __forceinline__ void st4(bf16 *p, f32x4 x) {
  *reinterpret_cast<bf16x4 *>(p) = to_bf16x4(x);
}

// 16 direct global->LDS loads of 16 bytes per lane (one wave): a 64 x 128 bf16 tile of token
// rows t0 .. t0 + 63 (rows past the chunk's n tokens repeat its last token) into the swizzled
// layout.  Instruction j fills LDS rows 4j .. 4j + 3; lane l writes physical unit l % 16 of row
// 4j + l / 16, which holds logical unit (l % 16) ^ sw(row).
__device__ __forceinline__ void dma_tile(bf16 *dst, const bf16 *__restrict__ src, int64_t t0,
                                         int n, int h, int H, int lane) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = 4 * j + (lane >> 4);
    const int c = (lane & 15) ^ sw(r);
    const int64_t t = t0 + min(r, n - 1);
    __builtin_amdgcn_global_load_lds(src + (t * H + h) * kD + 8 * c,
                                     (GDN_LDS void *)(dst + 512 * j), 16, 0, 0);
  }
}

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Fragment reads, 8 bytes per lane each (g = lane / 16, l = lane % 16 of the reading lane).
// kfrag: elements 32 ks + 4 g .. +3 and 32 ks + 16 + 4 g .. +3 of a 128-wide tile row -- the
// k-order of a pair of D-layout accumulators used as the other operand.
__device__ __forceinline__ bf16x8 kfrag(const bf16 *t, int row, int ks, int g) {
  return cat8(ld4(t + toff(row, 8 * ks + g)), ld4(t + toff(row, 8 * ks + 4 + g)));
}
// the same k-order over a row of a 32-wide block or of the 64-wide P
__device__ __forceinline__ bf16x8 bfrag(const bf16 *t, int row, int g) {
  return cat8(ld4(t + boff(row, g)), ld4(t + boff(row, 4 + g)));
}
__device__ __forceinline__ bf16x8 pfrag(const bf16 *t, int row, int ks, int g) {
  return cat8(ld4(t + poff(row, 8 * ks + g)), ld4(t + poff(row, 8 * ks + 4 + g)));
}
// transpose read of a 128-wide tile: rows rowbase .. rowbase + 3 of column colbase + l
__device__ __forceinline__ bf16x4 trfrag(const bf16 *t, int rowbase, int colbase, int l) {
  return lds_tr16(t + toff(rowbase + (l >> 2), (colbase >> 2) + (l & 3)));
}
// The lane index as an opaque value: address arithmetic derived from it is formed where it is
// used instead of being hoisted out of the chunk loop (which would hold ~50 address registers).
__device__ __forceinline__ int fresh_lane(int lane) {
  asm volatile("" : "+v"(lane));
  return lane;
}

}  // namespace

__global__ __launch_bounds__(512) void fwd_ws_kernel(FwdArgs a) {
  __shared__ WsSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 4, cl = lane & 15;
  // wave-uniform role (scalar branches: a wave never steps through the other role's barriers)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int unit = blockIdx.x, h = blockIdx.y, H = a.H;
  if (wave == 0) {
    Unit un;
    const bool ok = find_unit(a.cu, a.N, a.L, unit, false, lane, un);
    if (lane == 0) {
      sm.imisc[0] = ok ? un.seq : -1;
      sm.imisc[1] = un.c0;
      sm.imisc[2] = un.c1;
    }
  }
  __syncthreads();
  const int seq = __builtin_amdgcn_readfirstlane(sm.imisc[0]);
  if (seq < 0) return;
  const int c0 = __builtin_amdgcn_readfirstlane(sm.imisc[1]);
  const int c1 = __builtin_amdgcn_readfirstlane(sm.imisc[2]);
  const int64_t ts0 = a.cu[seq], ts1 = a.cu[seq + 1];
  if (ts0 < 0 || ts1 < ts0 || ts1 > a.T) return;  // malformed cu_seqlens: touch nothing
  const int nchunks_seq = (int)((ts1 - ts0 + kChunk - 1) / kChunk);
  const bf16 *__restrict__ gq_ = static_cast<const bf16 *>(a.q);
  const bf16 *__restrict__ gk_ = static_cast<const bf16 *>(a.k);
  const bf16 *__restrict__ gv_ = static_cast<const bf16 *>(a.v);
  const bf16 *__restrict__ gb_ = static_cast<const bf16 *>(a.beta);
  bf16 *__restrict__ go_ = static_cast<bf16 *>(a.o);

  // Parts the chain reads but prep never writes: the upper-right 16x16 blocks of T_TL and T_BR,
  // and P's tiles (0, 1) and (2, 3) above the diagonal.
  for (int i = tid; i < 2 * 2 * 256; i += 512) {
    const int set = i >> 9, blk = (i >> 8) & 1, e = i & 255, r = e >> 4, c = 16 + (e & 15);
    sm.tb[set][blk][boff(r, c >> 2) + (c & 3)] = (bf16)0.f;
  }
  for (int i = tid; i < 2 * 2 * 256; i += 512) {
    const int set = i >> 9, t = (i >> 8) & 1, e = i & 255;
    const int r = 32 * t + (e >> 4), c = 32 * t + 16 + (e & 15);
    sm.p[set][poff(r, c >> 2) + (c & 3)] = (bf16)0.f;
  }

  int cw = c0;
  if (a.truncate && c0 > 0) {
    __syncthreads();  // every wave has read the unit
    if (wave == 0) {
      const int w = warm_window(a.g, ts0, c0, h, H, a.log_thr, lane);
      if (lane == 0) sm.imisc[0] = w;
    }
    __syncthreads();
    cw = __builtin_amdgcn_readfirstlane(sm.imisc[0]);
  }

  auto chunk_t0 = [&](int c) { return ts0 + (int64_t)c * kChunk; };
  auto chunk_n = [&](int c) { return (int)min<int64_t>(kChunk, ts1 - chunk_t0(c)); };

  const bool is_chain = wave < 4;
  const int w = wave & 3;

  if (is_chain) {
    // ======================= chain waves: the state recurrence and the output =======================
    const int ncol = 32 * w;  // this wave's first state column
    // S[mt][nt] holds rows 16 mt + 4 gq + i, column ncol + 16 nt + cl
    f32x4 S[8][2];
    if (cw == 0 && a.h0 != nullptr) {
      const float *hp = a.h0 + (int64_t)seq * a.h0_stride + (int64_t)h * kD * kD;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            S[mt][nt][i] = hp[(16 * mt + 4 * gq + i) * kD + ncol + 16 * nt + cl];
      // consume the loads here, so that no wait for them is left inside the chunk loop
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) asm volatile("" : "+v"(S[mt][nt]));
    } else {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) S[mt][0] = S[mt][1] = zero4();
    }
    // V rows of chunk c for this wave's columns (16-byte units; rows past n repeat the chunk's last
    // token), and their store into the swizzled V tile
    struct VRows {
      uint4 x[4];
    };
    auto v_load = [&](int c) {
      const int64_t t0 = chunk_t0(c);
      const int n = chunk_n(c);
      VRows vp;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * j + (lane >> 2);
        const int64_t t = t0 + min(r, n - 1);
        vp.x[j] = *reinterpret_cast<const uint4 *>(gv_ + (t * H + h) * kD + ncol + 8 * (lane & 3));
      }
      return vp;
    };
    auto v_store = [&](const VRows &vp) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * j + (lane >> 2), c = 4 * w + (lane & 3);
        *reinterpret_cast<uint4 *>(&sm.v[r * kD + ((c ^ sw(r)) << 3)]) = vp.x[j];
      }
    };
    // the state as bf16 operand fragments, in the k-order of kfrag
    auto state_frags = [&](bf16x8(&sb)[4][2]) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) sb[ks][nt] = to_bf16x8(S[2 * ks][nt], S[2 * ks + 1][nt]);
    };

    // V of the first chunk goes to LDS now; the next chunk's V is held in registers until the
    // first chunk's residual has consumed the V tile (loads run one chunk ahead of their store).
    // The loads and stores are unconditional (past the unit's last chunk they repeat it, and
    // rewriting a V tile with its own contents is harmless), so no wait is placed on them
    // anywhere but at the store.
    VRows vp{};
    if (cw < c1) v_store(v_load(cw));
    wait_vm0();  // the initial state is in registers: no load is outstanding when the loop starts
    if (cw < c1) vp = v_load(min(cw + 1, c1 - 1));
    __syncthreads();  // chunk cw's K and Q are in LDS (prep waves)

    for (int c = cw; c <= c1; ++c) {
      if (c > cw) {
        // ---------------- chunk cc = c - 1 (prepared during the previous step) ----------------
        const int cc = c - 1;
        const int64_t t0 = chunk_t0(cc);
        const int n = chunk_n(cc);
        const bool emit = cc >= c0;
        const int Y = cc & 1;
        const bf16 *Kt = sm.kq[cc % 3][0], *Qt = sm.kq[cc % 3][1];
        const WsSmem::Vec &vc = sm.vec[Y];

        // ---- K h, then the residual R = diag(beta) (V - diag(e^gamma) K h), fp32
        f32x4 R[4][2];
        {
          const int ln = fresh_lane(lane), lg = ln >> 4, lc = ln & 15;
          bf16x8 sb[4][2];
          state_frags(sb);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) R[mt][0] = R[mt][1] = zero4();
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
              const bf16x8 af = kfrag(Kt, 16 * mt + lc, ks, lg);
#pragma unroll
              for (int nt = 0; nt < 2; ++nt) R[mt][nt] = mma_bf16(af, sb[ks][nt], R[mt][nt]);
            }
        }
        sched_fence();
        {
        const int ln = fresh_lane(lane), lg = ln >> 4, lc = ln & 15;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const f32x4 be = lds_f32x4(&vc.beta[16 * mt + 4 * gq]);
          const f32x4 ee = lds_f32x4(&vc.eg[16 * mt + 4 * gq]);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            const bf16x4 v4 = trfrag(sm.v, 16 * mt + 4 * lg, ncol + 16 * nt, lc);
#pragma unroll
            for (int i = 0; i < 4; ++i) R[mt][nt][i] = be[i] * ((float)v4[i] - ee[i] * R[mt][nt][i]);
          }
        }
        }
        v_store(vp);  // chunk cc + 1's V (this wave's columns of chunk cc are consumed)
        sched_fence();

        // ---- Delta_T = T_TL R_T;  R_B -= A_BL Delta_T;  Delta_B = T_BR R_B.  Delta is kept only
        //      as bf16 operand fragments: da for the output, dt = Delta o e^{gamma_last - gamma}
        //      for the state update (both in the k-order of kfrag over tokens)
        bf16x8 da[2][2], dt[2][2];
        {
          const int ln = fresh_lane(lane), lg = ln >> 4, lc = ln & 15;
          const bf16 *TL = sm.tb[Y][0], *BR = sm.tb[Y][1], *NA = sm.tb[Y][2];
          f32x4 Dl[2][2];
          bf16x8 rb[2];
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) rb[nt] = to_bf16x8(R[0][nt], R[1][nt]);
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            const bf16x8 af = bfrag(TL, 16 * mt + lc, lg);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) Dl[mt][nt] = mma_bf16(af, rb[nt], zero4());
          }
          const f32x4 e00 = lds_f32x4(&vc.edt[4 * gq]), e01 = lds_f32x4(&vc.edt[16 + 4 * gq]);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            da[0][nt] = to_bf16x8(Dl[0][nt], Dl[1][nt]);
            dt[0][nt] = to_bf16x8(Dl[0][nt] * e00, Dl[1][nt] * e01);
          }
#pragma unroll
          for (int mt = 2; mt < 4; ++mt) {
            const bf16x8 af = bfrag(NA, 16 * (mt - 2) + lc, lg);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) R[mt][nt] = mma_bf16(af, da[0][nt], R[mt][nt]);
          }
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) rb[nt] = to_bf16x8(R[2][nt], R[3][nt]);
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            const bf16x8 af = bfrag(BR, 16 * mt + lc, lg);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) Dl[mt][nt] = mma_bf16(af, rb[nt], zero4());
          }
          const f32x4 e10 = lds_f32x4(&vc.edt[32 + 4 * gq]), e11 = lds_f32x4(&vc.edt[48 + 4 * gq]);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            da[1][nt] = to_bf16x8(Dl[0][nt], Dl[1][nt]);
            dt[1][nt] = to_bf16x8(Dl[0][nt] * e10, Dl[1][nt] * e11);
          }
        }

        sched_fence();
        // ---- output, transposed: O^T = scale (e^gamma (S^T Q^T) + Delta^T P^T)
        if (emit) {
          const bf16 *P = sm.p[Y];
          bf16x8 sb[4][2];
          state_frags(sb);
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const int ln = fresh_lane(lane), lg = ln >> 4, lc = ln & 15;
            const int t = 16 * tt + cl;
            bf16x8 qf[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) qf[ks] = kfrag(Qt, 16 * tt + lc, ks, lg);
            bf16x8 pf[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
              if (ks <= (tt >> 1)) pf[ks] = pfrag(P, 16 * tt + lc, ks, lg);
            const float et = vc.eg[t];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
              f32x4 acc = zero4();
#pragma unroll
              for (int ks = 0; ks < 4; ++ks) acc = mma_bf16(sb[ks][nt], qf[ks], acc);
              acc *= et;
#pragma unroll
              for (int ks = 0; ks < 2; ++ks)
                if (ks <= (tt >> 1)) acc = mma_bf16(da[ks][nt], pf[ks], acc);
              acc *= a.scale;
              if (t < n)
                *reinterpret_cast<bf16x4 *>(go_ + ((t0 + t) * H + h) * kD + ncol + 16 * nt + 4 * gq) =
                    to_bf16x4(acc);
            }
            sched_fence();
          }
        }

        vp = v_load(min(cc + 2, c1 - 1));
        sched_fence();

        // ---- state update: h <- e^{gamma_last} h + K^T diag(e^{gamma_last - gamma}) Delta
        {
          const float egl = vc.egl[0];
#pragma unroll
          for (int mt = 0; mt < 8; ++mt) {
            const int ln = fresh_lane(lane), lg = ln >> 4, lc = ln & 15;
            const bf16x8 a0 = cat8(trfrag(Kt, 4 * lg, 16 * mt, lc), trfrag(Kt, 16 + 4 * lg, 16 * mt, lc));
            const bf16x8 a1 = cat8(trfrag(Kt, 32 + 4 * lg, 16 * mt, lc), trfrag(Kt, 48 + 4 * lg, 16 * mt, lc));
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
              S[mt][nt] = mma_bf16(a1, dt[1][nt], mma_bf16(a0, dt[0][nt], S[mt][nt] * egl));
            if (mt & 1) sched_fence();
          }
        }
      }
      __syncthreads();
    }

    if (a.ht != nullptr && c1 == nchunks_seq) {
      float *dst = a.ht + ((int64_t)seq * H + h) * kD * kD;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            dst[(16 * mt + 4 * gq + i) * kD + ncol + 16 * nt + cl] = S[mt][nt][i];
    }
  } else if (wave == 7) {
    // ======================= wave 7: K and Q from HBM into LDS, one chunk ahead =====================
    // (it issues no other LDS instruction, so nothing waits on these loads before the barrier)
    if (cw < c1) {
      dma_tile(sm.kq[cw % 3][0], gk_, chunk_t0(cw), chunk_n(cw), h, H, lane);
      if (cw >= c0) dma_tile(sm.kq[cw % 3][1], gq_, chunk_t0(cw), chunk_n(cw), h, H, lane);
    }
    wait_vm0();
    __syncthreads();
    for (int c = cw; c <= c1; ++c) {
      if (c + 1 < c1) {
        dma_tile(sm.kq[(c + 1) % 3][0], gk_, chunk_t0(c + 1), chunk_n(c + 1), h, H, lane);
        if (c + 1 >= c0)
          dma_tile(sm.kq[(c + 1) % 3][1], gq_, chunk_t0(c + 1), chunk_n(c + 1), h, H, lane);
      }
      wait_vm0();  // chunk c + 1's K and Q are in LDS before the barrier that hands them over
      __syncthreads();
    }
  } else {
    // ======================= waves 4-6: everything else that does not need the state ===============
    // g and beta of this lane's token in chunk c, loaded one chunk ahead as raw values (the
    // address is clamped to the chunk, so the loads are unconditional and never waited on early);
    // gb_value masks lanes past the chunk's end and converts
    struct GB {
      float g;
      unsigned short b;
    };
    auto gb_load = [&](int c) {
      const int64_t t = chunk_t0(c) + min(lane, chunk_n(c) - 1);
      GB x;
      x.g = a.g[t * H + h];
      x.b = reinterpret_cast<const unsigned short *>(gb_)[t * H + h];
      return x;
    };
    auto gb_value = [&](const GB &x, int n, float &gv, float &bv) {
      gv = lane < n ? x.g : 0.f;
      bv = lane < n ? __uint_as_float((unsigned)x.b << 16) : 0.f;
    };
    GB gbx{0.f, 0};
    if (cw < c1) gbx = gb_load(cw);
    __syncthreads();

    for (int c = cw; c <= c1; ++c) {
      if (c < c1) {
        // ---------------- chunk c ----------------
        const int n = chunk_n(c);
        const bool emit = c >= c0, more = c + 1 < c1;
        const int Y = c & 1;
        const bf16 *Kt = sm.kq[c % 3][0], *Qt = sm.kq[c % 3][1];
        float gv, bv;
        gb_value(gbx, n, gv, bv);
        if (more) gbx = gb_load(c + 1);
        const float gam = wave_inclusive_scan(gv, lane);
        const float gl = __shfl(gam, n - 1, 64);
        if (wave == 4) {
          // ---- gate vectors for the chain
          WsSmem::Vec &vc = sm.vec[Y];
          vc.beta[lane] = bv;
          vc.eg[lane] = __expf(gam);
          vc.edt[lane] = __expf(gl - gam);
          vc.gam[lane] = gam;
          if (lane == 0) vc.egl[0] = __expf(gl);
          // ---- A's diagonal 16x16 blocks (stored transposed) and A_10, A_32 (row-major), fp32
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int b0 = 2 * half, b1 = b0 + 1;
            f32x4 a00 = zero4(), a10 = zero4(), a11 = zero4();
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
              const bf16x8 f0 = kfrag(Kt, 16 * b0 + cl, ks, gq), f1 = kfrag(Kt, 16 * b1 + cl, ks, gq);
              a00 = mma_bf16(f0, f0, a00);
              a10 = mma_bf16(f1, f0, a10);
              a11 = mma_bf16(f1, f1, a11);
            }
            const f32x4 gr0 = lds_f32x4(&vc.gam[16 * b0 + 4 * gq]);
            const f32x4 br0 = lds_f32x4(&vc.beta[16 * b0 + 4 * gq]);
            const f32x4 gr1 = lds_f32x4(&vc.gam[16 * b1 + 4 * gq]);
            const f32x4 br1 = lds_f32x4(&vc.beta[16 * b1 + 4 * gq]);
            const float gi0 = vc.gam[16 * b0 + cl], gi1 = vc.gam[16 * b1 + cl];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int rl = 4 * gq + e;
              a00[e] = cl < rl ? br0[e] * __expf(gr0[e] - gi0) * a00[e] : 0.f;
              a11[e] = cl < rl ? br1[e] * __expf(gr1[e] - gi1) * a11[e] : 0.f;
              a10[e] = br1[e] * __expf(gr1[e] - gi0) * a10[e];
            }
            *reinterpret_cast<f32x4 *>(&sm.at[b0 * AB + cl * LA + 4 * gq]) = a00;
            *reinterpret_cast<f32x4 *>(&sm.at[b1 * AB + cl * LA + 4 * gq]) = a11;
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.ao[half * AB + (4 * gq + e) * LA + cl] = a10[e];
          }
          // ---- the four diagonal inverses by substitution: lane (block gq, column cl)
          {
            const float *ab = &sm.at[gq * AB];
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = r == cl ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < 15; ++i) {
              float col[16];
#pragma unroll
              for (int q = (i + 1) >> 2; q < 4; ++q) {
                const f32x4 v4 = lds_f32x4(ab + i * LA + 4 * q);
#pragma unroll
                for (int e = 0; e < 4; ++e) col[4 * q + e] = v4[e];
              }
#pragma unroll
              for (int r = i + 1; r < 16; ++r) x[r] -= col[r] * x[i];
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.tt[gq * AB + r * LA + cl] = x[r];
          }
          // ---- T_bb as bf16 into T_TL / T_BR: 4 rows of 4 columns per lane
#pragma unroll
          for (int it = 0; it < 4; ++it) {
            const int idx = lane + 64 * it, b = idx >> 6, r = (idx >> 2) & 15, qd = idx & 3;
            const f32x4 t4 = lds_f32x4(&sm.tt[b * AB + r * LA + 4 * qd]);
            st4(&sm.tb[Y][b >> 1][boff(16 * (b & 1) + r, 4 * (b & 1) + qd)], t4);
          }
          // ---- Tm_10 = -T_11 (A_10 T_00), Tm_32 = -T_33 (A_32 T_22), fp32 MFMA
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int b = 2 * q + 1, cb = 2 * q;
            f32x4 X = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s)
              X = mma_f32(sm.ao[q * AB + cl * LA + 4 * s + gq], sm.tt[cb * AB + (4 * s + gq) * LA + cl], X);
            f32x4 out = zero4();
#pragma unroll
            for (int e = 0; e < 4; ++e) out = mma_f32(sm.tt[b * AB + cl * LA + 4 * gq + e], X[e], out);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              sm.tb[Y][q][boff(16 + 4 * gq + e, cl >> 2) + (cl & 3)] = (bf16)(-out[e]);
          }
        } else {
          // ---- waves 5 and 6: the tiles of -A below the diagonal 32x32 blocks and P as bf16,
          //      formed transposed (lane (row r, group) holds 4 consecutive columns i of row r);
          //      wave 5 takes column blocks 0 and 3, wave 6 blocks 1 and 2 (7 tiles each)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int bj = wave == 5 ? 3 * jj : 1 + jj;
            bf16x8 fa[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) fa[ks] = kfrag(Kt, 16 * bj + cl, ks, gq);
            f32x4 gi;
#pragma unroll
            for (int e = 0; e < 4; ++e) gi[e] = __shfl(gam, 16 * bj + 4 * gq + e, 64);
            if (bj < 2) {
#pragma unroll
              for (int bi = 2; bi < 4; ++bi) {
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) acc = mma_bf16(fa[ks], kfrag(Kt, 16 * bi + cl, ks, gq), acc);
                const int r = 16 * bi + cl;
                const float gr = __shfl(gam, r, 64), br = __shfl(bv, r, 64);
                f32x4 val;
#pragma unroll
                for (int e = 0; e < 4; ++e) val[e] = -br * __expf(gr - gi[e]) * acc[e];
                st4(&sm.tb[Y][2][boff(r - 32, 4 * bj + gq)], val);
              }
            }
            if (emit) {
              for (int bi = bj; bi < 4; ++bi) {
                f32x4 acc = zero4();
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) acc = mma_bf16(fa[ks], kfrag(Qt, 16 * bi + cl, ks, gq), acc);
                const int r = 16 * bi + cl;
                const float gr = __shfl(gam, r, 64);
                f32x4 val;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  val[e] = (16 * bj + 4 * gq + e <= r) ? __expf(gr - gi[e]) * acc[e] : 0.f;
                st4(&sm.p[Y][poff(r, 4 * bj + gq)], val);
              }
            }
          }
        }
      }
      __syncthreads();
    }
  }
}

int fwd_ws_blocks_per_cu() {
  int blocks = 0;
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fwd_ws_kernel, 512, 0);
  return (e == hipSuccess && blocks > 0) ? blocks : 1;
}

hipError_t launch_fwd_ws(const FwdArgs &a, int64_t max_units, hipStream_t stream) {
  if (max_units <= 0) return hipSuccess;
  hipLaunchKernelGGL(fwd_ws_kernel, dim3((unsigned)max_units, a.H), dim3(512), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdn
