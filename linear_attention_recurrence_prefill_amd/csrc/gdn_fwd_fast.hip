// Forward of the chunked gated delta rule for bf16 inputs on gfx950.
//
// Same method as fwd_kernel (gdn_fwd.hip): gate cumsum, A = KK^T with beta and decay,
// Tm = (I + A)^-1, the state chain with the state held in MFMA accumulator registers, and the
// output ("How to Speed Up GDN Kernels for Qwen Models", sections "What GDN actually
// computes", "Lever 1", "Lever 2").  Two things change.
//
// The algebra of Delta: the WY form gives Delta = U - W h = Tm diag(beta) V - Tm
// diag(beta e^gamma) K h.  Here the triangular factor is applied to the residual directly,
//     R = diag(beta) (V - diag(e^gamma) K h),   Delta = Tm R,
// which is the same quantity with one 64x64xd product less per chunk (W and U are never
// formed), and one bf16 rounding of the residual instead of two of U and W h.
//
// The schedule (one workgroup of D/16 waves per (unit, head); wave w owns state columns
// [16 w, 16 w + 16)):
//   * two waves share each SIMD at d = 128, and every wave's state slice (16 columns) is small
//     enough that the whole chunk pipeline stays in registers without spilling;
//   * the next chunk's Q, K, V, g, beta are fetched into registers while the current chunk is
//     computed, then written to the second of two LDS buffer sets: the chain never waits on HBM;
//   * the inverse is formed recursively in place: the four 16x16 diagonal blocks by forward
//     substitution (one wave), the two 16x16 sub-diagonal blocks of the 32x32 halves
//     (Tm_10 = -Tm_11 A_10 Tm_00, Tm_32 = -Tm_33 A_32 Tm_22), then the lower-left 32x32 block
//     Tm_BL = -Tm_BR (A_BL Tm_TL); every A block is consumed before it is overwritten.  The
//     products that do not need Tm (K h and Q h, which share the state's bf16 fragments, and
//     P = (Q K^T) o decay) run on the waves the solve leaves idle;
//   * Q, K, V tiles are XOR-swizzled in LDS so every fragment read is free of bank conflicts;
//   * a chunk's O is staged in its V tile and written to HBM at the start of the next chunk.
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_tiles.h"
#include "gdn_unit.h"

namespace gdn {

// Q, K, V tiles are 64 x D bf16 without padding; 8-byte units are XOR-swizzled within each row
// (unit u of row r is stored at unit u ^ f(r), f(r) = 4 (r mod 4) + (r / 4 mod 4)).  Every
// fragment read in this kernel is 8 bytes per lane: 16 lanes reading one unit of 16 consecutive
// rows, or (transpose reads) 4 consecutive units of 4 consecutive rows, touch 16 distinct
// unit positions, i.e. all 32 banks once.
template <int D>
struct Swz {
  __device__ static __forceinline__ int f(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
  // element offset of 8-byte unit u (elements 4u .. 4u + 3) of row r
  __device__ static __forceinline__ int unit(int r, int u) { return r * D + 4 * (u ^ f(r)); }
  __device__ static __forceinline__ int elem(int r, int c) { return unit(r, c >> 2) + (c & 3); }
};

template <int D>
struct FastSmem {
  static constexpr int LDT = 64 + 4;  // fp32 row stride of A / Tm
  static constexpr int LDP = 64 + 8;  // bf16 row stride of P
  struct Buf {
    alignas(16) bf16 q[64 * D];
    alignas(16) bf16 k[64 * D];
    alignas(16) bf16 v[64 * D];    // V, then the chunk's O staged for the store
    alignas(16) float gam[64];     // within-chunk cumsum of g
    alignas(16) float beta[64];
    alignas(16) float eg[64];      // exp(gamma)
    alignas(16) float glast[4];
  };
  Buf buf[2];
  alignas(16) float at[64 * LDT];   // A, inverted in place into Tm
  alignas(16) bf16 p[64 * LDP];     // P = (Q K^T) o exp(gamma_r - gamma_i) [i <= r]
  alignas(16) float x[2][16 * 16];  // A_2c Tm_c-blocks, shared between waves during the solve
  alignas(16) int imisc[4];
};
static_assert(sizeof(FastSmem<128>) <= 160 * 1024, "LDS budget");

template <int D>
__global__ __launch_bounds__(64 * (D / 16)) void fwd_fast_kernel(FwdArgs a) {
  using SM = FastSmem<D>;
  using Buf = typename SM::Buf;
  using SW = Swz<D>;
  constexpr int LDT = SM::LDT, LDP = SM::LDP;
  constexpr int NW = D / 16;           // waves; wave w owns state columns [16 w, 16 w + 16)
  constexpr int NTH = 64 * NW;         // threads
  constexpr int MTD = D / 16;          // 16-row state tiles (d_k)
  constexpr int KSD = D / 32;          // 32-wide k-steps over d
  constexpr int UPR = D / 8;           // 16-byte units per bf16 row
  constexpr int UPT = 64 * UPR / NTH;  // units of one tile per thread
  __shared__ SM sm;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, gq = lane >> 4, cl = lane & 15;
  const int unit = blockIdx.x, h = blockIdx.y, H = a.H;
  if (wave == 0) {
    Unit un;
    const bool ok = find_unit(a.cu, a.N, a.T, a.L, unit, false, lane, un);
    if (lane == 0) {
      sm.imisc[0] = ok ? un.seq : -1;
      sm.imisc[1] = un.c0;
      sm.imisc[2] = un.c1;
    }
  }
  __syncthreads();
  const int seq = sm.imisc[0];
  if (seq < 0) return;
  const int c0 = sm.imisc[1], c1 = sm.imisc[2];
  const int64_t ts0 = a.cu[seq], ts1 = a.cu[seq + 1];
  if (ts0 < 0 || ts1 < ts0 || ts1 > a.T) return;  // malformed cu_seqlens: touch nothing
  const int nchunks_seq = (int)((ts1 - ts0 + kChunk - 1) / kChunk);
  const int hk = h / (H / a.HK);  // this value head's key head
  const bf16 *__restrict__ gq_ = static_cast<const bf16 *>(a.q);
  const bf16 *__restrict__ gk_ = static_cast<const bf16 *>(a.k);
  const bf16 *__restrict__ gv_ = static_cast<const bf16 *>(a.v);
  const bf16 *__restrict__ gb_ = static_cast<const bf16 *>(a.beta);
  bf16 *__restrict__ go_ = static_cast<bf16 *>(a.o);

  // Blocks above the diagonal of A/Tm and of P are never written by the chunk loop: zero once.
  for (int i = tid; i < 64 * 64; i += NTH) {
    const int r = i >> 6, c = i & 63;
    if ((c >> 4) > (r >> 4)) {
      sm.at[r * LDT + c] = 0.f;
      sm.p[r * LDP + c] = (bf16)0.f;
    }
  }

  int cw = c0;
  if (a.truncate && c0 > 0) {
    __syncthreads();  // every wave has read the unit
    if (wave == 0) {
      const int w = warm_window(a.g, ts0, c0, h, H, a.log_thr, lane);
      if (lane == 0) sm.imisc[0] = w;
    }
    __syncthreads();
    cw = sm.imisc[0];
  }

  const int ncol = 16 * wave;  // this wave's state columns
  f32x4 S[MTD];
  if (cw == 0 && a.h0 != nullptr) {
    const float *hp = a.h0 + (int64_t)seq * a.h0_stride + (int64_t)h * D * D;
#pragma unroll
    for (int mt = 0; mt < MTD; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) S[mt][i] = hp[(16 * mt + 4 * gq + i) * D + ncol + cl];
  } else {
#pragma unroll
    for (int mt = 0; mt < MTD; ++mt) S[mt] = zero4();
  }

  // ---- chunk inputs: fetched into registers, then written to an LDS buffer set
  uint4 pq[UPT], pk[UPT], pv[UPT];
  float pg = 0.f, pb = 0.f;
  auto fetch = [&](int c) {
    const bool em = c >= c0;
    const int64_t t0 = ts0 + (int64_t)c * kChunk;
    const int n = (int)min<int64_t>(kChunk, ts1 - t0);
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int u = tid + NTH * j, r = u / UPR, cu16 = u % UPR;
      pq[j] = pk[j] = pv[j] = uint4{0u, 0u, 0u, 0u};
      if (r < n) {
        const int64_t off = ((t0 + r) * H + h) * D + cu16 * 8;
        const int64_t off_qk = ((t0 + r) * a.HK + hk) * D + cu16 * 8;
        pk[j] = *reinterpret_cast<const uint4 *>(gk_ + off_qk);
        pv[j] = *reinterpret_cast<const uint4 *>(gv_ + off);
        if (em) pq[j] = *reinterpret_cast<const uint4 *>(gq_ + off_qk);
      }
    }
    if (wave == 0) {
      pg = lane < n ? a.g[(t0 + lane) * H + h] : 0.f;
      pb = lane < n ? (float)gb_[(t0 + lane) * H + h] : 0.f;
    }
  };
  // q/k L2 normalisation of one 16-byte unit of a row whose UPR units sit in UPR consecutive
  // lanes: the row's sum of squares by a butterfly over those lanes, then the unit scaled and
  // rounded back to bf16 (rows past the chunk's end are zero and stay zero)
  auto norm_unit = [&](uint4 &x) {
    unsigned wd[4] = {x.x, x.y, x.z, x.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(wd[i] << 16), hi = __uint_as_float(wd[i] & 0xFFFF0000u);
      s += lo * lo + hi * hi;
    }
#pragma unroll
    for (int off = 1; off < UPR; off <<= 1) s += __shfl_xor(s, off, 64);
    const float r = 1.f / sqrtf(s + kL2NormEps);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16 lo = (bf16)(r * __uint_as_float(wd[i] << 16));
      const bf16 hi = (bf16)(r * __uint_as_float(wd[i] & 0xFFFF0000u));
      wd[i] = (unsigned)__builtin_bit_cast(unsigned short, lo) |
              ((unsigned)__builtin_bit_cast(unsigned short, hi) << 16);
    }
    x = uint4{wd[0], wd[1], wd[2], wd[3]};
  };
  auto commit = [&](int c, Buf &B) {
    const bool em = c >= c0;
    const int64_t t0 = ts0 + (int64_t)c * kChunk;
    const int n = (int)min<int64_t>(kChunk, ts1 - t0);
    if (a.l2norm) {
#pragma unroll
      for (int j = 0; j < UPT; ++j) {
        norm_unit(pk[j]);
        if (em) norm_unit(pq[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int u = tid + NTH * j, r = u / UPR, cu16 = u % UPR;
      const int a0 = SW::unit(r, 2 * cu16), a1 = SW::unit(r, 2 * cu16 + 1);
      *reinterpret_cast<uint2 *>(&B.k[a0]) = uint2{pk[j].x, pk[j].y};
      *reinterpret_cast<uint2 *>(&B.k[a1]) = uint2{pk[j].z, pk[j].w};
      *reinterpret_cast<uint2 *>(&B.v[a0]) = uint2{pv[j].x, pv[j].y};
      *reinterpret_cast<uint2 *>(&B.v[a1]) = uint2{pv[j].z, pv[j].w};
      if (em) {
        *reinterpret_cast<uint2 *>(&B.q[a0]) = uint2{pq[j].x, pq[j].y};
        *reinterpret_cast<uint2 *>(&B.q[a1]) = uint2{pq[j].z, pq[j].w};
      }
    }
    if (wave == 0) {
      const float gam = wave_inclusive_scan(pg, lane);
      B.gam[lane] = gam;
      B.beta[lane] = pb;
      B.eg[lane] = __expf(gam);
      const float gl = __shfl(gam, n - 1, 64);
      if (lane == 0) B.glast[0] = gl;
    }
  };
  // Writes the O staged in B.v for the chunk that starts at o_t0.  It uses the thread -> unit
  // map of commit(), so a thread reads each O unit before it overwrites that unit with new V.
  auto store_o = [&](int64_t o_t0, int o_n, const Buf &B) {
#pragma unroll
    for (int j = 0; j < UPT; ++j) {
      const int u = tid + NTH * j, r = u / UPR, cu16 = u % UPR;
      if (r < o_n) {
        const uint2 lo = *reinterpret_cast<const uint2 *>(&B.v[SW::unit(r, 2 * cu16)]);
        const uint2 hi = *reinterpret_cast<const uint2 *>(&B.v[SW::unit(r, 2 * cu16 + 1)]);
        *reinterpret_cast<uint4 *>(go_ + ((o_t0 + r) * H + h) * D + cu16 * 8) =
            uint4{lo.x, lo.y, hi.x, hi.y};
      }
    }
  };

  int64_t o_t0 = -1;  // chunk whose O is staged in the previous buffer set, if any
  int o_n = 0;
  if (cw < c1) {
    fetch(cw);
    commit(cw, sm.buf[cw & 1]);
  }

  for (int c = cw; c < c1; ++c) {
    const bool emit = (c >= c0);
    const int64_t t0 = ts0 + (int64_t)c * kChunk;
    const int n = (int)min<int64_t>(kChunk, ts1 - t0);
    Buf &B = sm.buf[c & 1];
    __syncthreads();  // this chunk's buffer is written; the previous chunk is done with LDS
    if (o_t0 >= 0) store_o(o_t0, o_n, sm.buf[(c - 1) & 1]);
    o_t0 = -1;
    const bool more = c + 1 < c1;
    if (more) fetch(c + 1);
    const float glast = B.glast[0];

    // fragment reads from the swizzled tiles (8 bytes per lane each)
    auto nat8 = [&](const bf16 *t, int row, int c0) {  // elements c0 .. c0 + 7 of a row
      return cat8(lds_bf16x4(&t[SW::unit(row, c0 >> 2)]), lds_bf16x4(&t[SW::unit(row, (c0 >> 2) + 1)]));
    };
    auto perm8 = [&](const bf16 *t, int row, int c0) {  // c0 + 4 gq .. +3 and c0 + 16 + 4 gq .. +3
      return cat8(lds_bf16x4(&t[SW::unit(row, (c0 >> 2) + gq)]),
                  lds_bf16x4(&t[SW::unit(row, (c0 >> 2) + 4 + gq)]));
    };
    auto tr4 = [&](const bf16 *t, int rowbase, int colbase) {  // rows rowbase .. +3 of column colbase + cl
      return lds_tr16(&t[SW::unit(rowbase + (cl >> 2), (colbase >> 2) + (cl & 3))]);
    };

    // ---- A = strict_lower(diag(beta) (K K^T o decay)): 10 lower tiles over the waves
    for (int tau = wave; tau < 10; tau += NW) {
      const int bi = tile_bi(tau), bj = tile_bj(tau);
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks)
        acc = mma_bf16(nat8(B.k, 16 * bi + cl, 32 * ks + 8 * gq), nat8(B.k, 16 * bj + cl, 32 * ks + 8 * gq),
                       acc);
      const int j = 16 * bj + cl;
      const float gj = B.gam[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * bi + 4 * gq + i;
        sm.at[r * LDT + j] = (j < r) ? B.beta[r] * __expf(B.gam[r] - gj) * acc[i] : 0.f;
      }
    }
    __syncthreads();

    // K h and Q h for this wave's columns (the state's bf16 fragments are shared)
    f32x4 KS[4], QS[4];
    auto kq_products = [&]() {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) KS[mt] = QS[mt] = zero4();
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) {
        const bf16x8 sb = to_bf16x8(S[2 * ks], S[2 * ks + 1]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          KS[mt] = mma_bf16(perm8(B.k, 16 * mt + cl, 32 * ks), sb, KS[mt]);
          if (emit) QS[mt] = mma_bf16(perm8(B.q, 16 * mt + cl, 32 * ks), sb, QS[mt]);
        }
      }
    };

    // ---- wave 0: the four 16x16 diagonal blocks of Tm, in place (lane: block b, column j);
    //      the other waves: K h and Q h
    if (wave == 0) {
      const int b = lane >> 4, j = lane & 15;
      float *Ab = &sm.at[(16 * b) * LDT + 16 * b];
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < r; ++i) acc += Ab[r * LDT + i] * x[i];
        x[r] = (r < j) ? 0.f : ((r == j) ? 1.f : -acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) Ab[r * LDT + j] = x[r];
    } else {
      kq_products();
    }
    __syncthreads();

    // ---- wave 0: K h and Q h;  waves 1, 2: Tm_10 = -Tm_11 A_10 Tm_00 and
    //      Tm_32 = -Tm_33 A_32 Tm_22 in place;  the other waves: P = (Q K^T) o decay o mask
    if (wave == 0) {
      kq_products();
    } else if (wave < 3) {
      const int b = 1 + 2 * (wave - 1), cc = b - 1;
      f32x4 acc = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc = mma_f32(sm.at[(16 * b + cl) * LDT + 16 * cc + 4 * s + gq],
                      sm.at[(16 * cc + 4 * s + gq) * LDT + 16 * cc + cl], acc);
      f32x4 out = zero4();
#pragma unroll
      for (int i = 0; i < 4; ++i)
        out = mma_f32(sm.at[(16 * b + cl) * LDT + 16 * b + 4 * gq + i], acc[i], out);
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.at[(16 * b + 4 * gq + i) * LDT + 16 * cc + cl] = -out[i];
    } else if (emit) {
      for (int tau = wave - 3; tau < 10; tau += NW - 3) {
        const int bi = tile_bi(tau), bj = tile_bj(tau);
        f32x4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < KSD; ++ks)
          acc = mma_bf16(nat8(B.q, 16 * bi + cl, 32 * ks + 8 * gq),
                         nat8(B.k, 16 * bj + cl, 32 * ks + 8 * gq), acc);
        const int j = 16 * bj + cl;
        const float gj = B.gam[j];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * bi + 4 * gq + i;
          sm.p[r * LDP + j] = (bf16)((j <= r) ? __expf(B.gam[r] - gj) * acc[i] : 0.f);
        }
      }
    }
    __syncthreads();

    // ---- X = A_BL Tm_TL on waves 0-3: wave (b, c) = (2 + wave / 2, wave % 2) forms
    //      X_bc = sum_{j=c}^{1} A_bj Tm_jc; then Tm_BL = -Tm_BR X:
    //      Tm_2c = -Tm_22 X_2c ; Tm_3c = -(Tm_32 X_2c + Tm_33 X_3c)
    const int xb = 2 + ((wave >> 1) & 1), xc = wave & 1;
    f32x4 xv = zero4();
    if (wave < 4) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        if (jb < xc) continue;
#pragma unroll
        for (int s = 0; s < 4; ++s)
          xv = mma_f32(sm.at[(16 * xb + cl) * LDT + 16 * jb + 4 * s + gq],
                       sm.at[(16 * jb + 4 * s + gq) * LDT + 16 * xc + cl], xv);
      }
      if (xb == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sm.x[xc][(4 * gq + i) * 16 + cl] = xv[i];
      }
    }
    __syncthreads();
    if (wave < 4) {
      f32x4 out = zero4();
#pragma unroll
      for (int i = 0; i < 4; ++i)
        out = mma_f32(sm.at[(16 * xb + cl) * LDT + 16 * xb + 4 * gq + i], xv[i], out);
      if (xb == 3) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          out = mma_f32(sm.at[(48 + cl) * LDT + 32 + 4 * gq + i], sm.x[xc][(4 * gq + i) * 16 + cl],
                        out);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.at[(16 * xb + 4 * gq + i) * LDT + 16 * xc + cl] = -out[i];
    }
    __syncthreads();

    // ---- residual R = diag(beta) (V - diag(e^gamma) K h) as bf16 fragments over tokens
    bf16x8 rb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      f32x4 rv[2];
#pragma unroll
      for (int hlf = 0; hlf < 2; ++hlf) {
        const int mt = 2 * ks + hlf, r0 = 16 * mt + 4 * gq;
        const bf16x4 v4 = tr4(B.v, r0, ncol);
        const f32x4 be = lds_f32x4(&B.beta[r0]), ee = lds_f32x4(&B.eg[r0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) rv[hlf][i] = be[i] * ((float)v4[i] - ee[i] * KS[mt][i]);
      }
      rb[ks] = to_bf16x8(rv[0], rv[1]);
    }
    // ---- Delta = Tm R (Tm read with the same token permutation as R's fragments)
    f32x4 Dl[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      Dl[mt] = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (32 * ks > 16 * mt + 15) continue;  // Tm is lower triangular
        const float *tp = &sm.at[(16 * mt + cl) * LDT + 32 * ks + 4 * gq];
        Dl[mt] = mma_bf16(to_bf16x8(lds_f32x4(tp), lds_f32x4(tp + 16)), rb[ks], Dl[mt]);
      }
    }

    // ---- output: O = diag(e^gamma) Q h + P Delta, staged in this chunk's V tile
    if (emit) {
      const bf16x8 db0 = to_bf16x8(Dl[0], Dl[1]), db1 = to_bf16x8(Dl[2], Dl[3]);
      f32x4 O[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        O[mt] = lds_f32x4(&B.eg[16 * mt + 4 * gq]) * QS[mt];
        const bf16 *pp = &sm.p[(16 * mt + cl) * LDP + 4 * gq];
        O[mt] = mma_bf16(cat8(lds_bf16x4(pp), lds_bf16x4(pp + 16)), db0, O[mt]);
        if (mt >= 2)  // P is lower triangular: columns 32..63 only for rows 32..63
          O[mt] = mma_bf16(cat8(lds_bf16x4(pp + 32), lds_bf16x4(pp + 48)), db1, O[mt]);
        O[mt] *= a.scale;
      }
      __syncthreads();  // every wave is done reading V
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) B.v[SW::elem(16 * mt + 4 * gq + i, ncol + cl)] = (bf16)O[mt][i];
      o_t0 = t0;
      o_n = n;
    }

    // ---- state update: h <- e^{gamma_last} h + K^T diag(e^{gamma_last - gamma}) Delta
    {
      const float egl = __expf(glast);
      bf16x8 dt[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const f32x4 g0 = lds_f32x4(&B.gam[32 * ks + 4 * gq]);
        const f32x4 g1 = lds_f32x4(&B.gam[32 * ks + 16 + 4 * gq]);
        f32x4 e0, e1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          e0[i] = __expf(glast - g0[i]);
          e1[i] = __expf(glast - g1[i]);
        }
        dt[ks] = to_bf16x8(Dl[2 * ks] * e0, Dl[2 * ks + 1] * e1);
      }
#pragma unroll
      for (int mt = 0; mt < MTD; ++mt) {
        f32x4 acc = S[mt] * egl;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          acc = mma_bf16(cat8(tr4(B.k, 32 * ks + 4 * gq, 16 * mt), tr4(B.k, 32 * ks + 16 + 4 * gq, 16 * mt)),
                         dt[ks], acc);
        S[mt] = acc;
      }
    }

    // ---- the next chunk's inputs go to the other buffer set (its previous chunk is finished,
    //      and its staged O was written out at the top of this iteration)
    if (more) commit(c + 1, sm.buf[(c + 1) & 1]);
  }

  if (o_t0 >= 0) {  // the last emitted chunk's O
    __syncthreads();
    store_o(o_t0, o_n, sm.buf[(c1 - 1) & 1]);
  }
  if (a.ht != nullptr && c1 == nchunks_seq) {
    float *dst = a.ht + ((int64_t)seq * H + h) * D * D;
#pragma unroll
    for (int mt = 0; mt < MTD; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(16 * mt + 4 * gq + i) * D + ncol + cl] = S[mt][i];
  }
}

int fwd_fast_blocks_per_cu(int D) {
  int blocks = 0;
  const hipError_t e =
      D == 128 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fwd_fast_kernel<128>, 512, 0)
               : hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fwd_fast_kernel<64>, 256, 0);
  return (e == hipSuccess && blocks > 0) ? blocks : 1;
}

hipError_t launch_fwd_fast(const FwdArgs &a, int D, int64_t max_units, hipStream_t stream) {
  if (max_units <= 0) return hipSuccess;
  if (D == 128)
    hipLaunchKernelGGL(fwd_fast_kernel<128>, dim3((unsigned)max_units, a.H), dim3(512), 0, stream,
                       a);
  else
    hipLaunchKernelGGL(fwd_fast_kernel<64>, dim3((unsigned)max_units, a.H), dim3(256), 0, stream,
                       a);
  return hipGetLastError();
}

}  // namespace gdn
