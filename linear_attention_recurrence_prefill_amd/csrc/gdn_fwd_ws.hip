// Forward of the chunked gated delta rule for bf16 inputs with d_k = d_v = 128 on gfx950: a
// warp-specialised pipeline.
//
// The method is the chunked form of "How to Speed Up GDN Kernels for Qwen Models" (sections
// "What GDN actually computes", "Lever 1", "Lever 2"): per 64-token chunk, gamma = cumsum(g),
// A = strict_lower(diag(beta) (K K^T o e^{gamma_r - gamma_i})), Tm = (I + A)^-1, the state chain
// and the output.  The residual form of Delta is used (same quantity as U - W h):
//     Delta = Tm diag(beta) R',   R' = V - diag(e^gamma) K h.
//
// Work split.  Everything that does not depend on the state (the gate vectors, A, the inverse,
// P = (Q K^T) o decay o mask) is "prep"; the rest (K h, Delta, the output, the state update) is
// the "chain".  A workgroup has eight waves: waves 0-3 run the chain, wave w owning state columns
// [32 w, 32 w + 32); waves 4-6 prep chunk c + 1 while the chain runs chunk c; wave 7 forms chunk
// c + 2's gate vectors and streams its K and Q from HBM into LDS with direct global->LDS loads
// (with the in-kernel q/k normalisation, waves 5 and 6 also form the next chunk's row norms).
// Each chain wave streams its own columns of the next chunk's V the same way, into a tile only it
// reads.  One barrier per chunk hands the prepared chunk over; chain waves never wait for each
// other (each owns its columns of the state, of V and of the output), and their barrier waits for
// LDS accesses only, not for their global stores and loads.
//
// Delta by block forward substitution.  Split the chunk into 16-token blocks b = 0..3, write
// T_b = (I + A_bb)^-1 for the diagonal blocks of (I + A), fold beta into their columns
// (T'_b = T_b diag(beta_b)) and out of the rows of A's blocks below the diagonal
// (A_bj = diag(beta_b) A'_bj).  Then (I + A) Delta = diag(beta) R' is solved block by block:
//     Delta_0 = T'_0 R'_0,               Delta_1 = T'_1 (R'_1 - A'_10 Delta_0),
//     Delta_2 = T'_2 (R'_2 - A'_20 Delta_0 - A'_21 Delta_1),
//     Delta_3 = T'_3 (R'_3 - A'_30 Delta_0 - A'_31 Delta_1 - A'_32 Delta_2),
// with the two 32-token corrections (A'_2j, A'_3j for j < 2) as one K = 32 product.  Prep only
// inverts four 16x16 blocks (by substitution, on two waves) and never forms Tm's off-diagonal
// blocks; the chain spends 16 MFMAs per 16 state columns on Delta (12 with a full Tm).
//
// The output is formed transposed, O^T = (S^T Q^T) diag(scale e^gamma) + Delta^T P^T (P carries
// the scale).  A chain wave labels its 32 state columns so that the lane holding columns
// 4 i .. 4 i + 3 of one 16-column tile holds the next 4 in the other tile: each lane then writes 8
// consecutive columns of one token with one 16-byte store.  The stores go through a buffer
// resource whose range ends at the chunk's last token, so a ragged chunk needs no branch: the
// hardware drops the stores past its end.
//
// Addressing.  Every swizzled LDS access is a lane-constant byte offset (computed once, held in a
// register) plus an immediate: the swizzles depend on the row only modulo 16, and rows enter in
// multiples of 16.  Global loads and stores likewise use a uniform base and a lane-constant
// offset; only a sequence's ragged last chunk takes the per-lane clamped path.  The 16-row blocks
// of the K and Q tiles sit 16 bytes further apart than their size: reads of two blocks at the
// same lane offset would otherwise be fused into one two-address LDS read, which is issued as two
// passes over the same banks (twice the cycles of two single reads).
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_tiles.h"
#include "gdn_unit.h"

namespace gdn {
namespace {

constexpr int kD = 128;
constexpr int kRowBytes = kD * 2;  // one bf16 row of a K, Q or V tile
constexpr int kBlk = 16 * kRowBytes + 16;  // stride of the 16-row blocks of the K and Q tiles
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// 64 x 128 bf16 tiles (K, Q, V): rows of 256 bytes; the 16-byte unit c of row r is stored at unit
// c ^ sw(r).  For the reads below (16 lanes on one 8-byte unit of 16 consecutive rows, or
// transpose reads of 4 consecutive 8-byte units of 8 consecutive rows) each half-wave touches
// 32 distinct 8-byte bank pairs.
__device__ __forceinline__ int sw(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
// byte offset of the 8-byte unit u (elements 4u .. 4u + 3) of row r
__device__ __forceinline__ int toff(int r, int u) {
  return r * kRowBytes + (((u >> 1) ^ sw(r)) << 4) + ((u & 1) << 3);
}
// 32 x 32 bf16 block (-A'_BL): rows of 64 bytes, unit u of row r at u ^ 2 ((r / 4) % 4)
__device__ __forceinline__ int boff(int r, int u) { return r * 64 + ((u ^ (((r >> 2) & 3) << 1)) << 3); }
// 16 x 16 bf16 blocks (T'_b, -A'_10, -A'_32): rows of 32 bytes, unit u of row r at
// u ^ 2 ((r / 8) % 2)
__device__ __forceinline__ int soff(int r, int u) { return r * 32 + ((u ^ (((r >> 3) & 1) << 1)) << 3); }
// 64 x 64 bf16 P: rows of 128 bytes, unit u of row r at u ^ 2 ((r / 2) % 8)
__device__ __forceinline__ int poff(int r, int u) { return r * 128 + ((u ^ (((r >> 1) & 7) << 1)) << 3); }

constexpr int LA = 20;            // fp32 row stride of the 16x16 solve blocks
constexpr int AB = 16 * LA + 16;  // fp32 stride between solve blocks (spreads blocks over banks)

struct WsSmem {
  struct Vec {
    alignas(16) float beta[64];
    alignas(16) float eg[64];   // e^gamma
    alignas(16) float ego[64];  // scale e^gamma
    alignas(16) float edt[64];  // e^(gamma_last - gamma)
    alignas(16) float gam[64];
    alignas(16) float egl[4];   // e^gamma_last
  };
  alignas(16) char kq[3][2][4 * kBlk];  // [set][K, Q], three chunks in flight
  struct Blocks {
    alignas(16) char t[4][16 * 32];  // T'_0 .. T'_3
    alignas(16) char na10[16 * 32];  // -A'_10
    alignas(16) char na32[16 * 32];  // -A'_32
    alignas(16) char nabl[32 * 64];  // -A'_BL (rows 32..63, columns 0..31)
  };
  Blocks tb[2];
  alignas(16) char p[2][64 * 128];            // [set] P
  Vec vec[3];  // gate vectors: written one step ahead of prep, read by the chain a step later
  alignas(16) float at[4 * AB];  // A_bb transposed (row i = column i of A_bb), wave 4 only
  alignas(16) float tt[4 * AB];  // T_bb row-major, wave 4 only
  alignas(16) int imisc[4];
  int ready;   // chunk index + 1 whose A_22, A_33 (wave 7's part) are in at
  int landed;  // kNorm: chunk index + 1 whose K and Q tiles and gate vectors wave 7 has put in
};
static_assert(sizeof(WsSmem) <= 160 * 1024, "LDS budget");

__device__ __forceinline__ bf16x4 ld8(const char *p) { return *reinterpret_cast<const bf16x4 *>(p); }
__device__ __forceinline__ bf16x8 ld16(const char *p0, const char *p1) { return cat8(ld8(p0), ld8(p1)); }
__device__ __forceinline__ bf16x4 ldtr(const char *p) {
  return lds_tr16(reinterpret_cast<const bf16 *>(p));
}
__device__ __forceinline__ void st8(char *p, f32x4 x) { *reinterpret_cast<bf16x4 *>(p) = to_bf16x4(x); }
__device__ __forceinline__ f32x4 ldf4(const float *p) {  // 16-byte aligned
  return *reinterpret_cast<const f32x4 *>(p);
}

// A lane-constant value the compiler must keep in a register (it cannot rematerialise it at
// each use, which would cost address arithmetic inside the chunk loop).
__device__ __forceinline__ int pin(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// The 16x16 tiles waves 5 and 6 form per chunk: tile t is K's row block bj[t] times the row block
// bi[t] of K (q[t] == 0: A's blocks below the diagonal) or of Q (q[t] == 1: P).  Each wave's list
// covers two column blocks (wave 5: 0 and 3, wave 6: 1 and 2), 8 tiles each.
template <int W>
struct PrepTiles;
template <>
struct PrepTiles<5> {
  static constexpr int n = 8;
  static constexpr int bj[8] = {0, 0, 0, 0, 0, 0, 0, 3};
  static constexpr int bi[8] = {1, 2, 3, 0, 1, 2, 3, 3};
  static constexpr int q[8] = {0, 0, 0, 1, 1, 1, 1, 1};
};
template <>
struct PrepTiles<6> {
  static constexpr int n = 8;
  static constexpr int bj[8] = {1, 1, 2, 1, 1, 1, 2, 2};
  static constexpr int bi[8] = {2, 3, 3, 1, 2, 3, 2, 3};
  static constexpr int q[8] = {0, 0, 0, 1, 1, 1, 1, 1};
};

// A 4 x 4 block of 16-bit values over the four lanes of a quad, lane q holding column q (item i
// = row i, two to a dword, low half first): returns row q in lane q (item j = column j).  Two
// exchange stages: 2 x 2 blocks transposed between lanes q and q ^ 1 (byte permutes), then the
// off-diagonal 2 x 2 blocks swapped between lanes q and q ^ 2.
__device__ __forceinline__ uint2 quad_transpose16(uint2 d, int lane) {
  const unsigned p0 = __builtin_amdgcn_update_dpp(0u, d.x, 0xB1, 0xF, 0xF, true);  // lane ^ 1
  const unsigned p1 = __builtin_amdgcn_update_dpp(0u, d.y, 0xB1, 0xF, 0xF, true);
  const unsigned sel = (lane & 1) ? 0x03020706u : 0x05040100u;
  const unsigned a0 = __builtin_amdgcn_perm(p0, d.x, sel), a1 = __builtin_amdgcn_perm(p1, d.y, sel);
  const bool upper = (lane & 2) != 0;
  const unsigned y = __builtin_amdgcn_update_dpp(0u, upper ? a0 : a1, 0x4E, 0xF, 0xF, true);  // lane ^ 2
  return upper ? uint2{y, a1} : uint2{a0, y};
}

__device__ __forceinline__ void dma16(const char *g, char *l) {
  __builtin_amdgcn_global_load_lds(g, (GDN_LDS void *)l, 16, 0, 0);
}

}  // namespace

// kDump: the pass of the backward's forward recompute.  No output; per chunk it writes the state
// at the chunk's start in bf16 (a.dump_hc [chunks, H, D, D], the precision of the products that
// use it), Delta (a.dbg_delta [T, H, D]) and gamma (a.dbg_gamma [T, H]) in fp32, chunks numbered
// across sequences; in the truncate mode, for the unit's own chunks only (the warmup's belong
// to the unit before).  With kNorm it also writes the inverse norms of K's rows of those chunks
// to a.dump_rk [T, HK] when given (by the first value head of each key head).
// kTransition: the first pass of the exact split.  Workgroup (unit, head, z) runs the unit's
// chunks from a fixed start without output and writes its final state to a.unit_out[z]: z = 0
// from the zero state with the real V (the unit's own contribution B), z = 1 from the identity
// with V = 0 (the unit's transition matrix M, so that the state after the unit is
// M S_start + B for any start state).
// kNorm: q and k are L2-normalised per row.  The tiles stay as loaded; waves 5 (K) and 6 (Q)
// compute each row's inverse norm 1 / sqrt(|row|^2 + eps) once wave 7 has the chunk's K and Q in
// LDS, a step before prep uses them (wave 7 itself for the first chunk), and fold it into the
// per-token factors: in place into the chain's gate vectors (e^gamma of R', scale e^gamma of the
// output, e^{gamma_last - gamma} of the update; no other wave reads that chunk's vectors at that
// point, and waves 5 and 6 scale different ones), and through rn_s into A and P, whose prep
// applies it by rows and columns.  The normalised rows are never rounded to bf16, and the chain's
// code is the same as without the normalisation.
template <bool kTransition, bool kDump = false, bool kNorm = false>
__global__ __launch_bounds__(512) void fwd_ws_kernel(FwdArgs a) {
  __shared__ WsSmem sm;
  // kNorm: inverse row norms [chunk slot][K, Q][row], the slot as for the gate vectors
  __shared__ __attribute__((aligned(16))) float rn_s[kNorm ? 3 : 1][2][64];
  // V of the chunk on the chain, per chain wave its 32 columns: 64 rows of 64 bytes, the 16-byte
  // unit u of row r at unit u ^ 2 ((r / 4) % 2).  A variable of its own, so that the compiler
  // knows the chain waves' direct loads into it cannot touch the tiles they read meanwhile.
  __shared__ __attribute__((aligned(16))) char vt_s[4][64 * 64];
  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 4, cl = lane & 15;
  // wave-uniform role (scalar branches: a wave never steps through the other role's barriers)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int unit = a.longest_first ? blockIdx.y : blockIdx.x;
  const int h = a.longest_first ? blockIdx.x : blockIdx.y, H = a.H;
  const bool is_m = kTransition && blockIdx.z == 1;  // transition pass: the M half
  if (wave == 0) {
    Unit un;
    const bool ok = find_unit(a.cu, a.N, a.T, a.L, unit, kDump, lane, un, a.longest_first != 0);
    if (lane == 0) {
      sm.imisc[0] = ok ? un.seq : -1;
      sm.imisc[1] = un.c0;
      sm.imisc[2] = un.c1;
      if (kDump) sm.imisc[3] = (int)un.chunk_base;
    }
  }
  __syncthreads();
  const int seq = __builtin_amdgcn_readfirstlane(sm.imisc[0]);
  if (seq < 0) return;
  const int c0 = __builtin_amdgcn_readfirstlane(sm.imisc[1]);
  const int c1 = __builtin_amdgcn_readfirstlane(sm.imisc[2]);
  const int64_t chunk_base = kDump ? __builtin_amdgcn_readfirstlane(sm.imisc[3]) : 0;
  const int64_t ts0 = a.cu[seq], ts1 = a.cu[seq + 1];
  if (ts0 < 0 || ts1 < ts0 || ts1 > a.T) return;  // malformed cu_seqlens: touch nothing
  const int nchunks_seq = (int)((ts1 - ts0 + kChunk - 1) / kChunk);
  // a sequence's last unit has no successor; its map M is still formed when asked (the reverse
  // walk of the backward reads M transposed for every unit but a sequence's first)
  if (kTransition && c1 == nchunks_seq && !(is_m && a.unit_mt != nullptr && c0 > 0)) return;
  const int64_t tok_bytes = (int64_t)H * kRowBytes;      // stride of one token in v, o
  const int64_t tok_qk = (int64_t)a.HK * kRowBytes;      // ... in q, k
  const int hk = h / (H / a.HK);                          // this value head's key head
  const char *__restrict__ gq_ = static_cast<const char *>(a.q) + (int64_t)hk * kRowBytes;
  const char *__restrict__ gk_ = static_cast<const char *>(a.k) + (int64_t)hk * kRowBytes;
  const char *__restrict__ gv_ = static_cast<const char *>(a.v) + (int64_t)h * kRowBytes;
  const bf16 *__restrict__ gb_ = static_cast<const bf16 *>(a.beta);
  char *__restrict__ go_ = static_cast<char *>(a.o) + (int64_t)h * kRowBytes;

  // P's tiles (0, 1) and (2, 3) above the diagonal are read by the chain but never written by prep.
  for (int i = tid; i < 2 * 2 * 64; i += 512) {
    const int set = i >> 7, t = (i >> 6) & 1, r = 32 * t + ((i >> 2) & 15), u = 8 * t + 4 + (i & 3);
    *reinterpret_cast<uint2 *>(&sm.p[set][poff(r, u)]) = uint2{0u, 0u};
  }

  if (tid == 0) {
    sm.ready = 0;
    if (kNorm) sm.landed = 0;
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

  // kfrag offsets (chain and prep): elements 32 ks + 4 gq .. +3 and 32 ks + 16 + 4 gq .. +3 of row
  // cl (+ 16 m rows as an immediate) -- the k-order of a pair of D-layout accumulators used as
  // the other MFMA operand
  int o_kf[4][2];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) o_kf[ks][hf] = pin(toff(cl, 8 * ks + 4 * hf + gq));
  auto kfrag = [&](const char *t, int m, int ks) {
    return ld16(t + m * kBlk + o_kf[ks][0], t + m * kBlk + o_kf[ks][1]);
  };

  // A's diagonal 16x16 blocks b0 = 2 half and b1 = b0 + 1 in fp32, stored transposed into at
  // (row i of the stored block = column i of A_bb)
  auto a_diag = [&](const char *Kt, const WsSmem::Vec &vc, const float *rk, int half) {
    const int b0 = 2 * half, b1 = b0 + 1;
    f32x4 a00 = zero4(), a11 = zero4();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 f0 = kfrag(Kt, b0, ks), f1 = kfrag(Kt, b1, ks);
      a00 = mma_bf16(f0, f0, a00);
      a11 = mma_bf16(f1, f1, a11);
    }
    const f32x4 gr0 = ldf4(&vc.gam[16 * b0 + 4 * gq]), br0 = ldf4(&vc.beta[16 * b0 + 4 * gq]);
    const f32x4 gr1 = ldf4(&vc.gam[16 * b1 + 4 * gq]), br1 = ldf4(&vc.beta[16 * b1 + 4 * gq]);
    const float gi0 = vc.gam[16 * b0 + cl], gi1 = vc.gam[16 * b1 + cl];
    f32x4 nr0 = {1.f, 1.f, 1.f, 1.f}, nr1 = nr0;  // row x column inverse norms (kNorm)
    if constexpr (kNorm) {
      nr0 = ldf4(&rk[16 * b0 + 4 * gq]) * rk[16 * b0 + cl];
      nr1 = ldf4(&rk[16 * b1 + 4 * gq]) * rk[16 * b1 + cl];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rl = 4 * gq + e;
      a00[e] = cl < rl ? br0[e] * nr0[e] * __expf(gr0[e] - gi0) * a00[e] : 0.f;
      a11[e] = cl < rl ? br1[e] * nr1[e] * __expf(gr1[e] - gi1) * a11[e] : 0.f;
    }
    float *t0p = &sm.at[b0 * AB + cl * LA + 4 * gq], *t1p = &sm.at[b1 * AB + cl * LA + 4 * gq];
    *reinterpret_cast<float2 *>(t0p) = float2{a00[0], a00[1]};
    *reinterpret_cast<float2 *>(t0p + 2) = float2{a00[2], a00[3]};
    *reinterpret_cast<float2 *>(t1p) = float2{a11[0], a11[1]};
    *reinterpret_cast<float2 *>(t1p + 2) = float2{a11[2], a11[3]};
  };

  // kNorm: inverse norms 1 / sqrt(|row|^2 + eps) of the rows of chunk c's K (which = 0) or Q
  // (which = 1) tile, once it is in LDS, into rn_s and folded into the chunk's gate vectors (K:
  // e^gamma of R' and e^{gamma_last - gamma} of the update; Q: the output's scale e^gamma), which
  // gate_vectors wrote earlier.  Lane r sums row r, reading its 16-byte units in an order rotated
  // by r (no two lanes of a 16-row block on one bank group).
  auto row_norms = [&](int c, int which) __attribute__((always_inline)) {  // three call sites
    const int base = (lane >> 4) * kBlk + (lane & 15) * kRowBytes;
    const char *t = sm.kq[c % 3][which];
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const bf16x8 x = *reinterpret_cast<const bf16x8 *>(t + base + (((u + lane) & 15) << 4));
      const bf16x2 p0 = __builtin_shufflevector(x, x, 0, 1), p1 = __builtin_shufflevector(x, x, 2, 3);
      const bf16x2 p2 = __builtin_shufflevector(x, x, 4, 5), p3 = __builtin_shufflevector(x, x, 6, 7);
      s = __builtin_amdgcn_fdot2_f32_bf16(p0, p0, s, false);
      s = __builtin_amdgcn_fdot2_f32_bf16(p1, p1, s, false);
      s = __builtin_amdgcn_fdot2_f32_bf16(p2, p2, s, false);
      s = __builtin_amdgcn_fdot2_f32_bf16(p3, p3, s, false);
    }
    const float r = 1.f / sqrtf(s + kL2NormEps);
    rn_s[c % 3][which][lane] = r;
    if constexpr (kDump) {  // K's of the unit's own chunks, once per key head, for the backward
      if (which == 0 && a.dump_rk != nullptr && c >= c0 && h % (H / a.HK) == 0 && lane < chunk_n(c))
        a.dump_rk[(chunk_t0(c) + lane) * a.HK + h / (H / a.HK)] = r;
    }
    WsSmem::Vec &vc = sm.vec[c % 3];
    if (which == 0) {
      vc.eg[lane] *= r;
      vc.edt[lane] *= r;
    } else {
      vc.ego[lane] *= r;
    }
  };
  // the Q tile of chunk c carries output rows (it is loaded and normalised only then)
  auto emits = [&](int c) { return !kTransition && !kDump && c >= c0; };

  const int w = wave & 3;

  if (wave < 4) {
    // ======================= chain waves: the state recurrence and the output =======================
    const int ncol = 32 * w;  // this wave's first state column
    // lane-constant offsets: transpose reads of K (rows 4 gq + cl / 4, unit 4 mt + cl % 4) and of
    // this wave's V columns (unit 2 (cl % 4) + nt: the column labels below), 32-wide block rows,
    // P rows, and global offsets
    int o_tr[8], o_vtr[2], o_bf[2], o_pf[2][2];
    const int o_sf = pin(soff(cl, gq));  // 16x16 block row cl, elements 4 gq .. 4 gq + 3
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o_tr[mt] = pin(toff(4 * gq + (cl >> 2), 4 * mt + (cl & 3)));
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int r = 4 * gq + (cl >> 2), u = 2 * (cl & 3) + nt;
      o_vtr[nt] = pin(r * 64 + (((u >> 1) ^ (((r >> 2) & 1) << 1)) << 4) + ((u & 1) << 3));
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) o_bf[hf] = pin(boff(cl, 4 * hf + gq));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) o_pf[ks][hf] = pin(poff(cl, 8 * ks + 4 * hf + gq));
    // direct V loads: instruction j fills rows 16 j .. 16 j + 15 of this wave's V tile; lane l
    // writes physical unit l % 4 of row 16 j + l / 4, which holds logical unit (l % 4) ^ 2 ((l / 16) % 2)
    char *const vw = vt_s[w];
    const int vu = 4 * w + ((lane & 3) ^ (((lane >> 4) & 1) << 1));
    const int o_gv = pin((int)((lane >> 2) * tok_bytes) + vu * 16);
    const int o_go = pin((int)(cl * tok_bytes) + (ncol + 8 * gq) * 2);      // O stores
    // dump stores: the state (bf16, row 4 gq of a 128 x 128 matrix) and Delta (fp32, token 4 gq),
    // at this lane's column of tile nt
    int o_dh[2] = {0, 0}, o_dd[2] = {0, 0};
    if constexpr (kDump) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int col = ncol + 8 * (cl >> 2) + 4 * nt + (cl & 3);
        o_dh[nt] = pin((4 * gq * kD + col) * 2);
        o_dd[nt] = pin((4 * gq * H * kD + col) * 4);
      }
    }
    auto trk = [&](const char *t, int rows, int mt) { return ldtr(t + (rows / 16) * kBlk + o_tr[mt]); };

    // S[mt][nt] holds rows 16 mt + 4 gq + i of column ncol + 8 (cl / 4) + 4 nt + cl % 4 (tile nt's
    // column n is state column ncol + 8 (n / 4) + 4 nt + n % 4; K h, Delta, the update and V follow
    // the same labels, and a lane's output columns 4 gq .. 4 gq + 3 of the two tiles are adjacent)
    f32x4 S[8][2];
    const float *hp = nullptr;  // the start state, or null for zero
    if (!kTransition && a.unit_h0 != nullptr)
      hp = a.unit_h0 + ((int64_t)unit * H + h) * kD * kD;  // the exact split's final pass
    else if (!kTransition && cw == 0)
      hp = a.h0 == nullptr ? nullptr : a.h0 + (int64_t)seq * a.h0_stride + (int64_t)h * kD * kD;
    if (is_m) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            S[mt][nt][i] = 16 * mt + 4 * gq + i == ncol + 8 * (cl >> 2) + 4 * nt + (cl & 3) ? 1.f : 0.f;
    } else if (hp != nullptr) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            S[mt][nt][i] = hp[(16 * mt + 4 * gq + i) * kD + ncol + 8 * (cl >> 2) + 4 * nt + (cl & 3)];
      // consume the loads here, so that no wait for them is left inside the chunk loop
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) asm volatile("" : "+v"(S[mt][nt]));
    } else {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) S[mt][0] = S[mt][1] = zero4();
    }
    // V of chunk c for this wave's columns into its V tile (rows past a ragged chunk's end repeat
    // its last token)
    auto v_dma = [&](int c) {
      const int64_t t0 = chunk_t0(c);
      const int n = chunk_n(c);
      if (n == kChunk) {
#pragma unroll
        for (int j = 0; j < 4; ++j) dma16(gv_ + (t0 + 16 * j) * tok_bytes + o_gv, vw + 1024 * j);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t t = t0 + min(16 * j + (lane >> 2), n - 1);
          dma16(gv_ + t * tok_bytes + vu * 16, vw + 1024 * j);
        }
      }
    };
    // the state as bf16 operand fragments, in the k-order of kfrag
    auto state_frags = [&](bf16x8(&sb)[4][2]) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) sb[ks][nt] = to_bf16x8(S[2 * ks][nt], S[2 * ks + 1][nt]);
    };

    // V of the first chunk; each later chunk's V is loaded once the chunk before it has consumed
    // the tile (the compiler waits for the direct loads before the tile is read)
    if (is_m) {  // the transition is taken with V = 0: a zero V tile, never reloaded
      for (int i = lane; i < 64 * 64 / 16; i += 64) reinterpret_cast<uint4 *>(vw)[i] = uint4{0u, 0u, 0u, 0u};
    } else if (cw < c1) {
      v_dma(cw);
    }
    wait_vm0();  // the initial state and V are in place: no load is outstanding when the loop starts
    __syncthreads();  // chunk cw's K and Q are in LDS (wave 7)

    for (int c = cw; c <= c1; ++c) {
      if (c > cw) {
        // ---------------- chunk cc = c - 1 (prepared during the previous step) ----------------
        const int cc = c - 1;
        const int64_t t0 = chunk_t0(cc);
        const int n = chunk_n(cc);
        const bool emit = !kTransition && !kDump && cc >= c0;
        if (kDump && cc >= c0) {  // the state at the chunk's start (all rows in range; row
                                  // offsets as scalar operands); none for a warmup's chunks
          const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(
              a.dump_hc + ((chunk_base + cc) * H + h) * kD * kD, (short)0, kD * kD * 2, 0x00020000);
#pragma unroll
          for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int nt = 0; nt < 2; ++nt)
                __builtin_amdgcn_raw_buffer_store_b16(
                    __builtin_bit_cast(unsigned short, (bf16)S[mt][nt][i]), hr, o_dh[nt],
                    (16 * mt + i) * kD * 2, 0);
        }
        const int Y = cc & 1;
        const char *Kt = sm.kq[cc % 3][0], *Qt = sm.kq[cc % 3][1];
        const WsSmem::Vec &vc = sm.vec[cc % 3];

        // ---- K h, then R' = V - diag(e^gamma) K h, fp32
        f32x4 R[4][2];
        {
          bf16x8 sb[4][2];
          state_frags(sb);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) R[mt][0] = R[mt][1] = zero4();
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
              const bf16x8 af = kfrag(Kt, mt, ks);
#pragma unroll
              for (int nt = 0; nt < 2; ++nt) R[mt][nt] = mma_bf16(af, sb[ks][nt], R[mt][nt]);
            }
        }
        // this chunk's V, loaded directly into the tile a step ago, has landed
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        wait_vm0();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const f32x4 ee = *reinterpret_cast<const f32x4 *>(&vc.eg[16 * mt + 4 * gq]);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            const bf16x4 v4 = ldtr(vw + 1024 * mt + o_vtr[nt]);
#pragma unroll
            for (int i = 0; i < 4; ++i) R[mt][nt][i] = (float)v4[i] - ee[i] * R[mt][nt][i];
          }
        }
        // chunk cc + 1's V into the tile once every read of chunk cc's V has returned (the compiler
        // does not order the transpose reads against the direct loads by itself)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0xC07F);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (cc + 1 < c1 && !is_m) v_dma(cc + 1);

        // ---- Delta block by block (see the head of this file).  Delta is kept only as bf16 operand
        //      fragments: da for the output, dt = Delta o e^{gamma_last - gamma} for the state
        //      update (both in the k-order of kfrag over tokens)
        bf16x8 da[2][2], dt[2][2];
        {
          const WsSmem::Blocks &B = sm.tb[Y];
          auto sfrag = [&](const char *blk) { return ld8(blk + o_sf); };
          auto bfrag = [&](int m) { return ld16(B.nabl + 1024 * m + o_bf[0], B.nabl + 1024 * m + o_bf[1]); };
          const int64_t tok0 = t0;  // (t0 below names the block T'_{2h})
          // one 32-token half: Delta_{2h} = T'_{2h} R'_{2h}, Delta_{2h+1} = T'_{2h+1} (R'_{2h+1} -
          // A'_{2h+1,2h} Delta_{2h})
          auto half_solve = [&](int hb, const char *na) {
            const bf16x4 t0 = sfrag(B.t[2 * hb]), t1 = sfrag(B.t[2 * hb + 1]), nf = sfrag(na);
            f32x4 Dl0[2], Dl1[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) Dl0[nt] = mma_bf16_k16(t0, to_bf16x4(R[2 * hb][nt]), zero4());
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
              R[2 * hb + 1][nt] = mma_bf16_k16(nf, to_bf16x4(Dl0[nt]), R[2 * hb + 1][nt]);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) Dl1[nt] = mma_bf16_k16(t1, to_bf16x4(R[2 * hb + 1][nt]), zero4());
            if (kDump && cc >= c0) {  // Delta rows 32 hb + 4 gq + i and 32 hb + 16 + 4 gq + i;
                                      // rows at or past the chunk's end fall outside the range
              const __amdgpu_buffer_rsrc_t dr = __builtin_amdgcn_make_buffer_rsrc(
                  a.dbg_delta + (tok0 * H + h) * kD, (short)0, n * H * kD * 4, 0x00020000);
#pragma unroll
              for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                  // the row goes into the vector offset, which the range check covers
                  const int v0 = o_dd[nt] + (32 * hb + i) * H * kD * 4;
                  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(Dl0[nt][i]), dr,
                                                        v0, 0, 0);
                  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(Dl1[nt][i]), dr,
                                                        v0 + 16 * H * kD * 4, 0, 0);
                }
            }
            const f32x4 e0 = *reinterpret_cast<const f32x4 *>(&vc.edt[32 * hb + 4 * gq]);
            const f32x4 e1 = *reinterpret_cast<const f32x4 *>(&vc.edt[32 * hb + 16 + 4 * gq]);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
              da[hb][nt] = to_bf16x8(Dl0[nt], Dl1[nt]);
              dt[hb][nt] = to_bf16x8(Dl0[nt] * e0, Dl1[nt] * e1);
            }
          };
          half_solve(0, B.na10);
#pragma unroll
          for (int mt = 2; mt < 4; ++mt) {  // R'_B -= A'_BL Delta_T
            const bf16x8 af = bfrag(mt - 2);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) R[mt][nt] = mma_bf16(af, da[0][nt], R[mt][nt]);
          }
          half_solve(1, B.na32);
        }

        // ---- output, transposed: O^T = (S^T Q^T) diag(scale e^gamma) + Delta^T P^T
        if (emit) {
          const char *P = sm.p[Y];
          float et[4];
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) et[tt] = vc.ego[16 * tt + cl];
          f32x4 acc[4][2];
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) acc[tt][0] = acc[tt][1] = zero4();
          // e^gamma-scaled S^T Q^T, one k-step of all 8 (token block, column block) tiles at a time
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            bf16x8 sbk[2];
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) sbk[nt] = to_bf16x8(S[2 * ks][nt], S[2 * ks + 1][nt]);
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
              const bf16x8 qf = kfrag(Qt, tt, ks);
#pragma unroll
              for (int nt = 0; nt < 2; ++nt) acc[tt][nt] = mma_bf16(sbk[nt], qf, acc[tt][nt]);
            }
          }
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) acc[tt][nt] *= et[tt];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
              if (ks <= (tt >> 1)) {
                const bf16x8 pf = ld16(P + 2048 * tt + o_pf[ks][0], P + 2048 * tt + o_pf[ks][1]);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) acc[tt][nt] = mma_bf16(da[ks][nt], pf, acc[tt][nt]);
              }
            // rows of the 16-token block at or past the chunk's end fall outside the buffer range
            // and are dropped by the store
            const int nrows = max(0, n - 16 * tt);
            const __amdgpu_buffer_rsrc_t ob = __builtin_amdgcn_make_buffer_rsrc(
                go_ + (t0 + 16 * tt) * tok_bytes, (short)0, nrows * (int)tok_bytes, 0x00020000);
            {
              const bf16x8 o8 = to_bf16x8(acc[tt][0], acc[tt][1]);
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, o8), ob, o_go, 0, 0);
            }
          }
        }


        // ---- state update: h <- e^{gamma_last} h + K^T diag(e^{gamma_last - gamma}) Delta
        {
          const float egl = vc.egl[0];
#pragma unroll
          for (int mt = 0; mt < 8; ++mt) {
            const bf16x8 a0 = cat8(trk(Kt, 0, mt), trk(Kt, 16, mt));
            const bf16x8 a1 = cat8(trk(Kt, 32, mt), trk(Kt, 48, mt));
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
              S[mt][nt] = mma_bf16(a1, dt[1][nt], mma_bf16(a0, dt[0][nt], S[mt][nt] * egl));
          }
        }
      }
      lds_barrier();
    }

    if (kTransition) {
      // the unit's map in the middle pass's operand order: B (map_b_index), M (split,
      // map_m_hi_byte) and, for the backward's reverse walk, M^T; this lane holds rows
      // 16 mt + 4 gq + i of column c
      float *dst = a.unit_out + (((int64_t)blockIdx.z * a.units + unit) * H + h) * kD * kD;
      float *dt = (is_m && a.unit_mt != nullptr && c0 > 0)
                      ? a.unit_mt + ((int64_t)unit * H + h) * kD * kD
                      : nullptr;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int c = ncol + 8 * (cl >> 2) + 4 * nt + (cl & 3);
          if (!is_m) {
            *reinterpret_cast<f32x4 *>(dst + map_b_index(16 * mt + 4 * gq, c)) = S[mt][nt];
          } else {  // split into bf16 head and remainder (map_m_hi_byte)
            const bf16x4 hi = to_bf16x4(S[mt][nt]);
            const bf16x4 lo = to_bf16x4(S[mt][nt] - __builtin_convertvector(hi, f32x4));
            // the quad's lanes hold four consecutive columns (c % 4 = lane % 4): transposed, lane
            // q holds row 16 mt + 4 gq + q at those columns, 8 consecutive bytes of the map
            const uint2 th = quad_transpose16(__builtin_bit_cast(uint2, hi), lane);
            const uint2 tl = quad_transpose16(__builtin_bit_cast(uint2, lo), lane);
            char *dm = reinterpret_cast<char *>(dst) +
                       map_m_hi_byte(16 * mt + 4 * gq + (lane & 3), c - (lane & 3));
            *reinterpret_cast<uint2 *>(dm) = th;
            *reinterpret_cast<uint2 *>(dm + 1024) = tl;
            if (dt != nullptr) {  // M^T[c][r] = M[r][c]: the four rows are consecutive in k
              char *dmt = reinterpret_cast<char *>(dt) + map_m_hi_byte(c, 16 * mt + 4 * gq);
              *reinterpret_cast<bf16x4 *>(dmt) = hi;
              *reinterpret_cast<bf16x4 *>(dmt + 1024) = lo;
            }
          }
        }
    } else if (a.ht != nullptr && c1 == nchunks_seq) {
      float *dst = a.ht + ((int64_t)seq * H + h) * kD * kD;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            dst[(16 * mt + 4 * gq + i) * kD + ncol + 8 * (cl >> 2) + 4 * nt + (cl & 3)] = S[mt][nt][i];
    }
  } else if (wave == 7) {
    // ================ wave 7: gate vectors, and K and Q from HBM into LDS, one chunk ahead ===========
    // It writes the gate vectors before it issues the direct global->LDS loads and touches LDS
    // no more until the barrier, so nothing waits on those loads early.  DMA instruction j fills
    // LDS rows 4 j .. 4 j + 3; lane l writes physical unit l % 16 of row 4 j + l / 16, which holds
    // logical unit (l % 16) ^ sw(row).
    int o_dma[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = 4 * j + (lane >> 4);
      o_dma[j] = pin((int)(r * tok_qk) + (((lane & 15) ^ sw(r)) << 4));
    }
    auto dma_tile = [&](char *dst, const char *src, int c) {
      const int64_t t0 = chunk_t0(c);
      const int n = chunk_n(c);
      if (n == kChunk) {
        const char *base = src + t0 * tok_qk;
#pragma unroll
        for (int j = 0; j < 16; ++j) dma16(base + o_dma[j], dst + (j >> 2) * kBlk + 1024 * (j & 3));
      } else {  // ragged last chunk: rows past n repeat the last token
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int r = 4 * j + (lane >> 4);
          const int64_t t = t0 + min(r, n - 1);
          dma16(src + t * tok_qk + (((lane & 15) ^ sw(r)) << 4), dst + (j >> 2) * kBlk + 1024 * (j & 3));
        }
      }
    };
    // g and beta of this lane's token in chunk c (the address is clamped to the chunk; lanes past
    // its end are masked when the vectors are formed)
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
    // gamma = cumsum(g) and the vectors prep and the chain read, for chunk c
    auto gate_vectors = [&](const GB &x, int c) {
      const int n = chunk_n(c);
      const float gv = lane < n ? x.g : 0.f;
      const float bv = lane < n ? __uint_as_float((unsigned)x.b << 16) : 0.f;
      const float gam = wave_inclusive_scan_dpp(gv);
      const float gl = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gam), n - 1));
      WsSmem::Vec &vc = sm.vec[c % 3];
      vc.beta[lane] = bv;
      vc.eg[lane] = __expf(gam);
      vc.ego[lane] = a.scale * __expf(gam);
      vc.edt[lane] = __expf(gl - gam);
      vc.gam[lane] = gam;
      if (lane == 0) vc.egl[0] = __expf(gl);
      if (kDump && c >= c0 && lane < n) a.dbg_gamma[(chunk_t0(c) + lane) * H + h] = gam;
    };
    GB gbx{0.f, 0};
    if (cw < c1) {
      gbx = gb_load(cw);
      wait_vm0();
      gate_vectors(gbx, cw);
      dma_tile(sm.kq[cw % 3][0], gk_, cw);
      if (!kTransition && !kDump && cw >= c0) dma_tile(sm.kq[cw % 3][1], gq_, cw);
      if (cw + 1 < c1) gbx = gb_load(cw + 1);
    }
    wait_vm0();
    if (kNorm && cw < c1) {  // the first chunk's norms; waves 5 and 6 form the later chunks'
      row_norms(cw, 0);
      if (emits(cw))
        row_norms(cw, 1);
      else
        rn_s[cw % 3][1][lane] = 1.f;
    }
    __syncthreads();
    for (int c = cw; c <= c1; ++c) {
      if (c < c1) {  // A's diagonal blocks 2 and 3 of the chunk prep works on
        a_diag(sm.kq[c % 3][0], sm.vec[c % 3], rn_s[kNorm ? c % 3 : 0][0], 1);
        __hip_atomic_store(&sm.ready, c + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      if (c + 1 < c1) {
        gate_vectors(gbx, c + 1);
        dma_tile(sm.kq[(c + 1) % 3][0], gk_, c + 1);
        if (!kTransition && !kDump && c + 1 >= c0) dma_tile(sm.kq[(c + 1) % 3][1], gq_, c + 1);
        if (c + 2 < c1) gbx = gb_load(c + 2);
      }
      wait_vm0();  // chunk c + 1's K and Q are in LDS before the barrier that hands them over
      // kNorm: waves 5 and 6 form chunk c + 1's row norms from them before the same barrier
      if (kNorm && c + 1 < c1)
        __hip_atomic_store(&sm.landed, c + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      __syncthreads();
    }
  } else {
    // ======================= waves 4-6: everything else that does not need the state ===============
    __syncthreads();

    for (int c = cw; c <= c1; ++c) {
      if (c < c1) {
        // ---------------- chunk c ----------------
        const bool emit = !kTransition && !kDump && c >= c0;
        const int Y = c & 1;
        const char *Kt = sm.kq[c % 3][0], *Qt = sm.kq[c % 3][1];
        const WsSmem::Vec &vc = sm.vec[c % 3];
        if (wave == 4) {
          // ---- A's diagonal blocks 0 and 1 (wave 7 forms blocks 2 and 3 and publishes them
          //      through sm.ready; the bounded wait cannot hang)
          a_diag(Kt, vc, rn_s[kNorm ? c % 3 : 0][0], 0);
          int it = 0;
          for (; it < (1 << 22); ++it) {
            const int r = __hip_atomic_load(&sm.ready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
            if (__builtin_amdgcn_readfirstlane(r) >= c + 1) break;
            __builtin_amdgcn_s_sleep(1);
          }
          // a wait that ran out leaves a flag the host can read (gdn_device_faults); the
          // results of this launch are then not to be trusted
          if (it == (1 << 22) && lane == 0 && a.faults != nullptr)
            __hip_atomic_fetch_or(a.faults, kFaultDiagWait, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
          // ---- the four diagonal inverses by substitution: lane (block gq, column cl)
          {
            const float *ab = &sm.at[gq * AB];
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) x[r] = r == cl ? 1.f : 0.f;
            // all of the block's columns first (the loads do not depend on the substitution)
            float col[15][16];
#pragma unroll
            for (int i = 0; i < 15; ++i)
#pragma unroll
              for (int q = (i + 1) >> 1; q < 8; ++q) {
                const float2 v2 = *reinterpret_cast<const float2 *>(ab + i * LA + 2 * q);
                col[i][2 * q] = v2.x;
                col[i][2 * q + 1] = v2.y;
              }
#pragma unroll
            for (int i = 0; i < 15; ++i)
#pragma unroll
              for (int r = i + 1; r < 16; ++r) x[r] -= col[i][r] * x[i];
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.tt[gq * AB + r * LA + cl] = x[r];
          }
          // ---- T'_b = T_b diag(beta_b) as bf16: 4 rows of 4 columns per lane
#pragma unroll
          for (int it = 0; it < 4; ++it) {
            const int idx = lane + 64 * it, b = idx >> 6, r = (idx >> 2) & 15, qd = idx & 3;
            const f32x4 t4 = ldf4(&sm.tt[b * AB + r * LA + 4 * qd]) * ldf4(&vc.beta[16 * b + 4 * qd]);
            st8(&sm.tb[Y].t[b][soff(r, qd)], t4);
          }
        } else {
          // ---- waves 5 and 6: A's 16x16 blocks below the diagonal without their beta row factor,
          //      negated (-A'_10, -A'_32 and the lower-left 32x32 block -A'_BL), and P, as bf16.
          //      Tiles are formed transposed (lane (row r, group) holds 4 consecutive columns i
          //      of row r), all of a wave's tiles at once over the four k-steps so that their
          //      fragment loads and MFMAs overlap.
          auto run = [&](auto tiles) {
            using PT = decltype(tiles);
            f32x4 acc[PT::n];
#pragma unroll
            for (int t = 0; t < PT::n; ++t) acc[t] = zero4();
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
              bf16x8 kf4[4], qf4[4];
#pragma unroll
              for (int b = 0; b < 4; ++b) {
                bool needk = false, needq = false;
#pragma unroll
                for (int t = 0; t < PT::n; ++t) {
                  needk |= PT::bj[t] == b || (PT::q[t] == 0 && PT::bi[t] == b);
                  needq |= PT::q[t] == 1 && PT::bi[t] == b;
                }
                if (needk) kf4[b] = kfrag(Kt, b, ks);
                if (needq && emit) qf4[b] = kfrag(Qt, b, ks);
              }
#pragma unroll
              for (int t = 0; t < PT::n; ++t) {
                if (PT::q[t] == 0)
                  acc[t] = mma_bf16(kf4[PT::bj[t]], kf4[PT::bi[t]], acc[t]);
                else if (emit)
                  acc[t] = mma_bf16(kf4[PT::bj[t]], qf4[PT::bi[t]], acc[t]);
              }
            }
            WsSmem::Blocks &B = sm.tb[Y];
#pragma unroll
            for (int t = 0; t < PT::n; ++t) {
              const int bj = PT::bj[t], bi = PT::bi[t];
              if (PT::q[t] == 1 && !emit) continue;
              const f32x4 gi = ldf4(&vc.gam[16 * bj + 4 * gq]);
              const int r = 16 * bi + cl;
              const float gr = vc.gam[r];
              f32x4 nf = {1.f, 1.f, 1.f, 1.f};  // row x column inverse norms (kNorm)
              if constexpr (kNorm)
                nf = ldf4(&rn_s[c % 3][0][16 * bj + 4 * gq]) * rn_s[c % 3][PT::q[t]][r];
              f32x4 val;
              if (PT::q[t] == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) val[e] = -nf[e] * __expf(gr - gi[e]) * acc[t][e];
                char *dst = bi == 1 ? B.na10 + soff(cl, gq)
                            : (bj == 2 ? B.na32 + soff(cl, gq) : B.nabl + boff(r - 32, 4 * bj + gq));
                st8(dst, val);
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  val[e] = (16 * bj + 4 * gq + e <= r) ? a.scale * nf[e] * __expf(gr - gi[e]) * acc[t][e] : 0.f;
                st8(&sm.p[Y][poff(r, 4 * bj + gq)], val);
              }
            }
          };
          if (wave == 5)
            run(PrepTiles<5>{});
          else
            run(PrepTiles<6>{});
        }
      }
      // kNorm: chunk c + 1's row norms, K by wave 5 and Q by wave 6, once wave 7 has put in its
      // tiles and gate vectors (it does so in every step that has a chunk c + 1, before the
      // step's barrier; the wait is bounded all the same, as wave 4's).  The barrier waits for
      // these norms, so the two waves go before the chain waves on their SIMDs meanwhile.
      if (kNorm && c + 1 < c1 && wave != 4) {
        int it = 0;
        for (; it < (1 << 22); ++it) {
          const int r = __hip_atomic_load(&sm.landed, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
          if (__builtin_amdgcn_readfirstlane(r) >= c + 1) break;
          __builtin_amdgcn_s_sleep(1);
        }
        if (it == (1 << 22) && lane == 0 && a.faults != nullptr)
          __hip_atomic_fetch_or(a.faults, kFaultDiagWait, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_setprio(3);
        if (wave == 5)
          row_norms(c + 1, 0);
        else if (emits(c + 1))
          row_norms(c + 1, 1);
        else
          rn_s[(c + 1) % 3][1][lane] = 1.f;
        __builtin_amdgcn_s_setprio(0);
      }
      __syncthreads();
    }
  }
}

int fwd_ws_blocks_per_cu() {
  int blocks = 0;
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fwd_ws_kernel<false>, 512, 0);
  return (e == hipSuccess && blocks > 0) ? blocks : 1;
}

hipError_t launch_fwd_ws(const FwdArgs &a, int64_t max_units, hipStream_t stream) {
  if (max_units <= 0) return hipSuccess;
  const dim3 grid = a.longest_first ? dim3(a.H, (unsigned)max_units) : dim3((unsigned)max_units, a.H);
  if (a.l2norm)
    hipLaunchKernelGGL((fwd_ws_kernel<false, false, true>), grid, dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL(fwd_ws_kernel<false>, grid, dim3(512), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd_ws_dump(const FwdArgs &a, int64_t max_units, hipStream_t stream) {
  if (max_units <= 0) return hipSuccess;
  if (a.l2norm)
    hipLaunchKernelGGL((fwd_ws_kernel<false, true, true>), dim3((unsigned)max_units, a.H),
                       dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL((fwd_ws_kernel<false, true>), dim3((unsigned)max_units, a.H), dim3(512), 0,
                       stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd_ws_transition(const FwdArgs &a, int64_t units, hipStream_t stream) {
  if (units <= 0) return hipSuccess;
  if (a.l2norm)
    hipLaunchKernelGGL((fwd_ws_kernel<true, false, true>), dim3((unsigned)units, a.H, 2),
                       dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL(fwd_ws_kernel<true>, dim3((unsigned)units, a.H, 2), dim3(512), 0, stream, a);
  return hipGetLastError();
}

}  // namespace gdn
