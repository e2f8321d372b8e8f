// Device-side building blocks for the gfx950 gated delta rule kernels: vector types, MFMA
// wrappers, bf16 conversion and LDS fragment loads.
//
// MFMA lane layouts used throughout (wave64, lane l, group gq = l / 16, column c = l % 16):
//   v_mfma_f32_16x16x32_bf16  A[m][k]: lane m + 16 * (k / 8), item k % 8
//                             B[k][n]: lane n + 16 * (k / 8), item k % 8
//                             D[m][n]: lane n + 16 * (m / 4), item m % 4
//   v_mfma_f32_16x16x4_f32    A[m][k]: lane m + 16 * k;  B[k][n]: lane n + 16 * k;  D as above
// ds_read_b64_tr_b16 (16-lane groups): lane i of a group receives element i % 4 of the 8-byte
// words addressed by lanes i / 4, 4 + i / 4, 8 + i / 4, 12 + i / 4 of that group, in that
// order.  When lane j = 4 r + q of the group addresses row (base + r), column (n0 + 4 q) of a
// row-major bf16 matrix, lane i receives rows base..base+3 of column n0 + i: a column-major
// MFMA operand read from row-major storage.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define GDN_LDS __attribute__((address_space(3)))

__device__ __forceinline__ f32x4 mma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_16x16x16_bf16: A[m][k] at lane m + 16 (k / 4), item k % 4; B[k][n] at lane
// n + 16 (k / 4), item k % 4 (so a D-layout accumulator is a B operand as it stands).
__device__ __forceinline__ f32x4 mma_bf16_k16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                    __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Keeps the instruction scheduler from moving work across this point (bounds how far ahead
// loads are issued, and with it register pressure).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
// Tile t of the ten 16 x 16 tiles on and below the diagonal of a 64 x 64 matrix, numbered row by
// row (t = r (r + 1) / 2 + i): its block row r and block column i <= r.  Scalar arithmetic, for
// a wave-uniform t.
__device__ __forceinline__ void tri_tile(int t, int &r, int &i) {
  r = (t >= 1) + (t >= 3) + (t >= 6);
  i = t - r * (r + 1) / 2;
}
__device__ __forceinline__ bf16x4 lo4(bf16x8 x) { return __builtin_shufflevector(x, x, 0, 1, 2, 3); }
__device__ __forceinline__ bf16x4 hi4(bf16x8 x) { return __builtin_shufflevector(x, x, 4, 5, 6, 7); }

// Round to nearest even.  Converted in pairs so that each pair packs into one dword with one
// instruction (a 4-wide conversion is split into single conversions and byte permutes when its
// result is reinterpreted as integers).
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 lo = __builtin_convertvector((f32x2{x[0], x[1]}), bf16x2);
  const bf16x2 hi = __builtin_convertvector((f32x2{x[2], x[3]}), bf16x2);
  return __builtin_bit_cast(bf16x4, (uint2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)}));
}

__device__ __forceinline__ bf16x8 to_bf16x8(f32x4 a, f32x4 b) {
  return cat8(to_bf16x4(a), to_bf16x4(b));
}

// 4 consecutive bf16 (8 bytes, 8-byte aligned) from LDS.
__device__ __forceinline__ bf16x4 lds_bf16x4(const bf16 *p) {
  return *reinterpret_cast<const bf16x4 *>(p);
}
// 8 consecutive bf16 (16 bytes, 16-byte aligned) from LDS.
__device__ __forceinline__ bf16x8 lds_bf16x8(const bf16 *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}
// 4 consecutive fp32 (16 bytes, 16-byte aligned) from LDS.
__device__ __forceinline__ f32x4 lds_f32x4(const float *p) {
  return *reinterpret_cast<const f32x4 *>(p);
}

// Transposing 8-byte LDS read (see the layout note above).  p must be 8-byte aligned.
__device__ __forceinline__ bf16x4 lds_tr16(const bf16 *p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GDN_LDS i16x4 *)((GDN_LDS char *)p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <class E>
__device__ __forceinline__ E from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) {
  return x;
}
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) {
  return (bf16)x;
}

// A workgroup barrier that orders LDS accesses only: this wave's LDS reads and writes are complete
// before it (lgkmcnt(0)); its global loads and stores may still be in flight.  The signal fences
// keep the compiler from moving memory accesses across it.  (__syncthreads() would also wait
// for every outstanding global load, direct global->LDS loads of a next tile included.)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// A direct global->LDS load of 16 bytes per lane (lane l writes l_base + 16 l) that the
// compiler does not track.  With the builtin, the compiler makes any later LDS read that it cannot
// prove disjoint (a transposing read, for one) wait until the load has landed, which serialises a
// next-tile prefetch with the current tile's work.  The caller must wait for these loads itself
// (s_waitcnt vmcnt(0)) before the data is read, and must not read or write the destination
// until then.  The compiler's own vmcnt waits stay correct: loads retire in order, so an extra
// load in flight only makes a wait stricter.
__device__ __forceinline__ void dma16_untracked(const void *g, const void *l_base) {
  const unsigned la = __builtin_amdgcn_readfirstlane(
      (unsigned)(unsigned long)(__attribute__((address_space(3))) const void *)l_base);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "{m0}"(la) : "memory");
}

// Wave-wide inclusive prefix sum (64 lanes).
__device__ __forceinline__ float wave_inclusive_scan(float x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    float y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  return x;
}

// Wave-wide inclusive prefix sum (64 lanes) with DPP lane moves only (no LDS traffic): Hillis-
// Steele shifts 1, 2, 4, 8 within each row of 16 lanes (row_shr, lanes shifted in from outside the
// row read 0), then row 0's total added to row 1 and row 2's to row 3 (row_bcast:15), then the
// total of rows 0-1 added to rows 2 and 3 (row_bcast:31).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_moved(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, true));
}
__device__ __forceinline__ float wave_inclusive_scan_dpp(float x) {
  x += dpp_moved<0x111, 0xf>(x);  // row_shr:1
  x += dpp_moved<0x112, 0xf>(x);  // row_shr:2
  x += dpp_moved<0x114, 0xf>(x);  // row_shr:4
  x += dpp_moved<0x118, 0xf>(x);  // row_shr:8
  x += dpp_moved<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x += dpp_moved<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

// Sum over each row of 16 lanes (lanes 16 j .. 16 j + 15) with DPP lane moves only: pairs
// (quad_perm 1,0,3,2), quads (quad_perm 2,3,0,1), half-rows (row_half_mirror), rows (row_mirror).
// Every lane of a row receives the same bits (each step adds two equal partial sums in either
// order), and the order is fixed, so the result is reproducible.
__device__ __forceinline__ float row16_sum_dpp(float x) {
  x += dpp_moved<0xB1, 0xf>(x);
  x += dpp_moved<0x4E, 0xf>(x);
  x += dpp_moved<0x141, 0xf>(x);
  x += dpp_moved<0x140, 0xf>(x);
  return x;
}

// Wave-wide sum in fp64 (64 lanes); every lane receives the total.
__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

}  // namespace gdn
