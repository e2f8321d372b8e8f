// Internal interface of the backward's bf16, d = 128 kernels (gdn_bwd_chain.hip,
// gdn_bwd_grad.hip) and the reverse walk of the affine scan (gdn_fwd_split.hip).
#pragma once

#include "gdn_internal.h"

namespace gdn {

// Units of the reverse chain: the sequences split into segments of L chunks (L == 0: whole
// sequences), numbered as the forward numbers them (find_unit).
struct BwdUnits {
  int32_t L;
  int64_t units;
  // final pass: the state gradient at each unit's end [units, H, D, D] (null: dht, or zero)
  const float *unit_dend;
  // transition pass: [units, H, D, D], the state gradient at each unit's start from a zero end
  // gradient (B'); the unit's map of end to start gradient is the forward's M transposed
  float *unit_out;
  // truncate mode (final pass, L > 0): each unit's chain starts after its end, over the chunks
  // whose summed g reaches log_thr (warm_window_rev), from a zero gradient or dht at the
  // sequence's end; per-chunk outputs only for the unit's own chunks
  int32_t truncate;
  float log_thr;
};

// The reverse state-gradient chain.  Final pass: grid (units, H); per chunk it writes dh' (dhn),
// dR = Tm^T dDelta (into the ddelta slot, fp32 [T, H, D]) and dV.  Transition pass: grid
// (units, H), no per-chunk output, units that start a sequence are skipped.
hipError_t launch_bwd_chain_bf16(const BwdArgs &b, const BwdUnits &u, hipStream_t stream);
hipError_t launch_bwd_chain_bf16_transition(const BwdArgs &b, const BwdUnits &u,
                                            hipStream_t stream);
// Tm = (I + A)^-1 of every chunk from k, beta and the recompute's gamma, stored for the reverse
// chain as Tm^T = hi + lo: two bf16 64 x 64 tiles in its LDS layout (without the LDS copy's block
// padding), 16 KiB per (chunk, head).
hipError_t launch_bwd_tm(const BwdArgs &b, float *tmat, int64_t max_chunks, hipStream_t stream);
// Per-chunk gradients from the chain's dhn and dR (dV is the chain's).
hipError_t launch_bwd_grad_bf16(const BwdArgs &b, int64_t max_chunks, hipStream_t stream);
// The affine scan walked from each sequence's last unit to its first: S_end(u - 1) = M_u^T
// S_end(u) + B'_u from S_end(last) = s.h0 (dht, or zero), every unit's end state to s.unit_h0;
// s.unit_b holds B'_u and s.unit_m the forward's M_u transposed.
hipError_t launch_affine_scan_reverse(const SplitArgs &s, hipStream_t stream);

}  // namespace gdn
