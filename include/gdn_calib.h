/*
 * Calibration kernels of the measurement harness, in the same library as the gated delta rule
 * (libgdn_mi355x.so).  Neither is part of the operation: they measure the two ceilings that bound
 * it on the GPU at hand, so that a kernel's time can be set against peaks reached on the same
 * device as well as against the datasheet's (HBM bandwidth, the forward's bound; the bf16 matrix
 * rate, its second ceiling).
 *
 * Both enqueue one kernel on `stream` and return without synchronising; the caller times it with
 * events on that stream.  Device pointers only; nothing is allocated.  Errors: GDN_ERR_NULL_ARG for
 * a null pointer, GDN_ERR_BAD_ALIGNMENT for a pointer that is not 16-byte aligned,
 * GDN_ERR_BAD_SHAPE for a size out of range, GDN_ERR_UNSUPPORTED_ARCH off gfx950, GDN_ERR_HIP for a
 * failed launch (the detail from gdn_last_error()).
 */
#ifndef GDN_CALIB_H
#define GDN_CALIB_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#include "gdn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Stream copy: dst[0 .. bytes) = src[0 .. bytes), in 16-byte units by a grid-strided kernel that
 * keeps four loads in flight per lane.  bytes: a positive multiple of 16; src and dst 16-byte
 * aligned and not overlapping.  HBM bytes moved: 2 * bytes. */
gdn_status gdn_calib_copy(const void *src, void *dst, size_t bytes, hipStream_t stream);

/* bf16 matrix-core rate: `waves_per_cu * 256` waves each issue `iters` rounds of four
 * independent v_mfma_f32_32x32x16_bf16 (32 x 32 x 16 products, 32768 flop each) on operands held
 * in registers, and write one float per lane to out (size waves_per_cu * 256 * 64 floats) so the
 * work is kept.  Flop per call: waves_per_cu * 256 * iters * 4 * 32768.  waves_per_cu in 1..8,
 * iters in 1..2^20. */
gdn_status gdn_calib_mfma_bf16(float *out, int waves_per_cu, int iters, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_CALIB_H */
