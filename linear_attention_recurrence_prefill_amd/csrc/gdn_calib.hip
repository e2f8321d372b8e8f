// Calibration kernels: a stream copy (the HBM bandwidth a plain kernel reaches) and a loop of
// independent bf16 MFMAs on registers (the matrix-core rate).  They measure the ceilings the
// gated delta rule kernels are set against; they compute nothing of the operation.
#include "gdn_calib_internal.h"
#include "gdn_device.h"

namespace gdn {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;  // 16-byte loads in flight per lane

__global__ __launch_bounds__(kCopyThreads) void calib_copy_kernel(const u32x4 *__restrict__ src,
                                                                  u32x4 *__restrict__ dst,
                                                                  int64_t n) {
  constexpr int64_t kSpan = (int64_t)kCopyThreads * kCopyUnroll;
  const int64_t stride = (int64_t)gridDim.x * kSpan;
  int64_t i = (int64_t)blockIdx.x * kSpan + threadIdx.x;
  for (; i + (kCopyUnroll - 1) * kCopyThreads < n; i += stride) {
    u32x4 x[kCopyUnroll];
#pragma unroll
    for (int j = 0; j < kCopyUnroll; ++j) x[j] = __builtin_nontemporal_load(src + i + j * kCopyThreads);
#pragma unroll
    for (int j = 0; j < kCopyUnroll; ++j) __builtin_nontemporal_store(x[j], dst + i + j * kCopyThreads);
  }
#pragma unroll
  for (int j = 0; j < kCopyUnroll; ++j)  // this lane's part of the last, partial span
    if (i + j * kCopyThreads < n) dst[i + j * kCopyThreads] = src[i + j * kCopyThreads];
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Four independent 32 x 32 accumulators per wave: a round of four v_mfma_f32_32x32x16_bf16 is
// 4 x 32768 flop and keeps the matrix core busy across each instruction's latency.  (Eight
// 16 x 16 accumulators carried through the loop make the register allocator rotate them with
// register moves every round, which halves the rate.)
constexpr int kChains = 4;

__global__ __launch_bounds__(64) void calib_mfma_kernel(float *__restrict__ out, int iters) {
  const int lane = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (bf16)(0.001f * (float)((lane + j) & 7));
    b[j] = (bf16)(0.001f * (float)((lane * 3 + j) & 7));
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[c][j] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[c][j];
  out[(int64_t)blockIdx.x * 64 + lane] = s;
}

}  // namespace

hipError_t launch_calib_copy(const void *src, void *dst, int64_t units16, int cus,
                             hipStream_t stream) {
  const int64_t span = (int64_t)kCopyThreads * kCopyUnroll;
  const int64_t blocks = std::min<int64_t>((units16 + span - 1) / span, (int64_t)cus * 16);
  hipLaunchKernelGGL(calib_copy_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, stream,
                     static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), units16);
  return hipGetLastError();
}

hipError_t launch_calib_mfma(float *out, int waves, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(calib_mfma_kernel, dim3((unsigned)waves), dim3(64), 0, stream, out, iters);
  return hipGetLastError();
}

}  // namespace gdn
