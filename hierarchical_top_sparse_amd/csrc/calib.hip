// Calibration kernels: the achievable peaks the roofline fractions are also quoted against
// (not part of the method).
//  * copy_kernel: a plain streaming copy, 16 bytes per lane, 4 loads in flight per thread, so
//    that read + write bytes over time is the HBM bandwidth a kernel can reach;
//  * mfma_kernel: every wave runs chains of v_mfma_f32_16x16x32_bf16 with no memory traffic,
//    kMfmaChains independent accumulators so that the matrix core never waits on a result.
#include "common.hpp"
#include "kernels.hpp"

namespace llsa {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
constexpr int kMfmaChains = 8;

__global__ __launch_bounds__(kCopyThreads) void copy_kernel(const i32x4* __restrict__ src,
                                                            i32x4* __restrict__ dst,
                                                            long chunks) {
  const long base = (long)blockIdx.x * kCopyThreads * kCopyUnroll + threadIdx.x;
  i32x4 v[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const long c = base + (long)u * kCopyThreads;
    if (c < chunks) v[u] = src[c];
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const long c = base + (long)u * kCopyThreads;
    if (c < chunks) dst[c] = v[u];
  }
}

// A = B = all ones: after `iters` rounds every accumulator element is 32 * iters (exact in fp32
// up to 2^24).  Each thread stores the sum of its chains' first elements.
__global__ __launch_bounds__(256) void mfma_kernel(float* __restrict__ out, int iters) {
  bf16x8 a;
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = (bf16)1.0f;
  f32x4 acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = mfma_bf16_k32(a, a, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) s += acc[c][0];
  out[(long)blockIdx.x * 256 + threadIdx.x] = s;
}

hipError_t launch_calib_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  const long chunks = (long)(bytes / 16);
  const long per_block = (long)kCopyThreads * kCopyUnroll;
  LLSA_LAUNCH("copy_kernel", copy_kernel, dim3((unsigned)((chunks + per_block - 1) / per_block)),
              dim3(kCopyThreads), 0, stream, (const i32x4*)src, (i32x4*)dst, chunks);
  return hipGetLastError();
}

hipError_t launch_calib_mfma(float* out, int blocks, int iters, hipStream_t stream) {
  LLSA_LAUNCH("mfma_kernel", mfma_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, out,
              iters);
  return hipGetLastError();
}

}  // namespace llsa
