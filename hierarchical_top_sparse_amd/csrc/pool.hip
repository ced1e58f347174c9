// Hierarchical compression: recursive mean pooling of Q, K and V (paper summary sec. 三:
// level l has N / B^l tokens, each the mean of B level-(l-1) tokens).
//
// pool12_{bf16,f32}_kernel: one workgroup per (tensor, head, group of B level-1 blocks = B^2
//   tokens).  Reads the B^2 token rows once, every thread's loads in flight together
//   (coalesced 128/256-byte rows; raster layout reads 4x4 tiles as 4 row segments), writes
//   level 1 and reduces level 2 through LDS.  HBM-bound.
//   With B = 64 (8x8 tiles) the kernel writes the 64-token means instead, each the mean of four
//   consecutive 16-token means staged in LDS, and no second level.
// pool_next_kernel: level l from level l-1 (fp32, tiny): l >= 3 for B = 16, l >= 2 for B = 64.
// All sums are fp32 in a fixed order; the 1/B factor is exact.  pool12_kernel is the profiling
// name of both level-1/2 kernels.  Rows of 128 channels are pooled as two 64-channel slices.
#include "common.hpp"
#include "kernels.hpp"
#include "pool_impl.hpp"

namespace llsa {

template <int D>
__global__ __launch_bounds__(256) void pool12_bf16_kernel(PoolArgs args, int n, Grid grid,
                                                          int groups_per_head) {
  __shared__ __attribute__((aligned(16))) float sh[kBlock][D];
  pool12_bf16_group<D>(args, n, grid, groups_per_head, blockIdx.y, blockIdx.x, sh);
}

template <int D>
__global__ __launch_bounds__(256) void pool12_f32_kernel(PoolArgs args, int n, Grid grid,
                                                         int groups_per_head) {
  __shared__ __attribute__((aligned(16))) float sh[kBlock][D];
  pool12_f32_group<D>(args, n, grid, groups_per_head, blockIdx.y, blockIdx.x, sh);
}

template <int B, int D>
__global__ __launch_bounds__(256) void pool_next_kernel(PoolNextArgs args, long total_out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < total_out) pool_next_elem<B, D>(args, blockIdx.y, i);
}

hipError_t launch_pool(const Shape& s, const void* const x[3], float* const* lv[3],
                       hipStream_t stream) {
  PoolArgs a{};
  int nt = 0;
  for (int t = 0; t < 3; ++t) {
    if (!x[t]) continue;
    a.x[nt] = x[t];
    if (s.bshift == 4) {
      a.lv1[nt] = lv[t][0];
      a.lv2[nt] = s.levels >= 2 ? lv[t][1] : nullptr;
    } else {
      a.lv64[nt] = lv[t][0];
    }
    ++nt;
  }
  if (nt == 0) return hipSuccess;
  const int groups_per_head = s.n >> (2 * kBlockShift);
  const Grid grid{s.hbits, s.wbits, s.raster};
  const dim3 blocks((unsigned)(s.bh * groups_per_head), (unsigned)nt);
  if (s.bf16 && s.d == 64)
    LLSA_LAUNCH("pool12_kernel", pool12_bf16_kernel<64>, blocks, dim3(256), 0, stream, a, s.n,
                grid, groups_per_head);
  else if (s.bf16)
    LLSA_LAUNCH("pool12_kernel", pool12_bf16_kernel<128>, blocks, dim3(256), 0, stream, a, s.n,
                grid, groups_per_head);
  else if (s.d == 64)
    LLSA_LAUNCH("pool12_kernel", pool12_f32_kernel<64>, blocks, dim3(256), 0, stream, a, s.n,
                grid, groups_per_head);
  else
    LLSA_LAUNCH("pool12_kernel", pool12_f32_kernel<128>, blocks, dim3(256), 0, stream, a, s.n,
                grid, groups_per_head);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  for (int l = s.bshift == 4 ? 3 : 2; l <= s.levels; ++l) {
    PoolNextArgs b{};
    int m = 0;
    for (int t = 0; t < 3; ++t) {
      if (!x[t] || !lv[t][l - 1]) continue;
      if (!lv[t][l - 2]) return hipErrorInvalidValue;   // the level below was not stored
      b.in[m] = lv[t][l - 2];
      b.out[m] = lv[t][l - 1];
      ++m;
    }
    if (m == 0) continue;
    const long total = (long)s.bh * s.n_level(l) * s.d;
    const dim3 grid((unsigned)((total + 255) / 256), (unsigned)m);
    if (s.bshift == 4 && s.d == 64)
      LLSA_LAUNCH("pool_next_kernel", (pool_next_kernel<16, 64>), grid, dim3(256), 0, stream, b,
                  total);
    else if (s.bshift == 4)
      LLSA_LAUNCH("pool_next_kernel", (pool_next_kernel<16, 128>), grid, dim3(256), 0, stream, b,
                  total);
    else if (s.d == 64)
      LLSA_LAUNCH("pool_next_kernel", (pool_next_kernel<64, 64>), grid, dim3(256), 0, stream, b,
                  total);
    else
      LLSA_LAUNCH("pool_next_kernel", (pool_next_kernel<64, 128>), grid, dim3(256), 0, stream, b,
                  total);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace llsa
