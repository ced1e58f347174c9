// 2D index reordering (raster <-> Morton), a bit-exact permutation of token rows.
// Method: paper summary sec. 4.2 / Figure 2 and the article's sec. 四 (spatially coherent
// token order before 1D pooling).  HBM-bound copy: every lane moves 16-byte chunks, so each
// token row (128 or 256 B in bf16, 256 or 512 B in fp32) is read and written by whole
// contiguous segments.
#include "common.hpp"
#include "kernels.hpp"

namespace llsa {

constexpr int kReorderThreads = 256;
constexpr int kChunksPerThread = 4;

// chunks_per_row = row bytes / 16.  Forward: y[m] = x[raster(m)]; inverse: y[raster(m)] = x[m].
__global__ __launch_bounds__(kReorderThreads) void reorder_kernel(
    const i32x4* __restrict__ x, i32x4* __restrict__ y, int n, int hbits, int wbits,
    int cpr_shift, int inverse, long total_chunks) {
  const long base = ((long)blockIdx.x * kReorderThreads * kChunksPerThread) + threadIdx.x;
  i32x4 buf[kChunksPerThread];
  long dst[kChunksPerThread];
#pragma unroll
  for (int u = 0; u < kChunksPerThread; ++u) {
    const long c = base + (long)u * kReorderThreads;
    dst[u] = -1;
    if (c < total_chunks) {
      const long row = c >> cpr_shift;
      const int part = (int)(c & ((1 << cpr_shift) - 1));
      const long head = row >> (hbits + wbits);
      const int m = (int)(row & (n - 1));
      const long moved =
          (((head << (hbits + wbits)) + morton_to_raster(m, hbits, wbits)) << cpr_shift) + part;
      const long src = inverse ? c : moved;
      dst[u] = inverse ? moved : c;
      buf[u] = x[src];
    }
  }
#pragma unroll
  for (int u = 0; u < kChunksPerThread; ++u)
    if (dst[u] >= 0) y[dst[u]] = buf[u];
}

hipError_t launch_reorder(const Shape& s, const void* x, void* y, int inverse,
                          hipStream_t stream) {
  const int row_bytes = s.d * (s.bf16 ? 2 : 4);   // 128 .. 512: 8 .. 32 chunks per row
  int cpr_shift = 0;
  while ((16 << cpr_shift) < row_bytes) ++cpr_shift;
  const long total = (long)s.bh * s.n << cpr_shift;
  const long per_block = (long)kReorderThreads * kChunksPerThread;
  const long blocks = (total + per_block - 1) / per_block;
  LLSA_LAUNCH("reorder_kernel", reorder_kernel, dim3((unsigned)blocks), dim3(kReorderThreads), 0, stream,
                     (const i32x4*)x, (i32x4*)y, s.n, s.hbits, s.wbits, cpr_shift, inverse,
                     total);
  return hipGetLastError();
}

}  // namespace llsa
