// Dense block mask of the fine selection, for the mask-based comparator of the sparse
// backward.  The article's sec. 4.1 contrasts LLSA's index transpose with sparse attention
// kernels whose backward builds a T x T binary mask and so pays O(T^2) again; its Figure 4
// measures such a dense-mask baseline of the KV backward.  Here the mask is one byte per
// (query block, key block) pair at level 1, query-major as the forward's indices give it:
// mask[bh][a][c] = 1 iff c is in Sel_1[a].  Building it clears bh * n_1^2 bytes (HBM-bound)
// and then sets bh * n_1 * K of them.
#include "common.hpp"
#include "kernels.hpp"

namespace llsa {

constexpr int kMaskThreads = 256;
constexpr int kMaskChunks = 4;   // 16-byte chunks cleared per thread

__global__ __launch_bounds__(kMaskThreads) void mask_clear_kernel(i32x4* __restrict__ m,
                                                                  long chunks) {
  const long base = (long)blockIdx.x * kMaskThreads * kMaskChunks + threadIdx.x;
#pragma unroll
  for (int u = 0; u < kMaskChunks; ++u) {
    const long c = base + (long)u * kMaskThreads;
    if (c < chunks) m[c] = i32x4{0, 0, 0, 0};
  }
}

// One thread per pick (row a, slot i) of every (batch, head).
__global__ __launch_bounds__(kMaskThreads) void mask_set_kernel(const int32_t* __restrict__ sel,
                                                                uint8_t* __restrict__ m, int n1,
                                                                int k, long picks) {
  const long t = (long)blockIdx.x * kMaskThreads + threadIdx.x;
  if (t >= picks) return;
  const long row = t / k;   // bh * n1 + a
  const int c = sel[t];
  if (c >= 0 && c < n1) m[row * n1 + c] = 1;
}

hipError_t launch_block_mask(const Shape& s, const int32_t* sel1, uint8_t* mask,
                             hipStream_t stream) {
  const long n1 = s.n >> 4;   // 16-token blocks
  const long chunks = (long)s.bh * n1 * n1 / 16;   // n1 is a multiple of 16
  const long per_block = (long)kMaskThreads * kMaskChunks;
  LLSA_LAUNCH("mask_clear_kernel", mask_clear_kernel,
              dim3((unsigned)((chunks + per_block - 1) / per_block)), dim3(kMaskThreads), 0,
              stream, (i32x4*)mask, chunks);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const long picks = (long)s.bh * n1 * s.topk;
  LLSA_LAUNCH("mask_set_kernel", mask_set_kernel,
              dim3((unsigned)((picks + kMaskThreads - 1) / kMaskThreads)), dim3(kMaskThreads), 0,
              stream, sel1, mask, (int)n1, s.topk, picks);
  return hipGetLastError();
}

}  // namespace llsa
