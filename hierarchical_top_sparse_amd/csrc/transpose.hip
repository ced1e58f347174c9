// Sparse index transpose CSR -> CSC without atomics (paper summary sec. 4.1; the article's
// sec. 四 describes per-key counts, prefix-sum offsets and a flat vector of query ids).
//
// Every entry (row r, column c) becomes the 32-bit code (c << rbits) | r.  Sorting the codes
// groups entries by column with rows ascending, which is exactly the stable counting-sort
// order; the per-column counts and their prefix sum are then read off the sorted codes as run
// boundaries.  Sorting is a bitonic sort of 2048-code tiles in LDS followed by merge passes in
// which every code finds its output position by a binary search in the partner run.  No
// atomics anywhere, so the result is deterministic.  Codes of columns outside [0, cols) get
// the column `cols` and sort behind every kept entry.
#include "common.hpp"
#include "kernels.hpp"

namespace llsa {

constexpr int kTile = 2048;
constexpr int kTileThreads = 256;

__global__ __launch_bounds__(kTileThreads) void tile_sort_kernel(
    const int32_t* __restrict__ csr, uint32_t* __restrict__ out, int nnz, int k, int cols,
    int rbits, int tiles_per_mat) {
  __shared__ uint32_t s[kTile];
  const int mat = blockIdx.x / tiles_per_mat;
  const int tile = blockIdx.x - mat * tiles_per_mat;
  const int32_t* in = csr + (long)mat * nnz;
  const int t = threadIdx.x;
  for (int e = t; e < kTile; e += kTileThreads) {
    const int idx = tile * kTile + e;
    uint32_t code = 0xffffffffu;
    if (idx < nnz) {
      int c = in[idx];
      if (c < 0 || c >= cols) c = cols;
      code = ((uint32_t)c << rbits) | (uint32_t)(idx / k);
    }
    s[e] = code;
  }
  __syncthreads();
  for (int size = 2; size <= kTile; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = t; i < kTile; i += kTileThreads) {
        const int j = i ^ stride;
        if (j > i) {
          const uint32_t a = s[i], b = s[j];
          const bool ascending = (i & size) == 0;
          if ((a > b) == ascending) {
            s[i] = b;
            s[j] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  uint32_t* dst = out + (long)mat * nnz;
  for (int e = t; e < kTile; e += kTileThreads) {
    const int idx = tile * kTile + e;
    if (idx < nnz) dst[idx] = s[e];
  }
}

// Merge sorted runs of length `run` pairwise.  A code of the left run goes after the partner
// codes strictly smaller than it; a code of the right run after the left codes <= it.
__global__ __launch_bounds__(256) void merge_pass_kernel(const uint32_t* __restrict__ in,
                                                         uint32_t* __restrict__ out, int nnz,
                                                         int run, long total) {
  const long gi = (long)blockIdx.x * 256 + threadIdx.x;
  if (gi >= total) return;
  const int mat = (int)(gi / nnz);
  const int i = (int)(gi - (long)mat * nnz);
  const uint32_t* a = in + (long)mat * nnz;
  const int r = i / run;
  const int pair_start = (r & ~1) * run;
  const uint32_t x = a[i];
  const bool left = (r & 1) == 0;
  const int p0 = left ? pair_start + run : pair_start;
  const int p1 = left ? min(pair_start + 2 * run, nnz) : pair_start + run;
  int lo = p0, hi = max(p0, p1);   // search in [p0, p1)
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const uint32_t y = a[mid];
    const bool go_right = left ? (y < x) : (y <= x);
    if (go_right) lo = mid + 1;
    else hi = mid;
  }
  const int own_start = left ? pair_start : pair_start + run;
  const int pos = pair_start + (i - own_start) + (lo - p0);
  out[(long)mat * nnz + pos] = x;
}

// off[c] = first sorted position whose column is >= c; rows = low bits of the codes.
__global__ __launch_bounds__(256) void csc_finalize_kernel(const uint32_t* __restrict__ codes,
                                                           int32_t* __restrict__ off,
                                                           int32_t* __restrict__ rows_out,
                                                           int nnz, int cols, int rbits,
                                                           long total) {
  const long gi = (long)blockIdx.x * 256 + threadIdx.x;
  if (gi >= total) return;
  const int mat = (int)(gi / nnz);
  const int i = (int)(gi - (long)mat * nnz);
  const uint32_t* c = codes + (long)mat * nnz;
  int32_t* o = off + (long)mat * (cols + 1);
  const uint32_t code = c[i];
  const uint32_t rmask = rbits ? ((1u << rbits) - 1u) : 0u;
  rows_out[(long)mat * nnz + i] = (int32_t)(code & rmask);
  const int key = (int)(code >> rbits);
  const int prev = i > 0 ? (int)(c[i - 1] >> rbits) : -1;
  for (int kk = prev + 1; kk <= key && kk <= cols; ++kk) o[kk] = i;
  if (i == nnz - 1)
    for (int kk = key + 1; kk <= cols; ++kk) o[kk] = nnz;
}

static int ceil_log2(int v) {
  int b = 0;
  while ((1L << b) < v) ++b;
  return b;
}

size_t transpose_workspace_bytes(int nmat, int rows, int cols, int k) {
  (void)cols;
  return 2 * sizeof(uint32_t) * (size_t)nmat * (size_t)rows * (size_t)k;
}

hipError_t launch_index_transpose(int nmat, int rows, int cols, int k, const int32_t* csr,
                                  int32_t* off, int32_t* rows_out, void* ws,
                                  hipStream_t stream) {
  const int nnz = rows * k;
  const int rbits = ceil_log2(rows);
  const int tiles = (nnz + kTile - 1) / kTile;
  uint32_t* buf[2] = {(uint32_t*)ws, (uint32_t*)ws + (size_t)nmat * nnz};
  hipLaunchKernelGGL(tile_sort_kernel, dim3((unsigned)(nmat * tiles)), dim3(kTileThreads), 0,
                     stream, csr, buf[0], nnz, k, cols, rbits, tiles);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const long total = (long)nmat * nnz;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  int cur = 0;
  for (int run = kTile; run < nnz; run <<= 1) {
    hipLaunchKernelGGL(merge_pass_kernel, dim3(blocks), dim3(256), 0, stream, buf[cur],
                       buf[cur ^ 1], nnz, run, total);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    cur ^= 1;
  }
  hipLaunchKernelGGL(csc_finalize_kernel, dim3(blocks), dim3(256), 0, stream, buf[cur], off,
                     rows_out, nnz, cols, rbits, total);
  return hipGetLastError();
}

}  // namespace llsa
