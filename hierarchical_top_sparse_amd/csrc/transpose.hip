// Sparse index transpose CSR -> CSC without atomics (paper summary sec. 4.1; the article's
// sec. 四 describes per-key counts, prefix-sum offsets and a flat vector of query ids).
//
// Every entry (row r, column c) becomes the 32-bit code (c << rbits) | r.  Sorting the codes
// groups entries by column with rows ascending, which is exactly the stable counting-sort
// order; the per-column counts and their prefix sum are then read off the sorted codes as run
// boundaries.  No atomics anywhere, so the result is deterministic.
//  * tile_sort_kernel: bitonic sort of 4096-code tiles, 8 codes per thread in registers.
//    Compare-exchange partners inside a thread are handled in registers, partners in the same
//    wave by cross-lane shuffles, and only partners in other waves go through LDS.
//  * merge_kernel: merges sorted runs pairwise; each workgroup owns 2048 consecutive outputs,
//    finds its input ranges by a merge-path search, stages them in LDS and merges there.
//  * csc_finalize_kernel: row ids are the low bits of the codes; off[c] = first position whose
//    column is >= c.
// Codes of columns outside [0, cols) get the column `cols` and sort behind every kept entry.
#include "common.hpp"
#include "kernels.hpp"

namespace llsa {

constexpr int kPerThread = 8;
constexpr int kMaxTile = 4096;                     // codes per sort workgroup (512 threads)
constexpr int kMergeOut = 2048;                    // outputs per merge workgroup
constexpr int kMergeThreads = 256;

__device__ __forceinline__ void cmp_swap(uint32_t& lo, uint32_t& hi, bool asc) {
  const uint32_t a = lo, b = hi;
  const uint32_t mn = a < b ? a : b;
  const uint32_t mx = a < b ? b : a;
  lo = asc ? mn : mx;
  hi = asc ? mx : mn;
}

// One bitonic stage (block size SIZE, partner distance J) on this thread's 8 codes.
template <int SIZE, int J, int THREADS>
__device__ __forceinline__ void bitonic_stage(uint32_t (&v)[kPerThread], uint32_t* s, int t) {
  if constexpr (J < kPerThread) {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e)
      if ((e & J) == 0) cmp_swap(v[e], v[e | J], ((kPerThread * t + e) & SIZE) == 0);
  } else {
    constexpr int TJ = J / kPerThread;   // partner thread is t ^ TJ
    uint32_t p[kPerThread];
    if constexpr (TJ < 64) {
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) p[e] = (uint32_t)__shfl_xor((int)v[e], TJ, 64);
    } else {
      __syncthreads();
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) s[kPerThread * t + e] = v[e];
      __syncthreads();
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) p[e] = s[kPerThread * (t ^ TJ) + e];
    }
    const int i = kPerThread * t;
    const bool keep_min = ((i & J) == 0) == ((i & SIZE) == 0);
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const uint32_t mn = v[e] < p[e] ? v[e] : p[e];
      const uint32_t mx = v[e] < p[e] ? p[e] : v[e];
      v[e] = keep_min ? mn : mx;
    }
  }
}

template <int SIZE, int J, int THREADS>
__device__ __forceinline__ void bitonic_merge_steps(uint32_t (&v)[kPerThread], uint32_t* s,
                                                    int t) {
  bitonic_stage<SIZE, J, THREADS>(v, s, t);
  if constexpr (J > 1) bitonic_merge_steps<SIZE, J / 2, THREADS>(v, s, t);
}

template <int SIZE, int TILE, int THREADS>
__device__ __forceinline__ void bitonic_sort(uint32_t (&v)[kPerThread], uint32_t* s, int t) {
  bitonic_merge_steps<SIZE, SIZE / 2, THREADS>(v, s, t);
  if constexpr (SIZE < TILE) bitonic_sort<SIZE * 2, TILE, THREADS>(v, s, t);
}

// Sorts tiles of THREADS * 8 codes; tile i of matrix m covers entries [i*TILE, +TILE).
template <int THREADS>
__global__ __launch_bounds__(THREADS) void tile_sort_kernel(const int32_t* __restrict__ csr,
                                                            uint32_t* __restrict__ out, int nnz,
                                                            int k, int cols, int rbits,
                                                            int tiles_per_mat) {
  constexpr int TILE = THREADS * kPerThread;
  __shared__ uint32_t s[TILE];
  const int mat = blockIdx.x / tiles_per_mat;
  const int tile = blockIdx.x - mat * tiles_per_mat;
  const int32_t* in = csr + (long)mat * nnz;
  const int t = threadIdx.x;
  const int base = tile * TILE + kPerThread * t;   // this thread's 8 consecutive codes
  uint32_t v[kPerThread];
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int idx = base + e;
    uint32_t code = 0xffffffffu;
    if (idx < nnz) {
      int c = in[idx];
      if (c < 0 || c >= cols) c = cols;
      code = ((uint32_t)c << rbits) | (uint32_t)(idx / k);
    }
    v[e] = code;
  }
  bitonic_sort<2, TILE, THREADS>(v, s, t);
  uint32_t* dst = out + (long)mat * nnz;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e)
    if (base + e < nnz) dst[base + e] = v[e];
}

// Number of the first `diag` merged outputs that come from A (ties: A first), searched by the
// whole workgroup: every round each thread tests one probe, narrowing [lo, hi) 256-fold.
__device__ int merge_split_wg(const uint32_t* A, int la, const uint32_t* B, int lb, int diag,
                              int* scratch) {
  int lo = diag > lb ? diag - lb : 0;
  int hi = diag < la ? diag : la;
  while (hi - lo > 0) {
    const int span = hi - lo;
    const int step = (span + kMergeThreads - 1) / kMergeThreads;
    const int probe = lo + threadIdx.x * step;
    // predicate "A[probe] <= B[diag-1-probe]" is true for probe < split, false after
    const bool in_range = probe < hi;
    const bool pred = in_range && A[probe] <= B[diag - 1 - probe];
    __syncthreads();
    if (threadIdx.x == 0) scratch[0] = 0;
    __syncthreads();
    // the last probe with pred true bounds the split from below; the first false from above
    const unsigned long long m = __ballot(pred);
    if ((threadIdx.x & 63) == 0) scratch[1 + (threadIdx.x >> 6)] = __popcll(m);
    __syncthreads();
    int cnt = 0;
#pragma unroll
    for (int w = 0; w < kMergeThreads / 64; ++w) cnt += scratch[1 + w];
    // probes 0..cnt-1 are true (monotone): split lies in (lo + (cnt-1)*step, lo + cnt*step]
    const int new_lo = cnt > 0 ? lo + (cnt - 1) * step + 1 : lo;
    const int new_hi = min(hi, lo + cnt * step);
    if (step == 1) return new_hi > new_lo ? new_lo : new_lo;   // exact: split = lo + cnt
    lo = new_lo;
    hi = new_hi;
  }
  return lo;
}

// Number of the first `diag` merged outputs that come from A (ties: A first); serial search.
__device__ __forceinline__ int merge_split(const uint32_t* A, int la, const uint32_t* B, int lb,
                                           int diag) {
  int lo = diag > lb ? diag - lb : 0;
  int hi = diag < la ? diag : la;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (A[mid] <= B[diag - 1 - mid]) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// Merge sorted runs of length `run` pairwise; workgroup (x, mat) writes outputs
// [x * kMergeOut, +kMergeOut) of matrix mat.
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const uint32_t* __restrict__ in,
                                                             uint32_t* __restrict__ out, int nnz,
                                                             int run) {
  __shared__ uint32_t sa[kMergeOut];
  __shared__ uint32_t sb[kMergeOut];
  __shared__ int scratch[8];
  const int mat = blockIdx.y;
  const int o0 = blockIdx.x * kMergeOut;
  if (o0 >= nnz) return;
  const int o1 = min(o0 + kMergeOut, nnz);
  const uint32_t* src = in + (long)mat * nnz;
  const int pair_start = (o0 / (2 * run)) * (2 * run);
  const int la = min(run, nnz - pair_start);
  const int lb = max(0, min(run, nnz - pair_start - run));
  const uint32_t* A = src + pair_start;
  const uint32_t* B = src + pair_start + la;
  const int a0 = merge_split_wg(A, la, B, lb, o0 - pair_start, scratch);
  const int a1 = merge_split_wg(A, la, B, lb, o1 - pair_start, scratch);
  const int b0 = (o0 - pair_start) - a0, b1 = (o1 - pair_start) - a1;
  const int na = a1 - a0, nb = b1 - b0;
  for (int e = threadIdx.x; e < na; e += kMergeThreads) sa[e] = A[a0 + e];
  for (int e = threadIdx.x; e < nb; e += kMergeThreads) sb[e] = B[b0 + e];
  __syncthreads();
  // each thread merges 8 consecutive outputs
  const int d0 = threadIdx.x * 8;
  const int total = na + nb;
  if (d0 >= total) return;
  int ia = merge_split(sa, na, sb, nb, d0);
  int ib = d0 - ia;
  uint32_t* dst = out + (long)mat * nnz + o0 + d0;
  const int cnt = min(8, total - d0);
  for (int e = 0; e < cnt; ++e) {
    const bool take_a = ib >= nb || (ia < na && sa[ia] <= sb[ib]);
    dst[e] = take_a ? sa[ia++] : sb[ib++];
  }
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
  uint32_t* buf[2] = {(uint32_t*)ws, (uint32_t*)ws + (size_t)nmat * nnz};
  // the smallest tile that holds a matrix, up to 4096 codes (then merge passes)
  int threads = 64;
  while (threads * kPerThread < nnz && threads * kPerThread < kMaxTile) threads *= 2;
  const int tile = threads * kPerThread;
  const int tiles = (nnz + tile - 1) / tile;
  const dim3 grid((unsigned)(nmat * tiles));
  switch (threads) {
    case 64:
      LLSA_LAUNCH("tile_sort_kernel", tile_sort_kernel<64>, grid, dim3(64), 0, stream, csr, buf[0], nnz, k,
                         cols, rbits, tiles);
      break;
    case 128:
      LLSA_LAUNCH("tile_sort_kernel", tile_sort_kernel<128>, grid, dim3(128), 0, stream, csr, buf[0], nnz, k,
                         cols, rbits, tiles);
      break;
    case 256:
      LLSA_LAUNCH("tile_sort_kernel", tile_sort_kernel<256>, grid, dim3(256), 0, stream, csr, buf[0], nnz, k,
                         cols, rbits, tiles);
      break;
    default:
      LLSA_LAUNCH("tile_sort_kernel", tile_sort_kernel<512>, grid, dim3(512), 0, stream, csr, buf[0], nnz, k,
                         cols, rbits, tiles);
      break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  int cur = 0;
  const unsigned mtiles = (unsigned)((nnz + kMergeOut - 1) / kMergeOut);
  for (int run = tile; run < nnz; run <<= 1) {
    LLSA_LAUNCH("merge_kernel", merge_kernel, dim3(mtiles, (unsigned)nmat), dim3(kMergeThreads), 0,
                       stream, buf[cur], buf[cur ^ 1], nnz, run);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    cur ^= 1;
  }
  const long total = (long)nmat * nnz;
  LLSA_LAUNCH("csc_finalize_kernel", csc_finalize_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     stream, buf[cur], off, rows_out, nnz, cols, rbits, total);
  return hipGetLastError();
}

}  // namespace llsa
