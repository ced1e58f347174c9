// Sparse index transpose CSR -> CSC without atomics (paper summary sec. 4.1; the article's
// sec. 四 describes per-key counts, prefix-sum offsets and a flat vector of query ids).
//
// Every entry (row r, column c) becomes the 32-bit code (c << rbits) | r.  Sorting the codes
// groups entries by column with rows ascending, which is exactly the stable counting-sort
// order.  The sort is split into runs that are sorted independently; the CSC is then
// assembled from per-run column bounds, so that no kernel walks a long dependent chain of
// memory accesses.  No atomics anywhere, so the result is deterministic.
//  * tile_sort_kernel: bitonic sort of tiles of up to 4096 codes, 8 codes per thread in
//    registers (partners inside a thread in registers, in the same wave by cross-lane
//    shuffles, in other waves through LDS).  When the tiles are the final runs it also writes
//    the tile's column bounds lb[c] = #codes of the tile with column < c, c = 0..cols, by
//    binary searches in LDS (8 columns per thread in lockstep).
//  * merge_kernel: merges sorted runs pairwise (merge-path split, LDS staging); only used
//    while more than kMaxRuns runs remain.  csc_bounds_kernel then writes the bounds of the
//    merged runs (the same searches, in memory).
//  * csc_offsets_kernel (thread per column): off[c] = sum over runs of lb_r[c]; the run-r
//    codes of column c go to off[c] + sum_{r' < r} count_{r'}(c) onwards (runs are
//    consecutive row ranges of the CSR, so rows stay ascending).
//  * csc_scatter_kernel (thread per code): rows[start_r(c) + position in run - lb_r[c]].
// Codes of columns outside [0, cols) get the column `cols` and sort behind every kept entry.
#include "common.hpp"
#include "kernels.hpp"

namespace llsa {

constexpr int kPerThread = 8;
constexpr int kMaxTile = 4096;                     // codes per sort workgroup (512 threads)
constexpr int kMergeOut = 2048;                    // outputs per merge workgroup
constexpr int kMergeThreads = 256;
constexpr int kMaxRuns = 32;                       // sorted runs the CSC is assembled from

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
// lb[c] = first position of sorted codes[0, len) whose column is >= c, for the columns
// c = c_first + j * c_step, j < 8, searched in lockstep (8 independent binary searches).
// Column `cols` (where dropped entries sort) bounds the kept codes.
template <typename Codes>
__device__ __forceinline__ void column_bounds8(const Codes& codes, int len, int c_first, int c_step,
                                               int cols, int rbits, int32_t* lb) {
  int lo[8], hi[8];
  uint32_t key[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    lo[j] = 0;
    hi[j] = len;
    key[j] = (uint32_t)min(c_first + j * c_step, cols) << rbits;
  }
  for (int span = len; span > 0; span >>= 1) {   // ceil(log2(len + 1)) rounds
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (lo[j] < hi[j]) {
        const int mid = (lo[j] + hi[j]) >> 1;
        if (codes[mid] < key[j]) lo[j] = mid + 1;
        else hi[j] = mid;
      }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (c_first + j * c_step <= cols) lb[c_first + j * c_step] = lo[j];
}

template <int THREADS>
__global__ __launch_bounds__(THREADS) void tile_sort_kernel(const int32_t* __restrict__ csr,
                                                            uint32_t* __restrict__ out, int nnz,
                                                            int k, int cols, int rbits,
                                                            int tiles_per_mat,
                                                            int32_t* __restrict__ bounds) {
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
  if (bounds) {   // the tiles are the final runs: write this tile's column bounds
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) s[kPerThread * t + e] = v[e];
    __syncthreads();
    const int len = min(TILE, nnz - tile * TILE);
    int32_t* lb = bounds + (long)blockIdx.x * (cols + 1);
    for (int c0 = t; c0 <= cols; c0 += 8 * THREADS)
      column_bounds8(s, len, c0, THREADS, cols, rbits, lb);
  }
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

// Column bounds of merged runs: thread per (run, 8 columns), searching the run in memory.
__global__ __launch_bounds__(256) void csc_bounds_kernel(const uint32_t* __restrict__ codes,
                                                         int32_t* __restrict__ bounds, int nnz,
                                                         int cols, int rbits, int run,
                                                         int nruns) {
  const int mat = blockIdx.z;
  const int r = blockIdx.y;
  const int c0 = blockIdx.x * 256 * 8 + threadIdx.x;
  if (c0 > cols) return;
  const int len = min(run, nnz - r * run);
  const uint32_t* cm = codes + (long)mat * nnz + (long)r * run;
  column_bounds8(cm, len, c0, 256, cols, rbits, bounds + ((long)mat * nruns + r) * (cols + 1));
}

// Thread per column c = 0..cols: off[c], and start[r][c] = where run r's codes of column c go,
// minus lb_r[c] (so that a code at run position i lands at start[r][c] + i).
__global__ __launch_bounds__(256) void csc_offsets_kernel(const int32_t* __restrict__ bounds,
                                                          int32_t* __restrict__ start,
                                                          int32_t* __restrict__ off, int cols,
                                                          int nruns) {
  const int mat = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c > cols) return;
  const int32_t* lb = bounds + (long)mat * nruns * (cols + 1);
  int lo[kMaxRuns], hi[kMaxRuns];
  int total = 0;
#pragma unroll
  for (int r = 0; r < kMaxRuns; ++r) {
    lo[r] = hi[r] = 0;
    if (r < nruns) {
      lo[r] = lb[(long)r * (cols + 1) + c];
      if (c < cols) hi[r] = lb[(long)r * (cols + 1) + c + 1];
    }
    total += lo[r];
  }
  off[(long)mat * (cols + 1) + c] = total;
  if (c == cols) return;
  int32_t* st = start + (long)mat * nruns * cols;
  int acc = total;
#pragma unroll
  for (int r = 0; r < kMaxRuns; ++r)
    if (r < nruns) {
      st[(long)r * cols + c] = acc - lo[r];
      acc += hi[r] - lo[r];
    }
}

// Thread per code: its row goes to start[r][column] + its position in run r.
__global__ __launch_bounds__(256) void csc_scatter_kernel(const uint32_t* __restrict__ codes,
                                                          const int32_t* __restrict__ start,
                                                          int32_t* __restrict__ rows_out, int nnz,
                                                          int cols, int rbits, int run,
                                                          int nruns) {
  const int mat = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= nnz) return;
  const uint32_t code = codes[(long)mat * nnz + i];
  const int c = (int)(code >> rbits);
  if (c >= cols) return;   // dropped entry
  const int r = i / run;
  const int local = i - r * run;
  const uint32_t rmask = rbits ? ((1u << rbits) - 1u) : 0u;
  const int pos = start[((long)mat * nruns + r) * cols + c] + local;
  rows_out[(long)mat * nnz + pos] = (int32_t)(code & rmask);
}

static int ceil_log2(int v) {
  int b = 0;
  while ((1L << b) < v) ++b;
  return b;
}

struct TransposePlan {
  int threads;   // tile-sort workgroup size: tiles of threads * 8 codes
  int tile;
  int tiles;
  int run;       // length of the final sorted runs (after merges)
  int nruns;
};

static TransposePlan plan_transpose(int rows, int k) {
  TransposePlan p{};
  const int nnz = rows * k;
  p.threads = 64;   // the smallest tile that holds a matrix, up to 4096 codes
  while (p.threads * kPerThread < nnz && p.threads * kPerThread < kMaxTile) p.threads *= 2;
  p.tile = p.threads * kPerThread;
  p.tiles = (nnz + p.tile - 1) / p.tile;
  p.run = p.tile;
  while ((nnz + p.run - 1) / p.run > kMaxRuns) p.run <<= 1;
  p.nruns = (nnz + p.run - 1) / p.run;
  return p;
}

// Workspace: two code buffers [nmat, nnz], the run bounds [nmat, nruns, cols + 1] and the run
// starts [nmat, nruns, cols], each 256-byte aligned.
static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t transpose_workspace_bytes(int nmat, int rows, int cols, int k) {
  const TransposePlan p = plan_transpose(rows, k);
  const size_t nnz = (size_t)rows * k;
  return 2 * align256(sizeof(uint32_t) * nmat * nnz) +
         align256(sizeof(int32_t) * nmat * p.nruns * ((size_t)cols + 1)) +
         align256(sizeof(int32_t) * nmat * p.nruns * (size_t)cols);
}

hipError_t launch_index_transpose(int nmat, int rows, int cols, int k, const int32_t* csr,
                                  int32_t* off, int32_t* rows_out, void* ws,
                                  hipStream_t stream) {
  const int nnz = rows * k;
  const int rbits = ceil_log2(rows);
  const TransposePlan p = plan_transpose(rows, k);
  char* w = (char*)ws;
  const size_t code_bytes = align256(sizeof(uint32_t) * nmat * (size_t)nnz);
  uint32_t* buf[2] = {(uint32_t*)w, (uint32_t*)(w + code_bytes)};
  int32_t* bounds = (int32_t*)(w + 2 * code_bytes);
  int32_t* starts =
      (int32_t*)(w + 2 * code_bytes + align256(sizeof(int32_t) * nmat * p.nruns * ((size_t)cols + 1)));
  const bool merged = p.nruns < p.tiles;
  int32_t* tile_bounds = merged ? nullptr : bounds;
  const dim3 grid((unsigned)(nmat * p.tiles));
  switch (p.threads) {
    case 64:
      LLSA_LAUNCH("tile_sort_kernel", tile_sort_kernel<64>, grid, dim3(64), 0, stream, csr,
                  buf[0], nnz, k, cols, rbits, p.tiles, tile_bounds);
      break;
    case 128:
      LLSA_LAUNCH("tile_sort_kernel", tile_sort_kernel<128>, grid, dim3(128), 0, stream, csr,
                  buf[0], nnz, k, cols, rbits, p.tiles, tile_bounds);
      break;
    case 256:
      LLSA_LAUNCH("tile_sort_kernel", tile_sort_kernel<256>, grid, dim3(256), 0, stream, csr,
                  buf[0], nnz, k, cols, rbits, p.tiles, tile_bounds);
      break;
    default:
      LLSA_LAUNCH("tile_sort_kernel", tile_sort_kernel<512>, grid, dim3(512), 0, stream, csr,
                  buf[0], nnz, k, cols, rbits, p.tiles, tile_bounds);
      break;
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  int cur = 0;
  const unsigned mtiles = (unsigned)((nnz + kMergeOut - 1) / kMergeOut);
  for (int run = p.tile; run < p.run; run <<= 1) {
    LLSA_LAUNCH("merge_kernel", merge_kernel, dim3(mtiles, (unsigned)nmat), dim3(kMergeThreads),
                0, stream, buf[cur], buf[cur ^ 1], nnz, run);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    cur ^= 1;
  }
  const unsigned code_blocks = (unsigned)((nnz + 255) / 256);
  if (merged) {
    LLSA_LAUNCH("csc_bounds_kernel", csc_bounds_kernel,
                dim3((unsigned)((cols + 1 + 2047) / 2048), (unsigned)p.nruns, (unsigned)nmat),
                dim3(256), 0, stream, buf[cur], bounds, nnz, cols, rbits, p.run, p.nruns);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  LLSA_LAUNCH("csc_offsets_kernel", csc_offsets_kernel,
              dim3((unsigned)((cols + 1 + 255) / 256), (unsigned)nmat), dim3(256), 0, stream,
              bounds, starts, off, cols, p.nruns);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  LLSA_LAUNCH("csc_scatter_kernel", csc_scatter_kernel, dim3(code_blocks, (unsigned)nmat),
              dim3(256), 0, stream, buf[cur], starts, rows_out, nnz, cols, rbits, p.run,
              p.nruns);
  return hipGetLastError();
}

}  // namespace llsa
