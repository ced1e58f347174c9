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
//
// Matrices of at most kMaxRadixTiles tiles take a shorter path of two launches (several
// matrices, e.g. every level of a problem, in the same two launches):
//  * csc_radix_kernel: a stable LSD radix sort of each tile of 4096 entries by column, in LDS.
//    An entry's rank among the entries of its wave with the same digit comes from the digit's
//    ballots (the lanes whose digit bits all agree with its own), the counts of every (digit,
//    round, wave) go through one workgroup scan, and the entry moves to its scan offset plus
//    its rank.  Entries are held in (round, wave, lane) order, their order in the CSR, so each
//    pass is stable and rows stay ascending within a column.  A matrix that fits one tile gets
//    its CSC here (offsets by binary searches over the sorted columns); otherwise the tile
//    writes its sorted rows and its column bounds;
//  * csc_assemble_kernel (thread per column): off[c] = sum over the tiles of their bounds, and
//    the column's rows copied tile by tile.
// No atomics on either path.
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
// c = c_first + j * c_step, j < 8, searched in lockstep (8 independent binary searches, with
// no branches, so that each step's 8 loads are in flight together).
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
    uint32_t v[8];
    int mid[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      mid[j] = (lo[j] + hi[j]) >> 1;
      v[j] = codes[min(mid[j], len - 1)];   // in range; ignored once lo == hi
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool open = lo[j] < hi[j];
      const bool below = v[j] < key[j];
      lo[j] = open && below ? mid[j] + 1 : lo[j];
      hi[j] = open && !below ? mid[j] : hi[j];
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

// ====================================================================== radix path
constexpr int kRThreads = 512;
constexpr int kRTile = 4096;
constexpr int kRRounds = kRTile / kRThreads;          // entries per thread
constexpr int kRWaves = kRThreads / 64;
constexpr int kDigitBits = 5;
constexpr int kDigits = 1 << kDigitBits;
constexpr int kHist = kDigits * kRRounds * kRWaves;   // counts [digit][round][wave]
constexpr int kMaxRadixTiles = 64;                    // tiles per matrix the assembly reads
constexpr int kMaxCscMats = 8;                        // matrix sets per launch

struct CscSet {          // one set of nmat matrices rows x k -> cols
  const int32_t* csr;    // [nmat, nnz]
  int32_t* off;          // [nmat, cols + 1]
  int32_t* rows_out;     // [nmat, nnz]
  int32_t* trows;        // tiles > 1: [nmat, tiles, kRTile] sorted rows of each tile
  int32_t* bounds;       // tiles > 1: [nmat, tiles, cols + 1] column bounds of each tile
  int nmat, nnz, cols, k;
  int tiles;             // per matrix
  int passes;            // ceil(bits(cols + 1) / kDigitBits)
  int first_block;       // first workgroup of the set in the sort launch
  int first_cblock;      // first workgroup of the set in the assembly launch
  int cblocks;           // its assembly workgroups (0 when tiles == 1)
};
struct CscArgs {
  CscSet set[kMaxCscMats];
  int nsets;
};

__host__ __device__ constexpr size_t radix_lds_bytes() {
  return (size_t)kRTile * 8 + (size_t)kHist * 4 + (size_t)kRWaves * 4;
}

__global__ __launch_bounds__(kRThreads) void csc_radix_kernel(CscArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  uint32_t* col_s = (uint32_t*)smem;                  // [kRTile] columns in sorted order
  int32_t* row_s = (int32_t*)(col_s + kRTile);        // [kRTile] their rows
  uint32_t* hist = (uint32_t*)(row_s + kRTile);       // [kHist]
  uint32_t* wsum = hist + kHist;                      // [kRWaves]
  const int bid = blockIdx.x;
  int si = 0;
  while (si + 1 < a.nsets && bid >= a.set[si + 1].first_block) ++si;
  const CscSet& S = a.set[si];
  // the set's sizes in scalar registers once (read through the dynamic set index, the
  // compiler otherwise reloads them at each use, each reload waiting for all LDS traffic)
  int cols = S.cols, kk = S.k, nnz = S.nnz, passes = S.passes, tiles = S.tiles;
  asm volatile("" : "+s"(cols), "+s"(kk), "+s"(nnz), "+s"(passes), "+s"(tiles));
  const int local = bid - S.first_block;
  const int mat = local / tiles;
  const int tile = local - mat * tiles;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int base = tile * kRTile;
  const int len = min(kRTile, nnz - base);
  const int32_t* in = S.csr + (long)mat * nnz;
  uint32_t col[kRRounds];
  int32_t row[kRRounds];
  // every load issued before any is used (a load inside the bounds test made each one a
  // round trip of its own); past the tile's end a lane reads its last entry and ignores it
  int raw[kRRounds];
#pragma unroll
  for (int e = 0; e < kRRounds; ++e) raw[e] = in[base + min(e * kRThreads + t, len - 1)];
#pragma unroll
  for (int e = 0; e < kRRounds; ++e) {
    const int i = e * kRThreads + t;
    if (i < len) {
      int c = raw[e];
      if (c < 0 || c >= cols) c = cols;   // dropped: sorts behind the kept entries
      col[e] = (uint32_t)c;
      row[e] = (base + i) / kk;
    } else {
      col[e] = (uint32_t)cols + 1;          // padding: behind everything
      row[e] = -1;
    }
  }
  const uint64_t below = (1ull << lane) - 1;   // lanes before this one
  for (int p = 0; p < passes; ++p) {
    const int shift = p * kDigitBits;
    for (int h = t; h < kHist; h += kRThreads) hist[h] = 0;
    __syncthreads();
    int dig[kRRounds], rank[kRRounds];
#pragma unroll
    for (int e = 0; e < kRRounds; ++e) {
      const int d = (int)((col[e] >> shift) & (kDigits - 1));
      uint64_t same = ~0ull;   // lanes of the wave whose digit equals d
#pragma unroll
      for (int b = 0; b < kDigitBits; ++b) {
        const uint64_t bal = __builtin_amdgcn_ballot_w64((d >> b) & 1);
        same &= ((d >> b) & 1) ? bal : ~bal;
      }
      dig[e] = d;
      rank[e] = __builtin_popcountll(same & below);
      if (rank[e] == 0) hist[(d * kRRounds + e) * kRWaves + w] = __builtin_popcountll(same);
    }
    __syncthreads();
    // exclusive scan of the counts in (digit, round, wave) order, 4 per thread
    const uint32_t v0 = hist[4 * t], v1 = hist[4 * t + 1], v2 = hist[4 * t + 2],
                   v3 = hist[4 * t + 3];
    const uint32_t own = v0 + v1 + v2 + v3;
    uint32_t incl = own;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t y = (uint32_t)__shfl_up((int)incl, d, 64);
      if (lane >= d) incl += y;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    uint32_t excl = incl - own;
    for (int x = 0; x < w; ++x) excl += wsum[x];
    hist[4 * t] = excl;
    hist[4 * t + 1] = excl + v0;
    hist[4 * t + 2] = excl + v0 + v1;
    hist[4 * t + 3] = excl + v0 + v1 + v2;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kRRounds; ++e) {
      const int pos = (int)hist[(dig[e] * kRRounds + e) * kRWaves + w] + rank[e];
      col_s[pos] = col[e];
      row_s[pos] = row[e];
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kRRounds; ++e) {
      col[e] = col_s[e * kRThreads + t];
      row[e] = row_s[e * kRThreads + t];
    }
  }
  // the sorted tile: its rows, and lb[c] = first position whose column is >= c, c = 0..cols
  int32_t* lb;
  int32_t* rows_dst;
  if (tiles == 1) {
    lb = S.off + (long)mat * (cols + 1);
    rows_dst = S.rows_out + (long)mat * nnz;
  } else {
    lb = S.bounds + ((long)mat * tiles + tile) * (cols + 1);
    rows_dst = S.trows + ((long)mat * tiles + tile) * kRTile;
  }
#pragma unroll
  for (int e = 0; e < kRRounds; ++e)
    if (e * kRThreads + t < len) rows_dst[e * kRThreads + t] = row[e];
  for (int c0 = t; c0 <= cols; c0 += 8 * kRThreads)
    column_bounds8(col_s, len, c0, kRThreads, cols, 0, lb);
}

// Per column range: each of the cblocks workgroups of a matrix owns the CR real columns
// [c0, c0 + nc) (CR = assembly_cols(tiles)); the one that ends at `cols` also writes off[cols].
//  1. lbs[t][j] = lb_t[c0 + j], j = 0..nc, for every tile t (LDS, coalesced loads);
//  2. thread j < nc: off[c0 + j] = sum_t lbs[t][j], and base[t][j] = the destination of tile
//     t's first entry of that column minus its sorted position (off + the entries of the
//     column in tiles t' < t - lbs[t][j]), so that position i lands at base[t][j] + i;
//  3. the range's entries of tile t are the contiguous sorted positions [lbs[t][0], lbs[t][nc]);
//     all threads copy them (coalesced, 4 loads in flight per thread), each finding its
//     tile and column by binary searches in LDS.
__host__ __device__ constexpr int assembly_cols(int tiles) {
  return tiles <= 16 ? 256 : tiles <= 32 ? 128 : 64;
}
__host__ __device__ constexpr size_t assembly_lds_bytes(int tiles) {
  return sizeof(int32_t) * ((size_t)tiles * (2 * assembly_cols(tiles) + 1) + tiles + 1);
}

__global__ __launch_bounds__(256) void csc_assemble_kernel(CscArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int bid = blockIdx.x;
  int si = 0;
  while (si + 1 < a.nsets &&
         (a.set[si].cblocks == 0 || bid >= a.set[si].first_cblock + a.set[si].cblocks))
    ++si;
  const CscSet& S = a.set[si];
  const int tiles = S.tiles;
  const int CR = assembly_cols(tiles);
  const int per_mat = (S.cols + CR - 1) / CR;
  const int local = bid - S.first_cblock;
  const int mat = local / per_mat;
  const int c0 = (local - mat * per_mat) * CR;
  const int nc = min(CR, S.cols - c0);
  const int tid = threadIdx.x;
  const int stride = S.cols + 1;
  int32_t* lbs = (int32_t*)smem;                 // [tiles][nc + 1]
  int32_t* base = lbs + tiles * (CR + 1);        // [tiles][nc]
  int32_t* segpre = base + tiles * CR;           // [tiles + 1] prefix of segment lengths
  const int32_t* bnd = S.bounds + (long)mat * tiles * stride + c0;
  // 1. the tiles' bounds of the range
  const int nl = tiles * (nc + 1);
  for (int x0 = 0; x0 < nl; x0 += 4 * 256) {
    int32_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int x = x0 + u * 256 + tid;
      v[u] = x < nl ? bnd[(long)(x / (nc + 1)) * stride + x % (nc + 1)] : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int x = x0 + u * 256 + tid;
      if (x < nl) lbs[(x / (nc + 1)) * (CR + 1) + x % (nc + 1)] = v[u];
    }
  }
  __syncthreads();
  // 2. offsets and destination bases
  int32_t* off = S.off + (long)mat * stride + c0;
  if (tid < nc) {
    int total = 0;
    for (int t = 0; t < tiles; ++t) total += lbs[t * (CR + 1) + tid];
    off[tid] = total;
    for (int t = 0; t < tiles; ++t) {
      const int lo = lbs[t * (CR + 1) + tid];
      base[t * CR + tid] = total - lo;
      total += lbs[t * (CR + 1) + tid + 1] - lo;
    }
  }
  if (tid == 0) {
    if (c0 + nc == S.cols) {   // the range that ends at cols: off[cols] = the kept entries
      int total = 0;
      for (int t = 0; t < tiles; ++t) total += lbs[t * (CR + 1) + nc];
      off[nc] = total;
    }
    int acc = 0;
    for (int t = 0; t < tiles; ++t) {
      segpre[t] = acc;
      acc += lbs[t * (CR + 1) + nc] - lbs[t * (CR + 1)];
    }
    segpre[tiles] = acc;
  }
  __syncthreads();
  // 3. copy the entries of the range
  const int total = segpre[tiles];
  int32_t* rows_out = S.rows_out + (long)mat * S.nnz;
  const int32_t* trows = S.trows + (long)mat * tiles * kRTile;
  for (int f0 = 0; f0 < total; f0 += 4 * 256) {
    int32_t val[4];
    int dst[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int f = f0 + u * 256 + tid;
      dst[u] = -1;
      val[u] = 0;
      if (f < total) {
        int tlo = 0, thi = tiles - 1;   // last tile t with segpre[t] <= f
        while (tlo < thi) {
          const int m = (tlo + thi + 1) >> 1;
          if (segpre[m] <= f) tlo = m;
          else thi = m - 1;
        }
        const int32_t* lb_t = lbs + tlo * (CR + 1);
        const int i = lb_t[0] + (f - segpre[tlo]);
        int jlo = 0, jhi = nc - 1;      // last column j with lb_t[j] <= i
        while (jlo < jhi) {
          const int m = (jlo + jhi + 1) >> 1;
          if (lb_t[m] <= i) jlo = m;
          else jhi = m - 1;
        }
        dst[u] = base[tlo * CR + jlo] + i;
        val[u] = trows[(long)tlo * kRTile + i];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (dst[u] >= 0) rows_out[dst[u]] = val[u];
  }
}

static bool radix_eligible(int rows, int k) {
  return ((long)rows * k + kRTile - 1) / kRTile <= kMaxRadixTiles;
}
bool transpose_uses_radix(int rows, int k) { return radix_eligible(rows, k); }

static size_t align256_(size_t b) { return (b + 255) & ~(size_t)255; }

// Workspace of the radix path for one matrix set (0 when one tile holds a matrix).
static size_t radix_workspace_bytes(int nmat, int rows, int cols, int k) {
  const int tiles = (int)(((long)rows * k + kRTile - 1) / kRTile);
  if (tiles <= 1) return 0;
  return align256_(sizeof(int32_t) * (size_t)nmat * tiles * kRTile) +
         align256_(sizeof(int32_t) * (size_t)nmat * tiles * ((size_t)cols + 1));
}

static int bits_for(long v) {   // bits needed to write v
  int b = 1;
  while ((1L << b) <= v) ++b;
  return b;
}

// The radix path for up to kMaxCscMats matrix sets at once (two launches in all).
static hipError_t launch_csc_radix(int nsets, const int* nmat, const int* rows, const int* cols,
                                   const int* k, const int32_t* const* csr, int32_t* const* off,
                                   int32_t* const* rows_out, void* ws, hipStream_t stream) {
  CscArgs a{};
  a.nsets = nsets;
  char* w = (char*)ws;
  int blocks = 0, cblocks = 0;
  size_t alds = 0;
  for (int i = 0; i < nsets; ++i) {
    CscSet& S = a.set[i];
    S.csr = csr[i];
    S.off = off[i];
    S.rows_out = rows_out[i];
    S.nmat = nmat[i];
    S.nnz = rows[i] * k[i];
    S.cols = cols[i];
    S.k = k[i];
    S.tiles = (S.nnz + kRTile - 1) / kRTile;
    S.passes = (bits_for((long)cols[i] + 1) + kDigitBits - 1) / kDigitBits;
    S.first_block = blocks;
    blocks += nmat[i] * S.tiles;
    if (S.tiles > 1) {
      S.trows = (int32_t*)w;
      w += align256_(sizeof(int32_t) * (size_t)nmat[i] * S.tiles * kRTile);
      S.bounds = (int32_t*)w;
      w += align256_(sizeof(int32_t) * (size_t)nmat[i] * S.tiles * ((size_t)cols[i] + 1));
      S.first_cblock = cblocks;
      S.cblocks = nmat[i] * ((cols[i] + assembly_cols(S.tiles) - 1) / assembly_cols(S.tiles));
      cblocks += S.cblocks;
      alds = std::max(alds, assembly_lds_bytes(S.tiles));
    }
  }
  LLSA_LAUNCH("csc_radix_kernel", csc_radix_kernel, dim3((unsigned)blocks), dim3(kRThreads),
              radix_lds_bytes(), stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || cblocks == 0) return err;
  LLSA_LAUNCH("csc_assemble_kernel", csc_assemble_kernel, dim3((unsigned)cblocks), dim3(256),
              alds, stream, a);
  return hipGetLastError();
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

static size_t bitonic_workspace_bytes(int nmat, int rows, int cols, int k) {
  const TransposePlan p = plan_transpose(rows, k);
  const size_t nnz = (size_t)rows * k;
  return 2 * align256(sizeof(uint32_t) * nmat * nnz) +
         align256(sizeof(int32_t) * nmat * p.nruns * ((size_t)cols + 1)) +
         align256(sizeof(int32_t) * nmat * p.nruns * (size_t)cols);
}

size_t transpose_workspace_bytes(int nmat, int rows, int cols, int k) {
  return radix_eligible(rows, k) ? radix_workspace_bytes(nmat, rows, cols, k)
                                 : bitonic_workspace_bytes(nmat, rows, cols, k);
}

static hipError_t launch_bitonic(int nmat, int rows, int cols, int k, const int32_t* csr,
                                 int32_t* off, int32_t* rows_out, void* ws, hipStream_t stream) {
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

hipError_t launch_index_transpose(int nmat, int rows, int cols, int k, const int32_t* csr,
                                  int32_t* off, int32_t* rows_out, void* ws,
                                  hipStream_t stream) {
  if (radix_eligible(rows, k))
    return launch_csc_radix(1, &nmat, &rows, &cols, &k, &csr, &off, &rows_out, ws, stream);
  return launch_bitonic(nmat, rows, cols, k, csr, off, rows_out, ws, stream);
}

// Several matrix sets in order on one stream: the ones the radix path takes in its two
// launches, the others one after the other on the bitonic path; every part runs after the
// previous one, so they share one workspace.
size_t transpose_sets_workspace_bytes(int nsets, const int* nmat, const int* rows,
                                      const int* cols, const int* k) {
  size_t radix = 0, other = 0;
  for (int i = 0; i < nsets; ++i) {
    if (radix_eligible(rows[i], k[i]))
      radix += radix_workspace_bytes(nmat[i], rows[i], cols[i], k[i]);
    else
      other = std::max(other, bitonic_workspace_bytes(nmat[i], rows[i], cols[i], k[i]));
  }
  return std::max(radix, other);
}

hipError_t launch_transpose_sets(int nsets, const int* nmat, const int* rows, const int* cols,
                                 const int* k, const int32_t* const* csr, int32_t* const* off,
                                 int32_t* const* rows_out, void* ws, hipStream_t stream) {
  int rn = 0, rnmat[kMaxCscMats], rrows[kMaxCscMats], rcols[kMaxCscMats], rk[kMaxCscMats];
  const int32_t* rcsr[kMaxCscMats];
  int32_t* roff[kMaxCscMats];
  int32_t* rout[kMaxCscMats];
  for (int i = 0; i < nsets; ++i) {
    if (!radix_eligible(rows[i], k[i])) {
      const hipError_t e =
          launch_bitonic(nmat[i], rows[i], cols[i], k[i], csr[i], off[i], rows_out[i], ws, stream);
      if (e != hipSuccess) return e;
      continue;
    }
    rnmat[rn] = nmat[i];
    rrows[rn] = rows[i];
    rcols[rn] = cols[i];
    rk[rn] = k[i];
    rcsr[rn] = csr[i];
    roff[rn] = off[i];
    rout[rn] = rows_out[i];
    ++rn;
  }
  if (rn == 0) return hipSuccess;
  return launch_csc_radix(rn, rnmat, rrows, rcols, rk, rcsr, roff, rout, ws, stream);
}

}  // namespace llsa
