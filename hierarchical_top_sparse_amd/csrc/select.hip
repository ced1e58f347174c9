// Coarse-to-fine top-K selection (paper summary sec. 三; article sec. 三).
//
// One launch computes a range of levels.  Wave w owns a group of 16 sibling queries at
// the finest requested level lo (the 16 children of query w at level lo + 1, or 16 coarsest
// queries when lo = L), and first walks the chain of that group's ancestors from level hi
// down to lo + 1:
//   * the ancestor at level lv is a single query, ranked against all n_L keys (lv = L) or
//     against the K*B children of its parent's picks (lv < L);
//   * the 16 waves (16^2, ...) under one ancestor rank it redundantly with identical
//     arithmetic, and only the first of them stores its row, so there is no cross-wave
//     dependency and the whole selection is one kernel.
// The group itself is then ranked against the children of its parent's picks.
// A request that spans three or more levels down to level 1 is issued as two launches, levels
// hi .. 2 and then level 1 from the stored level-2 picks: the level-1 waves, by far the most,
// then skip the redundant chain (at 512x512 L=3 this is 27% faster; identical picks).
//
// Scores are fp32 dot products on the fp32 MFMA (v_mfma_f32_16x16x4f32) in the S^T
// orientation: lane (n, g) holds the scores of query n against candidates 4g..4g+3 of each
// 16-row candidate tile.  Tiles are loaded kTilesPerRound at a time, so a ranking costs one or
// two memory round trips rather than one per tile.
//  * A group (16 queries): each lane keeps a register top-KMAX list of its candidates, and the
//    four lanes of a query merge their lists with cross-lane steps.
//  * A single query is replicated over the 16 columns; each (tile, candidate) is then kept by
//    exactly one lane (lane (n, g) takes candidate 4g + n % 4 of the tiles t with
//    t % 4 = n / 4), and the 64 lists are merged across the whole wave.
// llsa_pool_select issues the same launches with extra workgroups after the selection's that
// pool V (select_pool12_kernel, select_pool_next_kernel): V is first read by the attention.
// Lists only take strictly better scores: every lane sees its candidates in ascending id order
// (picks are stored ascending), so ties keep the lower id; merges compare (score, id).  The K
// picks are stored ascending.  The picks a ranking starts from are held one per lane (lane i:
// pick i) and read with v_readlane.
#include "common.hpp"
#include "kernels.hpp"
#include "pool_impl.hpp"

namespace llsa {

constexpr int kSelWaves = 4;
constexpr int kSelMaxLv = 6;
constexpr int kNoId = 0x7fffffff;
constexpr int kTilesPerRound = 4;   // candidate tiles loaded at once

struct SelArgs {
  const float* q[kSelMaxLv];   // level l at index l - 1: [bh, n_l, 64] fp32
  const float* k[kSelMaxLv];
  int32_t* sel[kSelMaxLv];     // [bh, n_l, K]
  int bh;
  int n;        // tokens per head (level 0)
  int levels;   // L
  int topk;     // K
  int hi, lo;   // levels computed: hi down to lo
  int bshift;   // log2(B): 4 or 6; a pick's B children are B / 16 tiles of 16 candidates
};

__device__ __forceinline__ bool better(float s1, int i1, float s2, int i2) {
  return s1 > s2 || (s1 == s2 && i1 < i2);
}

// Inserts a candidate whose id is larger than every id already in the list (scores
// descending).  Lists of up to 8: c_j = s > ls[j] is monotone in j, so slot j keeps its entry
// (c_j false), takes the candidate (c_j and not c_{j-1}) or its predecessor's entry (c_{j-1}):
// all compares are independent, a chain of depth 3.  Longer lists: one compare-and-swap step
// per slot (their 16 or 32 compare masks would not stay in scalar registers).
template <int KMAX>
__device__ __forceinline__ void list_insert(float (&ls)[KMAX], int (&li)[KMAX], float s, int id) {
  if constexpr (KMAX > 8) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const bool b = s > ls[j];
      const float ts = ls[j];
      const int ti = li[j];
      ls[j] = b ? s : ts;
      li[j] = b ? id : ti;
      s = b ? ts : s;
      id = b ? ti : id;
    }
    return;
  }
  bool c[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) c[j] = s > ls[j];
#pragma unroll
  for (int j = KMAX - 1; j >= 1; --j) {
    ls[j] = c[j] ? (c[j - 1] ? ls[j - 1] : s) : ls[j];
    li[j] = c[j] ? (c[j - 1] ? li[j - 1] : id) : li[j];
  }
  ls[0] = c[0] ? s : ls[0];
  li[0] = c[0] ? id : li[0];
}

// Candidate rows first + n (channels 16g .. 16g + 15) of a 16-row tile; rows outside
// [0, n_rows) and tiles with first < 0 read as zeros (their scores are never inserted).
__device__ __forceinline__ void load_tile(const float* kh, int first, int n_rows, int n, int g,
                                          f32x4 (&kv)[4]) {
  const int row = first + n;
  const bool ok = first >= 0 && row < n_rows;
  const float* p = kh + (long)(ok ? row : 0) * kDim + 16 * g;
#pragma unroll
  for (int c = 0; c < 4; ++c) kv[c] = ok ? *(const f32x4*)(p + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
}

// acc[i] = score of query n against candidate 4g + i of the tile: the 64 channels are
// contracted in four independent MFMA chains (channels 16g + 4c + e, e = 0..3, per chain c).
__device__ __forceinline__ f32x4 score_tile(const f32x4 (&kv)[4], const f32x4 (&qv)[4]) {
  f32x4 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[c] = mfma_f32_k4(kv[c][e], qv[c][e], acc[c]);
  }
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// Extracts the K best (score, id) of the lists of the lanes in one xor-group (the lanes
// differing only in the bits of lane_bits), best first, into pick[0..K) of all those lanes
// (kNoId beyond K), then sorts pick ascending.
template <int KMAX, int LANE_BITS_LO, int LANE_BITS_HI>
__device__ __forceinline__ void merge_lists(float (&ls)[KMAX], int (&li)[KMAX], int K,
                                            int (&pick)[KMAX]) {
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    pick[r] = kNoId;
    if (r < K) {
      float bs = ls[0];
      int bi = li[0];
#pragma unroll
      for (int mask = LANE_BITS_LO; mask <= LANE_BITS_HI; mask <<= 1) {
        const float os = shfl_xor_f(bs, mask);
        const int oi = shfl_xor_i(bi, mask);
        if (better(os, oi, bs, bi)) {
          bs = os;
          bi = oi;
        }
      }
      pick[r] = bi;
      if (li[0] == bi) {   // pop the winner from its owner's list
#pragma unroll
        for (int j = 0; j + 1 < KMAX; ++j) {
          ls[j] = ls[j + 1];
          li[j] = li[j + 1];
        }
        ls[KMAX - 1] = -INFINITY;
        li[KMAX - 1] = kNoId;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < KMAX; ++i)
#pragma unroll
    for (int j = 0; j + 1 < KMAX - i; ++j) {
      const int lo = min(pick[j], pick[j + 1]);
      const int hi = max(pick[j], pick[j + 1]);
      pick[j] = lo;
      pick[j + 1] = hi;
    }
}

// Ranks the queries held in qv (columns n) against one candidate set and returns the K picks,
// ascending, as pick[0..K) (kNoId beyond K): per query n in the lanes of column n (SINGLE:
// the one query, in every lane).
//   all_keys: candidates are all n_rows keys of the level;
//   else:     candidates are the B = 2^bshift children of each pick in pickv (lane i holds
//             pick i of the parent, i < K; ids outside [0, n_rows / B) are skipped), B / 16
//             tiles per pick.
template <int KMAX, bool SINGLE>
__device__ __forceinline__ void rank_queries(const float* kh, int n_rows, bool all_keys,
                                             int pickv, int K, int bshift,
                                             const f32x4 (&qv)[4], int n, int g,
                                             int (&pick)[KMAX]) {
  float ls[KMAX];
  int li[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    ls[j] = -INFINITY;
    li[j] = kNoId;
  }
  const int n_parent = n_rows >> bshift;
  const int sub_shift = bshift - 4;   // log2 of the tiles per pick
  const int tiles = all_keys ? (n_rows + 15) >> 4 : K << sub_shift;
  for (int t0 = 0; t0 < tiles; t0 += kTilesPerRound) {
    f32x4 kv[kTilesPerRound][4];
    int first[kTilesPerRound];
#pragma unroll
    for (int i = 0; i < kTilesPerRound; ++i) {
      const int t = t0 + i;
      first[i] = -1;
      if (t < tiles) {
        if (all_keys) {
          first[i] = 16 * t;
        } else {
          const int pk = __builtin_amdgcn_readlane(pickv, t >> sub_shift);
          const int sub = t & ((1 << sub_shift) - 1);
          first[i] = (pk >= 0 && pk < n_parent) ? (pk << bshift) + 16 * sub : -1;
        }
      }
      load_tile(kh, first[i], n_rows, n, g, kv[i]);
    }
#pragma unroll
    for (int i = 0; i < kTilesPerRound; ++i) {
      if (first[i] < 0) continue;
      const f32x4 acc = score_tile(kv[i], qv);
      if constexpr (SINGLE) {
        // tile t0 + i is kept by the lanes with n / 4 == i (t0 is a multiple of 4)
        if ((n >> 2) == i) {
          const int e = n & 3;
          const float sc = e == 0 ? acc[0] : e == 1 ? acc[1] : e == 2 ? acc[2] : acc[3];
          const int cid = first[i] + 4 * g + e;
          if (cid < n_rows) list_insert<KMAX>(ls, li, sc, cid);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int cid = first[i] + 4 * g + e;
          if (cid < n_rows) list_insert<KMAX>(ls, li, acc[e], cid);
        }
      }
    }
  }
  if constexpr (SINGLE) merge_lists<KMAX, 1, 32>(ls, li, K, pick);
  else merge_lists<KMAX, 16, 32>(ls, li, K, pick);
}

// The waves of selection workgroup bid of nblocks (renumbered per XCD).
template <int KMAX>
__device__ __forceinline__ void select_group(const SelArgs& a, int bid, int nblocks) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int K = a.topk;
  const int lo = a.lo;
  const int bs = a.bshift;
  const int n_lo = a.n >> (bs * lo);
  const int groups = (n_lo + 15) >> 4;
  const int wave = uniform(xcd_block(bid, nblocks) * kSelWaves + (int)(threadIdx.x >> 6));
  if (wave >= a.bh * groups) return;
  const int head = uniform(wave / groups);
  const int grp = uniform(wave - head * groups);

  // picks of the parent of the level being ranked, one per lane
  int pickv = kNoId;
  if (lo < a.levels) {
    // the group's parent is query (16 grp) >> bs at level lo + 1
    if (a.hi == lo) {   // parent picks given: sel at level lo + 1
      if (lane < K)
        pickv = a.sel[lo][((long)head * (n_lo >> bs) + ((grp << 4) >> bs)) * K + lane];
    } else {
      // chain: ancestors at levels hi .. lo + 1, each a single query
      for (int lv = a.hi; lv > lo; --lv) {
        const int shift = bs * (lv - lo);
        const int anc = (grp << 4) >> shift;          // query id at level lv
        const int n_lv = a.n >> (bs * lv);
        const bool top = lv == a.levels;
        if (lv == a.hi && !top) {
          // parent picks of the topmost computed ancestor are given at level hi + 1
          if (lane < K)
            pickv = a.sel[lv][((long)head * (n_lv >> bs) + (anc >> bs)) * K + lane];
        }
        const float* qrow = a.q[lv - 1] + ((long)head * n_lv + anc) * kDim + 16 * g;
        f32x4 qv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) qv[c] = *(const f32x4*)(qrow + 4 * c);
        int pick[KMAX];
        rank_queries<KMAX, true>(a.k[lv - 1] + (long)head * n_lv * kDim, n_lv, top, pickv, K,
                                 bs, qv, n, g, pick);
        int nv = kNoId;
#pragma unroll
        for (int r = 0; r < KMAX; ++r)
          if (lane == r) nv = pick[r];
        pickv = nv;
        if (((grp << 4) & ((1 << shift) - 1)) == 0 && lane < K)
          a.sel[lv - 1][((long)head * n_lv + anc) * K + lane] = pickv;
      }
    }
  }

  // the group of 16 queries at level lo
  const float* qh = a.q[lo - 1] + (long)head * n_lo * kDim;
  const int q_id = grp * 16 + n;
  const bool qvalid = q_id < n_lo;
  f32x4 qv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    qv[c] = qvalid ? *(const f32x4*)(qh + (long)q_id * kDim + 16 * g + 4 * c)
                   : f32x4{0.f, 0.f, 0.f, 0.f};
  int pick[KMAX];
  rank_queries<KMAX, false>(a.k[lo - 1] + (long)head * n_lo * kDim, n_lo, lo == a.levels, pickv,
                            K, bs, qv, n, g, pick);
  if (g == 0 && qvalid) {
    int32_t* dst = a.sel[lo - 1] + ((long)head * n_lo + q_id) * K;
#pragma unroll
    for (int r = 0; r < KMAX; ++r)
      if (r < K) dst[r] = pick[r];
  }
}

template <int KMAX>
__global__ __launch_bounds__(64 * kSelWaves) void select_kernel(SelArgs a) {
  select_group<KMAX>(a, blockIdx.x, gridDim.x);
}

// A selection launch that also pools V (its levels 1 and 2 from the tokens, or level 3 from
// level 2): the selection's workgroups come first (sel_blocks, a multiple of 8, so that their
// XCDs are those of a plain launch) and raise their waves' issue priority; the pooling
// workgroups after them fill the chip while the few selection waves run their dependent
// chains.  V is first read by the attention, so nothing in the launch depends on it.
template <int KMAX>
__global__ __launch_bounds__(64 * kSelWaves) void select_pool12_kernel(SelArgs a, int sel_blocks,
                                                                       PoolArgs pa, int n,
                                                                       Grid grid, int gph) {
  __shared__ __attribute__((aligned(16))) float sh[kBlock][kDim];
  if ((int)blockIdx.x < sel_blocks) {
    __builtin_amdgcn_s_setprio(2);
    select_group<KMAX>(a, blockIdx.x, sel_blocks);
    return;
  }
  pool12_bf16_group(pa, n, grid, gph, 0, (int)blockIdx.x - sel_blocks, sh);
}

template <int KMAX>
__global__ __launch_bounds__(64 * kSelWaves) void select_pool_next_kernel(SelArgs a,
                                                                          int sel_blocks,
                                                                          PoolNextArgs pb,
                                                                          long total_out) {
  if ((int)blockIdx.x < sel_blocks) {
    __builtin_amdgcn_s_setprio(2);
    select_group<KMAX>(a, blockIdx.x, sel_blocks);
    return;
  }
  const long i = (long)((int)blockIdx.x - sel_blocks) * 256 + threadIdx.x;
  if (i < total_out) pool_next_elem<16>(pb, 0, i);
}

__global__ __launch_bounds__(256) void pool_next_v_kernel(PoolNextArgs pb, long total_out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < total_out) pool_next_elem<16>(pb, 0, i);
}

// Level-1 picks of 64-token blocks as the 16-token blocks they cover: row q of the output (a
// 16-token query block) lists, for each pick j of its 64-token block q / 4, the blocks
// 4j .. 4j + 3 (ascending, as the picks are).  With B = 16 a copy.  One thread per output.
__global__ __launch_bounds__(256) void expand_kernel(const int32_t* __restrict__ sel,
                                                     int32_t* __restrict__ fine, int sub_shift,
                                                     int k, long total) {
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  if (t >= total) return;
  const int kf = k << sub_shift;
  const long q16 = t / kf;            // (bh, 16-token query block)
  const int e = (int)(t - q16 * kf);
  const int j = sel[(q16 >> sub_shift) * k + (e >> sub_shift)];
  fine[t] = j < 0 ? -1 : (j << sub_shift) + (e & ((1 << sub_shift) - 1));
}

hipError_t launch_expand_blocks(const Shape& s, const int32_t* sel1, int32_t* fine,
                                hipStream_t stream) {
  const long total = (long)s.bh * (s.n >> kBlockShift) * s.fine_k;
  LLSA_LAUNCH("expand_kernel", expand_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256),
              0, stream, sel1, fine, s.bshift - kBlockShift, s.topk, total);
  return hipGetLastError();
}

// V's pooling carried by a selection launch: kind 1 = levels 1 and 2 from the tokens
// (pool12 of tensor 0 of pa), kind 2 = one level from the level below (B = 16).
struct PoolInSelect {
  int kind = 0;
  PoolArgs pa{};
  PoolNextArgs pb{};
  long total = 0;   // kind 2: output elements
};

static hipError_t launch_select_range(const Shape& s, const float* const* q_lv,
                                      const float* const* k_lv, int32_t* const* sel,
                                      int level_hi, int level_lo, hipStream_t stream,
                                      const PoolInSelect& pv = PoolInSelect{}) {
  SelArgs a{};
  for (int l = 0; l < s.levels && l < kSelMaxLv; ++l) {
    a.q[l] = q_lv[l];
    a.k[l] = k_lv[l];
    a.sel[l] = sel[l];
  }
  a.bh = s.bh;
  a.n = s.n;
  a.levels = s.levels;
  a.topk = s.topk;
  a.hi = level_hi;
  a.lo = level_lo;
  a.bshift = s.bshift;
  const int n_lo = s.n_level(level_lo);
  const long waves = (long)s.bh * ((n_lo + 15) >> 4);   // one per group
  const unsigned blocks = (unsigned)((waves + kSelWaves - 1) / kSelWaves);
  if (pv.kind != 0) {
    const unsigned sb = (blocks + 7) / 8 * 8;
    const dim3 wg(64 * kSelWaves);
    if (pv.kind == 1) {
      const int gph = s.n >> (2 * kBlockShift);
      const dim3 g(sb + (unsigned)(s.bh * gph));
      const Grid tg{s.hbits, s.wbits, s.raster};
      if (s.topk <= 8)
        LLSA_LAUNCH("select_pool_kernel", select_pool12_kernel<8>, g, wg, 0, stream, a, (int)sb,
                    pv.pa, s.n, tg, gph);
      else if (s.topk <= 16)
        LLSA_LAUNCH("select_pool_kernel", select_pool12_kernel<16>, g, wg, 0, stream, a,
                    (int)sb, pv.pa, s.n, tg, gph);
      else
        LLSA_LAUNCH("select_pool_kernel", select_pool12_kernel<32>, g, wg, 0, stream, a,
                    (int)sb, pv.pa, s.n, tg, gph);
    } else {
      const dim3 g(sb + (unsigned)((pv.total + 255) / 256));
      if (s.topk <= 8)
        LLSA_LAUNCH("select_pool_kernel", select_pool_next_kernel<8>, g, wg, 0, stream, a,
                    (int)sb, pv.pb, pv.total);
      else if (s.topk <= 16)
        LLSA_LAUNCH("select_pool_kernel", select_pool_next_kernel<16>, g, wg, 0, stream, a,
                    (int)sb, pv.pb, pv.total);
      else
        LLSA_LAUNCH("select_pool_kernel", select_pool_next_kernel<32>, g, wg, 0, stream, a,
                    (int)sb, pv.pb, pv.total);
    }
    return hipGetLastError();
  }
  if (s.topk <= 8)
    LLSA_LAUNCH("select_kernel", select_kernel<8>, dim3(blocks), dim3(64 * kSelWaves), 0, stream,
                a);
  else if (s.topk <= 16)
    LLSA_LAUNCH("select_kernel", select_kernel<16>, dim3(blocks), dim3(64 * kSelWaves), 0,
                stream, a);
  else
    LLSA_LAUNCH("select_kernel", select_kernel<32>, dim3(blocks), dim3(64 * kSelWaves), 0,
                stream, a);
  return hipGetLastError();
}

hipError_t launch_select(const Shape& s, const float* const* q_lv, const float* const* k_lv,
                         int32_t* const* sel, int level_hi, int level_lo, hipStream_t stream) {
  if (level_lo == 1 && level_hi >= 3) {
    const hipError_t e = launch_select_range(s, q_lv, k_lv, sel, level_hi, 2, stream);
    if (e != hipSuccess) return e;
    return launch_select_range(s, q_lv, k_lv, sel, 1, 1, stream);
  }
  return launch_select_range(s, q_lv, k_lv, sel, level_hi, level_lo, stream);
}

// Pooling of Q, K and V and the selection of every level, as llsa_pool then llsa_select
// (levels L..1).  With B = 16, bf16 tokens, V given and L >= 2, V's pooling rides in the
// selection launches (levels 1-2 in the first, level 3 in the level-1 launch when L >= 3,
// levels 4.. after it); otherwise the two calls run as they are.  Same results either way:
// every kernel body and its arithmetic are the ones of the plain launches.
hipError_t launch_pool_select(const Shape& s, const void* const x[3], float* const* lv[3],
                              int32_t* const* sel, hipStream_t stream) {
  const int L = s.levels;
  const bool fuse = x[2] && s.bf16 && s.bshift == kBlockShift && L >= 2 && lv[2][1];
  if (!fuse) {
    const hipError_t e = launch_pool(s, x, lv, stream);
    if (e != hipSuccess) return e;
    return launch_select(s, lv[0], lv[1], sel, L, 1, stream);
  }
  const void* qk[3] = {x[0], x[1], nullptr};
  hipError_t e = launch_pool(s, qk, lv, stream);
  if (e != hipSuccess) return e;
  PoolInSelect p12;
  p12.kind = 1;
  p12.pa.x[0] = x[2];
  p12.pa.lv1[0] = lv[2][0];
  p12.pa.lv2[0] = lv[2][1];
  if (L == 2) return launch_select_range(s, lv[0], lv[1], sel, 2, 1, stream, p12);
  e = launch_select_range(s, lv[0], lv[1], sel, L, 2, stream, p12);
  if (e != hipSuccess) return e;
  PoolInSelect pn;
  if (lv[2][2]) {
    pn.kind = 2;
    pn.pb.in[0] = lv[2][1];
    pn.pb.out[0] = lv[2][2];
    pn.total = (long)s.bh * s.n_level(3) * kDim;
  }
  e = launch_select_range(s, lv[0], lv[1], sel, 1, 1, stream, pn);
  if (e != hipSuccess) return e;
  for (int l = 4; l <= L; ++l) {   // V's levels above 3: the plain kernel, level by level
    if (!lv[2][l - 1]) continue;
    if (!lv[2][l - 2]) return hipErrorInvalidValue;
    PoolNextArgs b{};
    b.in[0] = lv[2][l - 2];
    b.out[0] = lv[2][l - 1];
    const long total = (long)s.bh * s.n_level(l) * kDim;
    LLSA_LAUNCH("pool_next_kernel", pool_next_v_kernel, dim3((unsigned)((total + 255) / 256)),
                dim3(256), 0, stream, b, total);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace llsa
