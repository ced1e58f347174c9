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
// 16-row candidate tile, and channels g D/4 .. g D/4 + D/4 - 1 of the rows (D = head_dim, 64
// or 128).  Tiles are loaded tiles_per_round(D) at a time, so a ranking costs one or two
// memory round trips rather than one per tile.
//  * A group (16 queries): each lane keeps a register top-KMAX list of its candidates (a tile's
//    four are sorted by a 5-comparator network and merged in by a bitonic top-KMAX merge), and
//    the four lanes of a query exchange and merge their whole lists twice (v_permlane16_swap,
//    v_permlane32_swap).
//  * A single query is replicated over the 16 columns; each (tile, candidate) is then kept by
//    exactly one lane (lane (n, g) takes candidate 4g + n % 4 of the tiles t with
//    t % 4 = n / 4), and the 64 lists are merged across the whole wave (DPP, then the swaps).
// llsa_pool_select issues the same launches with extra workgroups after the selection's that
// pool V (select_pool12_kernel, select_pool_next_kernel): V is first read by the attention.
// The ranking is a strict total order: a higher score first and, between equal scores, the
// lower id.  Candidates are held as 64-bit keys in that order (score bits made unsigned-order
// above the complemented id), so every compare is one unsigned compare and the picks do not
// depend on how the candidates are split among lanes or merged.  The K picks are stored
// ascending.  The picks a ranking starts from are held one per lane (lane i: pick i) and read
// with v_readlane.
#include "common.hpp"
#include "kernels.hpp"
#include "pool_impl.hpp"

namespace llsa {

constexpr int kSelWaves = 4;
constexpr int kSelMaxLv = 6;
constexpr int kNoId = 0x7fffffff;
// candidate tiles loaded at once (their rows stay in registers: fewer for wider rows)
__host__ __device__ constexpr int tiles_per_round(int D) { return D == 64 ? 4 : 2; }

struct SelArgs {
  const float* q[kSelMaxLv];   // level l at index l - 1: [bh, n_l, head_dim] fp32
  const float* k[kSelMaxLv];
  int32_t* sel[kSelMaxLv];     // [bh, n_l, K]
  int bh;
  int n;        // tokens per head (level 0)
  int levels;   // L
  int topk;     // K
  int hi, lo;   // levels computed: hi down to lo
  int bshift;   // log2(B): 4 or 6; a pick's B children are B / 16 tiles of 16 candidates
  int parts;    // waves per group at level lo (1 or 2): part p ranks rounds p, p + parts, ..
};

// Candidate rows first + n (channels g D/4 .. g D/4 + D/4 - 1) of a 16-row tile; rows outside
// [0, n_rows) and tiles with first < 0 read as zeros (their scores are never inserted).
template <int D>
__device__ __forceinline__ void load_tile(const float* kh, int first, int n_rows, int n, int g,
                                          f32x4 (&kv)[D / 16]) {
  const int row = first + n;
  const bool ok = first >= 0 && row < n_rows;
  const float* p = kh + (long)(ok ? row : 0) * D + (D / 4) * g;
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    kv[c] = ok ? *(const f32x4*)(p + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
}

// acc[i] = score of query n against candidate 4g + i of the tile: the D channels are
// contracted in four independent MFMA chains (chain c takes the lane's vectors j = c, c + 4,
// ..., channels g D/4 + 4j + e, e = 0..3).
template <int D>
__device__ __forceinline__ f32x4 score_tile(const f32x4 (&kv)[D / 16], const f32x4 (&qv)[D / 16]) {
  f32x4 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = c; j < D / 16; j += 4)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[c] = mfma_f32_k4(kv[j][e], qv[j][e], acc[c]);
  }
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// A candidate as one unsigned 64-bit key whose order is the ranking: the score's bits in an
// order-preserving unsigned form (-0 taken as +0) above the complemented id, so that a larger
// key is a larger score or, for equal scores, a lower id.  Every ordering below is on keys,
// which makes the picks independent of how candidates are grouped and merged.
using key64 = unsigned long long;
// Empty list slot: upper half 1, below every candidate's key (a candidate's upper half is at
// least 0x007fffff for any non-NaN score), decodes to kNoId.  A candidate a lane does not
// take gets upper half 0, below every slot, and is never kept.
constexpr key64 kPadKey = (1ull << 32) | 0x80000000ull;

// s + 0 turns -0 into +0 (round to nearest), so both zeros map to the same key
__device__ __forceinline__ unsigned key_hi(float s) {
  const unsigned u = f_bits(s + 0.f);
  return u ^ ((unsigned)((int)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ key64 make_key(float s, int id, bool take) {
  return ((key64)(take ? key_hi(s) : 0u) << 32) | (unsigned)~id;
}
__device__ __forceinline__ int key_id(key64 k) { return (int)~(unsigned)k; }
__device__ __forceinline__ key64 key_max(key64 a, key64 b) { return b > a ? b : a; }
// compare-exchange for a descending order: a takes the larger key, b the other one (x ^ y ^
// max, so one compare serves both)
__device__ __forceinline__ void ce_desc(key64& a, key64& b) {
  const key64 x = a, y = b;
  const key64 m = y > x ? y : x;
  a = m;
  // v_bitop3 with truth table 0x96: the three-input xor
  const unsigned lo = __builtin_amdgcn_bitop3_b32((unsigned)x, (unsigned)y, (unsigned)m, 0x96);
  const unsigned hi = __builtin_amdgcn_bitop3_b32((unsigned)(x >> 32), (unsigned)(y >> 32),
                                                  (unsigned)(m >> 32), 0x96);
  b = ((key64)hi << 32) | lo;
}

// Sorts a bitonic sequence of N keys into descending order (half-cleaners of strides N/2..1).
template <int N>
__device__ __forceinline__ void bitonic_merge_desc(key64 (&k)[N]) {
#pragma unroll
  for (int st = N / 2; st >= 1; st >>= 1)
#pragma unroll
    for (int i = 0; i < N; ++i)
      if ((i & st) == 0) ce_desc(k[i], k[i + st]);
}

// L (descending) := the N largest keys of L and b (descending, M <= N): with b padded to N
// by the lowest key, max(L[i], b[N - 1 - i]) holds exactly those N keys as a bitonic
// sequence, which the half-cleaners sort.
template <int N, int M>
__device__ __forceinline__ void merge_into(key64 (&L)[N], const key64 (&b)[M]) {
#pragma unroll
  for (int i = 0; i < M; ++i) L[N - 1 - i] = key_max(L[N - 1 - i], b[i]);
  bitonic_merge_desc<N>(L);
}

// Inserts one key into L (descending).  Up to 8 slots: c_j = x > L[j] is monotone in j, so
// slot j keeps its key, takes x or takes its predecessor's (independent compares, depth 3);
// longer lists one compare-exchange step per slot (their masks would not stay in scalar
// registers).
template <int N>
__device__ __forceinline__ void key_insert(key64 (&L)[N], key64 x) {
  if constexpr (N > 8) {
#pragma unroll
    for (int j = 0; j < N; ++j) ce_desc(L[j], x);
    return;
  }
  bool c[N];
#pragma unroll
  for (int j = 0; j < N; ++j) c[j] = x > L[j];
#pragma unroll
  for (int j = N - 1; j >= 1; --j) L[j] = c[j] ? (c[j - 1] ? L[j - 1] : x) : L[j];
  L[0] = c[0] ? x : L[0];
}

// The four keys of a tile sorted descending (optimal 5-comparator network).
__device__ __forceinline__ void sort4_desc(key64 (&k)[4]) {
  ce_desc(k[0], k[1]);
  ce_desc(k[2], k[3]);
  ce_desc(k[0], k[2]);
  ce_desc(k[1], k[3]);
  ce_desc(k[1], k[2]);
}

// Cross-lane steps of the merges, all on the VALU.  Each replaces a lane's list by the top N
// of its own and a partner lane's list, which both lanes then hold:
//   1, 2: partner within the quad (DPP quad_perm swapping lanes 0-1/2-3, then 0-2/1-3);
//   4: within 8 lanes (DPP row_half_mirror: lane i and 7 - i, one from each quad);
//   8: within 16 lanes (DPP row_mirror: lane i and 15 - i, one from each half);
//   16, 32: v_permlane16_swap (rows 0-1, 2-3) / v_permlane32_swap (halves of the wave), which
//   return both lanes' values in the same order to both, so the two compute the same merge.
// Keys are pairwise distinct (pads are equal and interchangeable), so the merged, sorted list
// does not depend on which side a list came from.
template <int STEP>
__device__ __forceinline__ void both_sides(key64 x, key64& a, key64& b) {
  const unsigned lo = (unsigned)x, hi = (unsigned)(x >> 32);
  if constexpr (STEP <= 8) {
    constexpr int ctrl = STEP == 1 ? 0xB1 : STEP == 2 ? 0x4E : STEP == 4 ? 0x141 : 0x140;
    const unsigned plo = (unsigned)__builtin_amdgcn_update_dpp(0, (int)lo, ctrl, 0xF, 0xF, false);
    const unsigned phi = (unsigned)__builtin_amdgcn_update_dpp(0, (int)hi, ctrl, 0xF, 0xF, false);
    a = x;
    b = ((key64)phi << 32) | plo;
  } else {
    const auto l2 = STEP == 16 ? __builtin_amdgcn_permlane16_swap(lo, lo, false, false)
                               : __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto h2 = STEP == 16 ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                               : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    a = ((key64)h2[0] << 32) | l2[0];
    b = ((key64)h2[1] << 32) | l2[1];
  }
}

template <int STEP, int N>
__device__ __forceinline__ void merge_with_partner(key64 (&L)[N]) {
  // max(a[i], b[N - 1 - i]) over the pair (i, N - 1 - i), so each list is read before written
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const int j = N - 1 - i;
    key64 ai, bi, aj, bj;
    both_sides<STEP>(L[i], ai, bi);
    both_sides<STEP>(L[j], aj, bj);
    L[i] = key_max(ai, bj);
    L[j] = key_max(aj, bi);
  }
  bitonic_merge_desc<N>(L);
}

// Merges the lists of the lanes in one group (all 64 lanes for LANE_BITS_LO = 1, the 4 lanes
// n, n + 16, n + 32, n + 48 for LANE_BITS_LO = 16): afterwards every lane of it holds the
// group's best KMAX keys, descending.
template <int KMAX, int LANE_BITS_LO, int LANE_BITS_HI>
__device__ __forceinline__ void merge_lanes(key64 (&L)[KMAX]) {
  static_assert(LANE_BITS_HI == 32 && (LANE_BITS_LO == 1 || LANE_BITS_LO == 16), "groups");
  if constexpr (LANE_BITS_LO == 1) {
    merge_with_partner<1>(L);
    merge_with_partner<2>(L);
    merge_with_partner<4>(L);
    merge_with_partner<8>(L);
  }
  merge_with_partner<16>(L);
  merge_with_partner<32>(L);
}

// The ids of the first K keys of L (kNoId beyond K and for empty slots), sorted ascending.
template <int KMAX>
__device__ __forceinline__ void picks_of(const key64 (&L)[KMAX], int K, int (&pick)[KMAX]) {
#pragma unroll
  for (int r = 0; r < KMAX; ++r) pick[r] = r < K ? key_id(L[r]) : kNoId;
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

// Ranks the queries held in qv (columns n) against one candidate set (this wave's share of it:
// rounds of tiles part, part + parts, ..) and returns each query's best KMAX keys, descending,
// in L of every lane of column n (SINGLE: the one query, in every lane).
//   all_keys: candidates are all n_rows keys of the level;
//   else:     candidates are the B = 2^bshift children of each pick in pickv (lane i holds
//             pick i of the parent, i < K; ids outside [0, n_rows / B) are skipped), B / 16
//             tiles per pick.
template <int KMAX, bool SINGLE, int D>
__device__ __forceinline__ void rank_queries(const float* kh, int n_rows, bool all_keys,
                                             int pickv, int K, int bshift,
                                             const f32x4 (&qv)[D / 16], int n, int g,
                                             int part, int parts, key64 (&L)[KMAX]) {
  constexpr int kTilesPerRound = tiles_per_round(D);
#pragma unroll
  for (int j = 0; j < KMAX; ++j) L[j] = kPadKey;
  const int n_parent = n_rows >> bshift;
  const int sub_shift = bshift - 4;   // log2 of the tiles per pick
  const int tiles = all_keys ? (n_rows + 15) >> 4 : K << sub_shift;
  for (int t0 = part * kTilesPerRound; t0 < tiles; t0 += parts * kTilesPerRound) {
    f32x4 kv[kTilesPerRound][D / 16];
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
      load_tile<D>(kh, first[i], n_rows, n, g, kv[i]);
    }
#pragma unroll
    for (int i = 0; i < kTilesPerRound; ++i) {
      if (first[i] < 0) continue;
      const f32x4 acc = score_tile<D>(kv[i], qv);
      // branch-free: a candidate a lane does not take enters below every slot
      if constexpr (SINGLE) {
        // tile t = t0 + i is kept by the lanes with n / 4 == t % 4
        const int e = n & 3;
        const float sc = e == 0 ? acc[0] : e == 1 ? acc[1] : e == 2 ? acc[2] : acc[3];
        const int cid = first[i] + 4 * g + e;
        const bool take = (n >> 2) == ((t0 + i) & 3) && cid < n_rows;
        key_insert<KMAX>(L, make_key(sc, cid, take));
      } else {
        key64 tk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int cid = first[i] + 4 * g + e;
          tk[e] = make_key(acc[e], cid, cid < n_rows);
        }
        sort4_desc(tk);
        merge_into<KMAX, 4>(L, tk);
      }
    }
  }
  if constexpr (SINGLE) merge_lanes<KMAX, 1, 32>(L);
  else merge_lanes<KMAX, 16, 32>(L);
}

// The waves of selection workgroup bid of nblocks (renumbered per XCD).  With parts = 2 the
// two waves of a group each rank half of its candidate tiles, the second hands its lists to
// the first through LDS, and the first merges and stores (the keys' total order makes the
// picks independent of the split).
template <int KMAX, int D>
__device__ __forceinline__ void select_group(const SelArgs& a, int bid, int nblocks) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int K = a.topk;
  const int lo = a.lo;
  const int bs = a.bshift;
  const int parts = a.parts;
  const int n_lo = a.n >> (bs * lo);
  const int groups = (n_lo + 15) >> 4;
  const int slot = uniform(xcd_block(bid, nblocks) * kSelWaves + (int)(threadIdx.x >> 6));
  const int wave = uniform(slot / parts);          // the group
  const int part = uniform(slot - wave * parts);
  const bool active = wave < a.bh * groups;
  if (parts == 1 && !active) return;
  const int head = uniform(active ? wave / groups : 0);
  const int grp = uniform(active ? wave - head * groups : 0);
  const int q_id = grp * 16 + n;
  const bool qvalid = q_id < n_lo;
  key64 L[KMAX];

  if (active) {
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
          const float* qrow = a.q[lv - 1] + ((long)head * n_lv + anc) * D + (D / 4) * g;
          f32x4 qv[D / 16];
#pragma unroll
          for (int c = 0; c < D / 16; ++c) qv[c] = *(const f32x4*)(qrow + 4 * c);
          key64 La[KMAX];
          rank_queries<KMAX, true, D>(a.k[lv - 1] + (long)head * n_lv * D, n_lv, top, pickv, K,
                                      bs, qv, n, g, 0, 1, La);
          int pick[KMAX];
          picks_of<KMAX>(La, K, pick);
          int nv = kNoId;
#pragma unroll
          for (int r = 0; r < KMAX; ++r)
            if (lane == r) nv = pick[r];
          pickv = nv;
          if (part == 0 && ((grp << 4) & ((1 << shift) - 1)) == 0 && lane < K)
            a.sel[lv - 1][((long)head * n_lv + anc) * K + lane] = pickv;
        }
      }
    }

    // the group of 16 queries at level lo
    const float* qh = a.q[lo - 1] + (long)head * n_lo * D;
    f32x4 qv[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      qv[c] = qvalid ? *(const f32x4*)(qh + (long)q_id * D + (D / 4) * g + 4 * c)
                     : f32x4{0.f, 0.f, 0.f, 0.f};
    rank_queries<KMAX, false, D>(a.k[lo - 1] + (long)head * n_lo * D, n_lo, lo == a.levels,
                                 pickv, K, bs, qv, n, g, part, parts, L);
  }
  if (parts > 1) {   // every wave of the workgroup takes the barrier
    __shared__ key64 xl[kSelWaves / 2][16][KMAX];
    const int pair = (int)(threadIdx.x >> 7);
    if (active && part == 1 && g == 0) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j) xl[pair][n][j] = L[j];
    }
    __syncthreads();
    if (!active || part != 0) return;
#pragma unroll
    for (int i = 0; i < KMAX; ++i) L[i] = key_max(L[i], xl[pair][n][KMAX - 1 - i]);
    bitonic_merge_desc<KMAX>(L);
  }
  if (g == 0 && qvalid) {
    int pick[KMAX];
    picks_of<KMAX>(L, K, pick);
    int32_t* dst = a.sel[lo - 1] + ((long)head * n_lo + q_id) * K;
#pragma unroll
    for (int r = 0; r < KMAX; ++r)
      if (r < K) dst[r] = pick[r];
  }
}

template <int KMAX, int D>
__global__ __launch_bounds__(64 * kSelWaves) void select_kernel(SelArgs a) {
  select_group<KMAX, D>(a, blockIdx.x, gridDim.x);
}

// A selection launch that also pools V (its levels 1 and 2 from the tokens, or level 3 from
// level 2): the selection's workgroups come first (sel_blocks, a multiple of 8, so that their
// XCDs are those of a plain launch) and raise their waves' issue priority; the pooling
// workgroups after them fill the chip while the few selection waves run their dependent
// chains.  V is first read by the attention, so nothing in the launch depends on it.
template <int KMAX, int D>
__global__ __launch_bounds__(64 * kSelWaves) void select_pool12_kernel(SelArgs a, int sel_blocks,
                                                                       PoolArgs pa, int n,
                                                                       Grid grid, int gph) {
  __shared__ __attribute__((aligned(16))) float sh[kBlock][D];
  if ((int)blockIdx.x < sel_blocks) {
    __builtin_amdgcn_s_setprio(2);
    select_group<KMAX, D>(a, blockIdx.x, sel_blocks);
    return;
  }
  pool12_bf16_group<D>(pa, n, grid, gph, 0, (int)blockIdx.x - sel_blocks, sh);
}

template <int KMAX, int D>
__global__ __launch_bounds__(64 * kSelWaves) void select_pool_next_kernel(SelArgs a,
                                                                          int sel_blocks,
                                                                          PoolNextArgs pb,
                                                                          long total_out) {
  if ((int)blockIdx.x < sel_blocks) {
    __builtin_amdgcn_s_setprio(2);
    select_group<KMAX, D>(a, blockIdx.x, sel_blocks);
    return;
  }
  const long i = (long)((int)blockIdx.x - sel_blocks) * 256 + threadIdx.x;
  if (i < total_out) pool_next_elem<16, D>(pb, 0, i);
}

template <int D>
__global__ __launch_bounds__(256) void pool_next_v_kernel(PoolNextArgs pb, long total_out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < total_out) pool_next_elem<16, D>(pb, 0, i);
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

template <int KMAX, int D>
static hipError_t launch_select_kernels(const Shape& s, const SelArgs& a, unsigned blocks,
                                        const PoolInSelect& pv, hipStream_t stream) {
  const dim3 wg(64 * kSelWaves);
  if (pv.kind == 0) {
    LLSA_LAUNCH("select_kernel", (select_kernel<KMAX, D>), dim3(blocks), wg, 0, stream, a);
    return hipGetLastError();
  }
  const unsigned sb = (blocks + 7) / 8 * 8;
  if (pv.kind == 1) {
    const int gph = s.n >> (2 * kBlockShift);
    const Grid tg{s.hbits, s.wbits, s.raster};
    LLSA_LAUNCH("select_pool_kernel", (select_pool12_kernel<KMAX, D>),
                dim3(sb + (unsigned)(s.bh * gph)), wg, 0, stream, a, (int)sb, pv.pa, s.n, tg,
                gph);
  } else {
    LLSA_LAUNCH("select_pool_kernel", (select_pool_next_kernel<KMAX, D>),
                dim3(sb + (unsigned)((pv.total + 255) / 256)), wg, 0, stream, a, (int)sb,
                pv.pb, pv.total);
  }
  return hipGetLastError();
}

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
  // a group's candidate tiles at level lo: two waves share them where the groups are few
  // (levels >= 2) and there is more than one round of tiles
  const int tiles_lo = level_lo == s.levels ? (n_lo + 15) / 16 : s.topk << (s.bshift - 4);
  a.parts = level_lo >= 2 && tiles_lo > tiles_per_round(s.d) ? 2 : 1;
  const long waves = (long)s.bh * ((n_lo + 15) >> 4) * a.parts;   // parts per group
  const unsigned blocks = (unsigned)((waves + kSelWaves - 1) / kSelWaves);
  const auto by_k = [&](auto dc) {
    constexpr int D = decltype(dc)::value;
    if (s.topk <= 8) return launch_select_kernels<8, D>(s, a, blocks, pv, stream);
    if (s.topk <= 16) return launch_select_kernels<16, D>(s, a, blocks, pv, stream);
    return launch_select_kernels<32, D>(s, a, blocks, pv, stream);
  };
  return s.d == 64 ? by_k(std::integral_constant<int, 64>{})
                   : by_k(std::integral_constant<int, 128>{});
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
    pn.total = (long)s.bh * s.n_level(3) * s.d;
  }
  e = launch_select_range(s, lv[0], lv[1], sel, 1, 1, stream, pn);
  if (e != hipSuccess) return e;
  for (int l = 4; l <= L; ++l) {   // V's levels above 3: the plain kernel, level by level
    if (!lv[2][l - 1]) continue;
    if (!lv[2][l - 2]) return hipErrorInvalidValue;
    PoolNextArgs b{};
    b.in[0] = lv[2][l - 2];
    b.out[0] = lv[2][l - 1];
    const long total = (long)s.bh * s.n_level(l) * s.d;
    const dim3 g((unsigned)((total + 255) / 256));
    if (s.d == 64)
      LLSA_LAUNCH("pool_next_kernel", pool_next_v_kernel<64>, g, dim3(256), 0, stream, b, total);
    else
      LLSA_LAUNCH("pool_next_kernel", pool_next_v_kernel<128>, g, dim3(256), 0, stream, b, total);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace llsa
