// Coarse-to-fine top-K selection (paper summary sec. 三; article sec. 三).
//
// One wave scores a group of 16 level-l queries against a shared candidate list:
//   coarsest level L : the group's candidates are all n_L keys (full Q_L K_L^T);
//   level l < L      : the group is the 16 children of one level-(l+1) query P, and the
//                      candidates are the 16 children of each of P's K picks (K*B keys,
//                      one 16x16 score tile per pick, i.e. 16 contiguous key rows).
// Scores are fp32 dot products on the fp32 MFMA (v_mfma_f32_16x16x4f32) in the S^T
// orientation: lane (n, g) holds the scores of query n against candidates 4g..4g+3 of each
// tile.  Each lane streams its candidates through a register top-KMAX list, and the four
// lanes of a query merge their lists with cross-lane reductions.  Ties go to the lower id;
// the K picks are stored ascending.
#include "common.hpp"
#include "kernels.hpp"

namespace llsa {

constexpr int kSelWaves = 4;
constexpr int kNoId = 0x7fffffff;

__device__ __forceinline__ bool better(float s1, int i1, float s2, int i2) {
  return s1 > s2 || (s1 == s2 && i1 < i2);
}

template <int KMAX>
__device__ __forceinline__ void list_insert(float (&ls)[KMAX], int (&li)[KMAX], float s, int id) {
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const bool b = better(s, id, ls[j], li[j]);
    const float ts = ls[j];
    const int ti = li[j];
    ls[j] = b ? s : ts;
    li[j] = b ? id : ti;
    s = b ? ts : s;
    id = b ? ti : id;
  }
}

// q_l, k_l: [bh, n_l, 64] fp32.  parent: [bh, n_l / 16, K] (nullptr at the coarsest level).
// out: [bh, n_l, K].
template <int KMAX>
__global__ __launch_bounds__(64 * kSelWaves) void select_kernel(
    const float* __restrict__ q_l, const float* __restrict__ k_l,
    const int32_t* __restrict__ parent, int32_t* __restrict__ out, int bh, int n_l, int K,
    int coarsest) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * kSelWaves + (threadIdx.x >> 6);
  const int groups = (n_l + 15) >> 4;
  if (wave >= bh * groups) return;
  const int head = wave / groups;
  const int grp = wave - head * groups;
  const int n = lane & 15;
  const int g = lane >> 4;
  const float* qh = q_l + (long)head * n_l * kDim;
  const float* kh = k_l + (long)head * n_l * kDim;

  // B operand: Q[a][16g + s] for k-step s (the d axis is permuted so that each lane reads
  // 16 contiguous channels).
  const int a = grp * 16 + n;
  const bool qvalid = a < n_l;
  f32x4 qv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    qv[c] = qvalid ? *(const f32x4*)(qh + (long)a * kDim + 16 * g + 4 * c) : f32x4{0, 0, 0, 0};

  float ls[KMAX];
  int li[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    ls[j] = -INFINITY;
    li[j] = kNoId;
  }

  const int tiles = coarsest ? (n_l + 15) >> 4 : K;
  const int32_t* prow = coarsest ? nullptr : parent + ((long)head * (n_l >> 4) + grp) * K;
  const int n_parent = n_l >> 4;
  for (int ct = 0; ct < tiles; ++ct) {
    // candidate rows of this tile: first + r, r = 0..15
    int first;
    bool tile_ok = true;
    if (coarsest) {
      first = ct * 16;
    } else {
      const int pick = prow[ct];
      tile_ok = pick >= 0 && pick < n_parent;
      first = tile_ok ? pick * 16 : 0;
    }
    const int crow = first + n;   // A-operand row owned by this lane (m = lane & 15)
    const bool cvalid = tile_ok && crow < n_l;
    f32x4 kv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
      kv[c] = cvalid ? *(const f32x4*)(kh + (long)crow * kDim + 16 * g + 4 * c)
                     : f32x4{0, 0, 0, 0};
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = mfma_f32_k4(kv[c][e], qv[c][e], acc);
    // acc[i] = score of query n against candidate row first + 4g + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cid = first + 4 * g + i;
      if (tile_ok && cid < n_l) list_insert<KMAX>(ls, li, acc[i], cid);
    }
  }

  // merge the four lists of query n (lanes n, n+16, n+32, n+48)
  int pick[KMAX];
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    pick[r] = kNoId;
    if (r < K) {
      float bs = ls[0];
      int bi = li[0];
#pragma unroll
      for (int mask = 16; mask <= 32; mask <<= 1) {
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
  // ascending ids (kNoId entries beyond K sort last)
#pragma unroll
  for (int i = 0; i < KMAX; ++i)
#pragma unroll
    for (int j = 0; j + 1 < KMAX - i; ++j) {
      const int lo = min(pick[j], pick[j + 1]);
      const int hi = max(pick[j], pick[j + 1]);
      pick[j] = lo;
      pick[j + 1] = hi;
    }
  if (g == 0 && qvalid) {
    int32_t* dst = out + ((long)head * n_l + a) * K;
#pragma unroll
    for (int r = 0; r < KMAX; ++r)
      if (r < K) dst[r] = pick[r];
  }
}

hipError_t launch_select(const Shape& s, const float* const* q_lv, const float* const* k_lv,
                         int32_t* const* sel, int level_hi, int level_lo, hipStream_t stream) {
  for (int l = level_hi; l >= level_lo; --l) {
    const int n_l = s.n_level(l);
    const bool coarsest = (l == s.levels);
    const int groups = (n_l + 15) >> 4;
    const long waves = (long)s.bh * groups;
    const unsigned blocks = (unsigned)((waves + kSelWaves - 1) / kSelWaves);
    const int32_t* parent = coarsest ? nullptr : sel[l];
    if (s.topk <= 8)
      LLSA_LAUNCH("select_kernel", select_kernel<8>, dim3(blocks), dim3(64 * kSelWaves), 0, stream,
                         q_lv[l - 1], k_lv[l - 1], parent, sel[l - 1], s.bh, n_l, s.topk,
                         (int)coarsest);
    else
      LLSA_LAUNCH("select_kernel", select_kernel<16>, dim3(blocks), dim3(64 * kSelWaves), 0, stream,
                         q_lv[l - 1], k_lv[l - 1], parent, sel[l - 1], s.bh, n_l, s.topk,
                         (int)coarsest);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace llsa
