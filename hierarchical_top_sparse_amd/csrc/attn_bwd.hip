// Sparse attention backward (paper summary sec. 4.1 and Figure 4: the KV gradient is
// computed key-major over a CSR->CSC sparse index transpose, so no T x T mask is formed).
//
// Three stages, all deterministic (every sum in a fixed order; the only atomics are integer
// completion counts that order work, never sums of data):
//  1. bwd_query_kernel  (query-major, one wave per level-1 query block, one workgroup per
//     level-2 group of 16 blocks): D = sum_e P_e dP_e (exact, from the recomputed scores, so
//     the rounded O is never needed), dQ over the block's fine and coarse keys,
//     and, for the coarse keys, the workgroup's partial dK/dV sums (every query of a level-2
//     group shares the same coarse keys).
//  2. coarse_grad_kernel (one launch for all levels >= 2): each coarse key j of level l gathers
//     dK_l[j] = sum over the ancestors a in CSC_l[j] of the partials of a's slot holding j,
//     over every partial unit under a.
//  3. bwd_key_kernel (key-major, one one-wave workgroup per level-1 key block): walks the
//     query blocks in CSC_1[j] two at a time, accumulates dK, dV on the MFMA, and adds the
//     pooled gradients pushed down to the block's tokens (dK_l[ancestor] / 16^l, chain rule
//     of the mean).
//
// MFMA data flow (bf16 16x16x32, fp32 accumulation): products that contract over head_dim
// read row-major operands; products that contract over keys or queries read their row-major
// operand from LDS with ds_read_b64_tr_b16.  Chunks of 32 keys (or queries) use the same row
// interleave as the forward, so score tiles come out in the B-operand layout of the next MFMA.
// D (head_dim) is 64 or 128: rows, contraction chains and accumulators scale with it; with 128
// channels a query-major wave owns one query block instead of two (its accumulators double),
// so a level-2 group has 4 partial units instead of 2.
#include <mutex>

#include "../../include/llsa.h"
#include "common.hpp"
#include "kernels.hpp"

namespace llsa {

constexpr int kMaxLv = 6;
// LDS row stride in bf16 elements: D + 8 (144 bytes for 64 channels)
__host__ __device__ constexpr int bstride(int D) { return D + 8; }
constexpr int kMaxCoarse = 32;      // coarse slots handled by the fused partial sums

struct BwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* dout;
  const float* lse;
  const float* k_lv[kMaxLv];
  const float* v_lv[kMaxLv];
  const int32_t* sel[kMaxLv];
  const int32_t* csc_off[kMaxLv];
  const int32_t* csc_rows[kMaxLv];
  bf16* dq;
  bf16* dk;
  bf16* dv;
  float* dd;                   // D, [bh, N]
  float* part_k;               // [bh, n2, units, n_coarse, D]
  float* part_v;
  float* dk_lv[kMaxLv];        // level l >= 2: [bh, n_l, D]
  float* dv_lv[kMaxLv];
  const uint8_t* mask;         // block mask [bh, n_1, n_1] (mask-scanning key pass only)
  // key blocks with more than kKeyChunk CSC_1 entries: their entries beyond the first chunk go
  // to overflow chunks, each one wave of its own, whose partial sums the key block adds
  int32_t* ov_start;           // [bh, n_1] first overflow chunk of key block j
  int32_t* ov_count;           // [bh, n_1] overflow chunks of key block j
  int32_t* ov_table;           // [bh, ov_cap] chunk t: (key block << 16) | chunk index m >= 1
  int32_t* ov_total;           // [bh] overflow chunks of the head
  int32_t* ov_done;            // [bh, n_1] overflow chunks of key block j written (the plan
                               // sets them to 0)
  float* ov_part;              // [bh, ov_cap, 64 lanes, D / 2]: raw dK, dV sums of a chunk
  int ov_cap;                  // overflow chunks per head the buffers hold
  int ov_waves;                // overflow waves per head: wave g runs chunks g, g + ov_waves, ..
  int ov_blocks;               // leading workgroups of the key-major launch that run the
                               // overflow chunks (64 channels), or 0 (a launch of their own)
  int plan_blocks;             // leading workgroups of the query-major launch that run the
                               // overflow plan (one per head, padded to a multiple of 8), or 0
  int bh;
  int n;
  Grid grid;
  int levels;
  int topk;            // K: coarse keys per level
  int fine_k;          // picks per 16-token query block (rows of sel[0], CSC_1): K B / 16
  int bshift;          // log2(B) of the coarse levels: 4 or 6
  int enrich;          // 1 if there are coarse keys (coarse_levels > 0)
  int coarse_levels;   // coarse keys of levels 2 .. 1 + coarse_levels
  float lbias;         // log2-domain bias per level: log2(B) (weight B^l) or 0 (weight 1)
  int exclude;         // 1: a coarse key over a key selected one level finer is dropped
  float scale;
  float c2;   // scale * log2(e)
  int units_log2;      // log2 of the partial units (query-major workgroups) per level-2 group
};

__device__ __forceinline__ int chunk_key(int r, int t) { return 8 * (r >> 2) + (r & 3) + 4 * t; }

// x = hi + lo with both parts in bf16: the pair carries ~16 mantissa bits, so products that
// sum values of both signs (dS sums to zero per query) keep fp32-level accuracy on the MFMA.
__device__ __forceinline__ void split8(const float (&x)[2][4], bf16x8& hi, bf16x8& lo) {
  split8_bf16(f32x4{x[0][0], x[0][1], x[0][2], x[0][3]}, f32x4{x[1][0], x[1][1], x[1][2], x[1][3]},
              hi, lo);
}

__device__ __forceinline__ void split_f32x8(f32x4 a, f32x4 b, bf16x8& hi, bf16x8& lo) {
  split8_bf16(a, b, hi, lo);
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (bf16)0.f;
  return z;
}

// A operand (rows of a row-major LDS matrix): lane (m, g) gets row `row`, cols 32s + 8g..+7
template <int D>
__device__ __forceinline__ bf16x8 lds_row8(const bf16* st, int row, int s, int g) {
  return *(const bf16x8*)(st + row * bstride(D) + 32 * s + 8 * g);
}
// Transposed operand: rows k0 + 8g .. +7 (k axis) at column block 16*t4 (lane gets its column)
template <int D>
__device__ __forceinline__ bf16x8 lds_tr8(const bf16* st, int t4, int lane) {
  const int g = lane >> 4;
  const int r = (lane & 15) >> 2;
  const int c = lane & 3;
  const bf16* base = st + (8 * g + r) * bstride(D) + 16 * t4 + 4 * c;
  const bf16x4 lo = lds_read_tr16(base);
  const bf16x4 hi = lds_read_tr16(base + 4 * bstride(D));
  bf16x8 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    out[e] = lo[e];
    out[e + 4] = hi[e];
  }
  return out;
}

// ====================================================================== stage 1: query-major
// One workgroup per half of a level-2 group (8 query blocks, which share their coarse keys);
// each of its 4 waves owns 2 consecutive query blocks and works on its own:
//  * its 2 K picks are ranked in LDS into the ascending list U of distinct key blocks with a
//    2-bit mask of the blocks that picked each; U is streamed with row-major loads (16 K rows
//    and 16 V rows per block, two blocks ahead in registers) through the wave's LDS tiles;
//  * for each pick, one 16 x 16 tile: S^T = K Q^T and dP^T = V dO^T (16x16x32), P, P dP, and
//    A += K^T (P dP), Bv += K^T P (hi + lo parts, one 16x16x32 each), so D = sum P dP is
//    exact and dQ = scale (A - D Bv) needs one pass (the bf16 O is never read);
//  * the coarse keys (staged once per workgroup as bf16 hi + lo, each wave counting its share in
//    LDS and waiting for the count only where it reads them) add their tiles; at the end of
//    a block its coarse scores are recomputed in the Q K^T orientation, which puts P and dS in
//    the B-operand layout of the partial sums dV_c += P^T dO and dK_c += dS^T Q over the
//    block's queries (Q and dO rows staged in the wave's tiles);
//  * the 4 waves' partials are summed in a fixed order into the half-group's partial rows.
constexpr int kQWaves = 4;
// query blocks per wave: 2, or 1 with 128 channels
__host__ __device__ constexpr int q_blocks(int D) { return D == 64 ? 2 : 1; }
// partial units (workgroups) per level-2 group
__host__ __device__ constexpr int q_units(int D) { return kBlock / (kQWaves * q_blocks(D)); }
constexpr int kQPickList = 64;  // pick-list capacity per wave (pick slots per block: 64 / QB)
constexpr int kPickSentinel = 0x7f000000;

__host__ __device__ constexpr int bwdq_wave_lds_bytes(int D) {
  return 2 * 16 * bstride(D) * 2 + 4 * kQPickList * 4 + 48 * 4;
}
// ... then the coarse tiles, each slot's bias and key id, with overlap exclusion per-block
// biases [waves][blocks][ctiles * 16], and the count of waves that have staged their share of
// the coarse tiles.  The end-of-kernel reduction reuses the first kQWaves * 16 * D floats.
static size_t bwd_query_lds_bytes(int D, int n_coarse, bool exclude) {
  const int ctiles = (n_coarse + 15) / 16;
  const size_t bytes = (size_t)kQWaves * bwdq_wave_lds_bytes(D) +
                       (size_t)ctiles * 4 * 16 * bstride(D) * 2 +
                       (sizeof(float) + sizeof(int)) * 16 * ctiles +
                       (exclude ? sizeof(float) * kQWaves * q_blocks(D) * 16 * ctiles : 0) + 16;
  return std::max(bytes, sizeof(float) * kQWaves * 16 * D);
}

__device__ __forceinline__ void split4(const float (&x)[4], bf16x4& hi, bf16x4& lo) {
  split4_bf16(x[0], x[1], x[2], x[3], hi, lo);
}

__device__ void key_plan(const BwdArgs& a, int head, int* wsum);   // stage 3's plan

template <int NCT, int D>   // NCT: coarse tiles of 16 slots (0, 1 or 2); D: head_dim
__global__ __launch_bounds__(64 * kQWaves) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1)))
void bwd_query_kernel(BwdArgs a) {
  constexpr int kQBlocks = q_blocks(D);              // query blocks per wave
  constexpr int kUnits = q_units(D);                 // partial units per level-2 group
  constexpr int kQPickSlots = kQPickList / kQBlocks;   // pick slots per query block (K <= 32)
  constexpr int kStride = bstride(D);
  constexpr int PPR = D / 8;                         // 16-byte pieces per row
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int r4 = (lane & 15) >> 2, c4 = lane & 3;   // transposed-read lane roles
  const int n1 = a.n >> kBlockShift;
  const int n2 = n1 >> kBlockShift;
  if ((int)blockIdx.x < a.plan_blocks) {   // leading workgroups: the key-major overflow plan
    if ((int)blockIdx.x < a.bh) key_plan(a, blockIdx.x, (int*)smem);
    return;
  }
  const int unit =
      uniform(xcd_block(blockIdx.x - a.plan_blocks, gridDim.x - a.plan_blocks));
  const int head = uniform(unit / (kUnits * n2));
  const int rem = uniform(unit - head * kUnits * n2);
  const int a2 = rem / kUnits;
  const int pb_first = a2 * kBlock + (rem % kUnits) * (kBlock / kUnits) + kQBlocks * w;
  const int K = a.topk;
  const int KF = a.fine_k;
  const long tok_base = (long)head * a.n;
  const int n_coarse = NCT > 0 ? a.coarse_levels * K : 0;

  char* wb = smem + w * bwdq_wave_lds_bytes(D);
  bf16* kt = (bf16*)wb;                 // staged K rows (Q rows at a block's end)
  bf16* vt = kt + 16 * kStride;         // staged V rows (dO rows at a block's end)
  int* keys = (int*)(vt + 16 * kStride);
  int* sorted = keys + kQPickList;
  int* uoff = sorted + kQPickList;
  int* umask = uoff + kQPickList;
  float* lsh = (float*)(umask + kQPickList);   // [2][16] log2-domain LSE of the blocks' queries
  float* dsh = lsh + 32;                       // [16] D of the current block's queries
  bf16* ct = (bf16*)(smem + kQWaves * bwdq_wave_lds_bytes(D));   // [NCT][K hi, K lo, V hi, V lo]
  float* cbias = (float*)(ct + NCT * 4 * 16 * kStride);
  int* cid = (int*)(cbias + 16 * NCT);          // key id of each coarse slot (-1: none)
  float* wxb = (float*)(cid + 16 * NCT) + w * kQBlocks * 16 * NCT;   // exclusion: [bb][slot]
  int* staged =
      (int*)((float*)(cid + 16 * NCT) + (a.exclude ? kQWaves * kQBlocks * 16 * NCT : 0));
  if (NCT > 0) {
    if (tid == 0) *staged = 0;
    __syncthreads();   // the count is zero (the waves start together, so this costs little)
  }
  // A wave reads the coarse tiles only at the end of its blocks (or for the exclusion biases),
  // so each wave counts its staged share and goes on; a reader waits for the count.  The waves
  // of a workgroup are resident together and stage without waiting for anything.
  auto wait_staged = [&]() {
    while (__hip_atomic_load(staged, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < kQWaves)
      __builtin_amdgcn_s_sleep(1);
  };

  const uint32_t head_bytes = (uint32_t)a.n * D * 2;
  const rsrc_t rq = make_rsrc_uniform((const char*)a.q + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rk = make_rsrc_uniform((const char*)a.k + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rv = make_rsrc_uniform((const char*)a.v + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rdo =
      make_rsrc_uniform((const char*)a.dout + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rl = make_rsrc_uniform(a.lse + tok_base, (uint32_t)a.n * 4);

  // ---- the wave's picks (lane 32b + i: pick i of block b) and its query-side operands
  int key = kPickSentinel | lane;
  if ((lane % kQPickSlots) < KF) {
    const int j =
        a.sel[0][((long)head * n1 + pb_first + lane / kQPickSlots) * KF + lane % kQPickSlots];
    if (j >= 0 && j < n1) key = (j << 8) | lane;
  }
  bf16x8 qh[kQBlocks][D / 32], dh[kQBlocks][D / 32];   // B operands: lane (n, g) row n,
                                                       // channels 32s + 8g ..
  float lraw[kQBlocks];
#pragma unroll
  for (int bb = 0; bb < kQBlocks; ++bb) {
    const int pb = pb_first + bb;
    const uint32_t qrow =
        (uint32_t)(block_corner(pb, a.grid) + tile_offset(n, a.grid)) * D * 2;
#pragma unroll
    for (int s2 = 0; s2 < D / 32; ++s2) {
      qh[bb][s2] = buf_load8(rq, qrow + (32 * s2 + 8 * g) * 2);
      dh[bb][s2] = buf_load8(rdo, qrow + (32 * s2 + 8 * g) * 2);
    }
    lraw[bb] = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rl, (uint32_t)(pb * kBlock + n) * 4, 0, 0));
  }

  // ---- coarse keys of the group (slot e / PPR, channels 8 (e % PPR) ..): bf16 hi + lo parts
  if (NCT > 0) {
    for (int e = tid; e < NCT * 16 * PPR; e += 64 * kQWaves) {
      const int cslot = e / PPR, c8 = (e % PPR) * 8;
      f32x4 k0 = {0.f, 0.f, 0.f, 0.f}, k1 = k0, v0 = k0, v1 = k0;
      float bias = -INFINITY;
      int cslot_id = -1;
      if (cslot < n_coarse) {
        const int l = 2 + cslot / K;
        const int nl = a.n >> (a.bshift * l);
        const int anc = (a2 << (2 * kBlockShift)) >> (a.bshift * l);   // level-l ancestor
        const int id = a.sel[l - 1][((long)head * nl + anc) * K + (cslot - (l - 2) * K)];
        if (id >= 0 && id < nl) {
          cslot_id = id;
          const float* kp = a.k_lv[l - 1] + ((long)head * nl + id) * D + c8;
          const float* vp = a.v_lv[l - 1] + ((long)head * nl + id) * D + c8;
          k0 = *(const f32x4*)kp;
          k1 = *(const f32x4*)(kp + 4);
          v0 = *(const f32x4*)vp;
          v1 = *(const f32x4*)(vp + 4);
          bias = a.lbias * (float)l;   // log2(B^l), or 0 for unit weights
          if (a.exclude && l >= 3 && c8 == 0) {
            // level >= 3: dropped for the whole group if it is the parent of one of the keys
            // selected at level l - 1 for the group's level-(l-1) ancestor
            const int nf = a.n >> (a.bshift * (l - 1));
            const int ancf = (a2 << (2 * kBlockShift)) >> (a.bshift * (l - 1));
            for (int i = 0; i < K; ++i)
              if ((a.sel[l - 2][((long)head * nf + ancf) * K + i] >> a.bshift) == id)
                bias = -INFINITY;
          }
        }
      }
      bf16* base = ct + (cslot >> 4) * 4 * 16 * kStride + (cslot & 15) * kStride + c8;
      bf16x8 hi, lo;
      split_f32x8(k0, k1, hi, lo);
      *(bf16x8*)base = hi;
      *(bf16x8*)(base + 16 * kStride) = lo;
      split_f32x8(v0, v1, hi, lo);
      *(bf16x8*)(base + 32 * kStride) = hi;
      *(bf16x8*)(base + 48 * kStride) = lo;
      if (c8 == 0) {
        cbias[cslot] = bias;
        cid[cslot] = cslot_id;
      }
    }
  }

  // ---- U: ranks of the wave's pick keys, distinct ids, owner masks
  keys[lane] = key;
  umask[lane] = 0;
  if (g < kQBlocks) lsh[16 * g + n] = (g == 0 ? lraw[0] : lraw[kQBlocks - 1]) * kLog2e;
  wave_lds_sync();
  {
    int r = 0;
#pragma unroll 4
    for (int u = 0; u < kQPickList; u += 4) {
      const i32x4 kk = *(const i32x4*)(keys + u);
#pragma unroll
      for (int e = 0; e < 4; ++e) r += kk[e] < key ? 1 : 0;
    }
    sorted[r] = key;
  }
  wave_lds_sync();
  float lse2[kQBlocks];   // log2-domain LSE of query n of each block
#pragma unroll
  for (int bb = 0; bb < kQBlocks; ++bb) lse2[bb] = lraw[bb] * kLog2e;
  const int sk = sorted[lane];
  const bool valid = sk < kPickSentinel;
  const int prev = sorted[lane > 0 ? lane - 1 : 0];
  const bool first = valid && (lane == 0 || (prev >> 8) != (sk >> 8));
  const uint64_t fm = __builtin_amdgcn_ballot_w64(first);
  const int n_u = uniform(__builtin_popcountll(fm));
  {
    const int u = __builtin_popcountll(fm & (~0ull >> (63 - lane))) - 1;
    if (first) {   // the run of this key block: one entry per block that picked it
      int m = 0;
      for (int r = lane; r < min(lane + kQBlocks, kQPickList); ++r) {
        const int o = sorted[r];
        if ((o >> 8) != (sk >> 8)) break;
        m |= 1 << ((o & 63) / kQPickSlots);
      }
      uoff[u] = block_corner(sk >> 8, a.grid) * D * 2;
      umask[u] = m;
    }
  }
  wave_lds_sync();

  // ---- the stream of U: row-major loads (lane l: pieces l, l + 64, .. of 16 rows x PPR
  // pieces)
  constexpr int kLd = 16 * PPR / 64;
  uint32_t poff[kLd];
#pragma unroll
  for (int m = 0; m < kLd; ++m) {
    const int e = lane + 64 * m;
    poff[m] = (uint32_t)tile_offset(e / PPR, a.grid) * D * 2 + 16 * (e % PPR);
  }
  struct BlockLd {
    i32x4 k[kLd], v[kLd];
  };
  auto load_u = [&](int u) -> BlockLd {
    BlockLd f;
    const uint32_t b = u < n_u ? (uint32_t)uniform(uoff[min(u, kQPickList - 1)]) : kNoRow;
#pragma unroll
    for (int m = 0; m < kLd; ++m) {
      f.k[m] = __builtin_amdgcn_raw_buffer_load_b128(rk, b + poff[m], 0, 0);
      f.v[m] = __builtin_amdgcn_raw_buffer_load_b128(rv, b + poff[m], 0, 0);
    }
    return f;
  };
  BlockLd fa = load_u(0), fb = load_u(1);
  if (NCT > 0) {
    if (lane == 0)   // this wave's share of the coarse tiles is staged
      __hip_atomic_fetch_add(staged, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    // with overlap exclusion, per-block biases: a level-2 slot is dropped for block bb if one
    // of bb's fine picks lies in its span (the 16-token block j is in key (16 j) >> 2 log2(B))
    if (a.exclude) {
      wait_staged();
      for (int sl = lane; sl < 16 * NCT; sl += 64) {
        const int id = cid[sl];
        const bool lv2 = sl < K && id >= 0;
#pragma unroll
        for (int bb = 0; bb < kQBlocks; ++bb) {
          bool hit = false;
          if (lv2)
            for (int i = 0; i < KF; ++i) {
              const int kk = keys[kQPickSlots * bb + i];
              hit |= kk < kPickSentinel &&
                     (((kk >> 8) << kBlockShift) >> (2 * a.bshift)) == id;
            }
          wxb[bb * 16 * NCT + sl] = hit ? -INFINITY : cbias[sl];
        }
      }
      wave_lds_sync();
    }
  }

  f32x4 acc_a[kQBlocks][D / 16], acc_b[kQBlocks][D / 16];
  float dpart[kQBlocks];
#pragma unroll
  for (int bb = 0; bb < kQBlocks; ++bb) {
    dpart[bb] = 0.f;
#pragma unroll
    for (int t4 = 0; t4 < D / 16; ++t4)
      acc_a[bb][t4] = acc_b[bb][t4] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One 16-key tile of block bb: K rows kr (+ lo parts klo), V rows vr (+ vlo), per-key biases.
  auto tile = [&](auto bbc, const bf16* kr, const bf16* klo, const bf16* vr, const bf16* vlo,
                  const float* kbias) {
    constexpr int bb = decltype(bbc)::value;
    f32x4 st = {0.f, 0.f, 0.f, 0.f}, dp = st;
#pragma unroll
    for (int s2 = 0; s2 < D / 32; ++s2) {
      st = mfma_bf16_k32(lds_row8<D>(kr, n, s2, g), qh[bb][s2], st);
      dp = mfma_bf16_k32(lds_row8<D>(vr, n, s2, g), dh[bb][s2], dp);
      if (klo) {
        st = mfma_bf16_k32(lds_row8<D>(klo, n, s2, g), qh[bb][s2], st);
        dp = mfma_bf16_k32(lds_row8<D>(vlo, n, s2, g), dh[bb][s2], dp);
      }
    }
    float p[4], w1[4];
    f32x4 b4 = {0.f, 0.f, 0.f, 0.f};
    if (kbias) b4 = *(const f32x4*)(kbias + 4 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = fast_exp2(fmaf(st[i], a.c2, b4[i] - lse2[bb]));
      w1[i] = p[i] * dp[i];
      dpart[bb] += w1[i];
    }
    bf16x4 a_hi, a_lo, b_hi, b_lo;
    split4(w1, a_hi, a_lo);
    split4(p, b_hi, b_lo);
#pragma unroll
    for (int t4 = 0; t4 < D / 16; ++t4) {
      const int off = (4 * g + r4) * kStride + 16 * t4 + 4 * c4;
      const bf16x4 ktr = lds_read_tr16(kr + off);
      acc_a[bb][t4] = mfma_bf16_k16x2(ktr, a_hi, ktr, a_lo, acc_a[bb][t4]);
      acc_b[bb][t4] = mfma_bf16_k16x2(ktr, b_hi, ktr, b_lo, acc_b[bb][t4]);
      if (klo) {
        const bf16x4 ktl = lds_read_tr16(klo + off);
        acc_a[bb][t4] = mfma_bf16_k16(ktl, a_hi, acc_a[bb][t4]);
        acc_b[bb][t4] = mfma_bf16_k16(ktl, b_hi, acc_b[bb][t4]);
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  auto block_u = [&](const BlockLd& f, int u) {
#pragma unroll
    for (int m = 0; m < kLd; ++m) {
      const int e = lane + 64 * m;
      const int at = (e / PPR) * kStride + (e % PPR) * 8;
      *(i32x4*)(kt + at) = f.k[m];
      *(i32x4*)(vt + at) = f.v[m];
    }
    wave_lds_sync();
    const int mask = uniform(umask[u]);
    if (mask & 1) tile(I0{}, kt, nullptr, vt, nullptr, nullptr);
    if constexpr (kQBlocks > 1)
      if (mask & 2) tile(I1{}, kt, nullptr, vt, nullptr, nullptr);
    wave_lds_sync();
  };
  for (int u = 0; u < n_u; u += 2) {
    block_u(fa, u);
    fa = load_u(u + 2);
    if (u + 1 >= n_u) break;
    block_u(fb, u + 1);
    fb = load_u(u + 3);
  }

  // C^T[d][slot]: lane (slot, g)
  f32x4 cpk[NCT > 0 ? NCT : 1][D / 16], cpv[NCT > 0 ? NCT : 1][D / 16];
#pragma unroll
  for (int c = 0; c < (NCT > 0 ? NCT : 1); ++c)
#pragma unroll
    for (int t4 = 0; t4 < D / 16; ++t4) cpk[c][t4] = cpv[c][t4] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto finish = [&](auto bbc) {
    constexpr int bb = decltype(bbc)::value;
    const int pb = pb_first + bb;
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const bf16* cb0 = ct + c * 4 * 16 * kStride;
      tile(bbc, cb0, cb0 + 16 * kStride, cb0 + 32 * kStride, cb0 + 48 * kStride,
           (a.exclude ? wxb + bb * 16 * NCT : cbias) + 16 * c);
    }
    const float Dn = group4_sum(dpart[bb]);
    if (g == 0) a.dd[tok_base + pb * kBlock + n] = Dn;
    const int qrow = block_corner(pb, a.grid) + tile_offset(n, a.grid);
    bf16* dqp = a.dq + (tok_base + qrow) * D;
#pragma unroll
    for (int t4 = 0; t4 < D / 16; ++t4) {
      f32x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = (acc_a[bb][t4][i] - Dn * acc_b[bb][t4][i]) * a.scale;
      *(bf16x4*)(dqp + 16 * t4 + 4 * g) = pack4_bf16(r);
    }
    if (NCT > 0) {
      // Q and dO rows of the block (row n = query n) in the wave's tiles, D per query
#pragma unroll
      for (int s2 = 0; s2 < D / 32; ++s2) {
        *(bf16x8*)(kt + n * kStride + 32 * s2 + 8 * g) = qh[bb][s2];
        *(bf16x8*)(vt + n * kStride + 32 * s2 + 8 * g) = dh[bb][s2];
      }
      if (g == 0) dsh[n] = Dn;
      wave_lds_sync();
      const f32x4 dq4 = *(const f32x4*)(dsh + 4 * g);          // D of queries 4g + i
      const f32x4 lq4 = *(const f32x4*)(lsh + 16 * bb + 4 * g);  // LSE of queries 4g + i
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        const bf16* cb0 = ct + c * 4 * 16 * kStride;
        // S = Q K_c^T, dP = dO V_c^T: lane (n, g) holds queries 4g + i against slot n
        f32x4 sq = {0.f, 0.f, 0.f, 0.f}, dpq = sq;
#pragma unroll
        for (int s2 = 0; s2 < D / 32; ++s2) {
          sq = mfma_bf16_k32(qh[bb][s2], lds_row8<D>(cb0, n, s2, g), sq);
          sq = mfma_bf16_k32(qh[bb][s2], lds_row8<D>(cb0 + 16 * kStride, n, s2, g), sq);
          dpq = mfma_bf16_k32(dh[bb][s2], lds_row8<D>(cb0 + 32 * kStride, n, s2, g), dpq);
          dpq = mfma_bf16_k32(dh[bb][s2], lds_row8<D>(cb0 + 48 * kStride, n, s2, g), dpq);
        }
        const float bias = (a.exclude ? wxb + bb * 16 * NCT : cbias)[16 * c + n];
        float pq[4], sv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pq[i] = fast_exp2(fmaf(sq[i], a.c2, bias - lq4[i]));
          sv[i] = pq[i] * (dpq[i] - dq4[i]);
        }
        bf16x4 p_hi, p_lo, s_hi, s_lo;
        split4(pq, p_hi, p_lo);
        split4(sv, s_hi, s_lo);
#pragma unroll
        for (int t4 = 0; t4 < D / 16; ++t4) {
          const int off = (4 * g + r4) * kStride + 16 * t4 + 4 * c4;
          const bf16x4 dot = lds_read_tr16(vt + off);   // dO^T
          const bf16x4 qtt = lds_read_tr16(kt + off);   // Q^T
          cpv[c][t4] = mfma_bf16_k16x2(dot, p_hi, dot, p_lo, cpv[c][t4]);
          cpk[c][t4] = mfma_bf16_k16x2(qtt, s_hi, qtt, s_lo, cpk[c][t4]);
        }
      }
      wave_lds_sync();
    }
  };
  if (NCT > 0) wait_staged();
  finish(I0{});
  if constexpr (kQBlocks > 1) finish(I1{});

  if (NCT > 0) {
    // ---- the 4 waves' partials summed in wave order (0 + 1 + 2 + 3) into the unit's rows,
    // one chunk (a coarse tile's dK or dV: 16 slots x 64 floats) at a time: every wave stores
    // its part in its own LDS region, then every thread adds 4 elements of the 4 regions and
    // stores them, so no wave waits for another's turn.  All earlier LDS use is over after
    // the first barrier.
    float* red = (float*)smem;   // [kQWaves][16 * D]
    constexpr int kChunk = 16 * D;
    const long out_base = ((long)head * kUnits * n2 + rem) * n_coarse * D;
#pragma unroll
    for (int chunk = 0; chunk < 2 * NCT; ++chunk) {
      const int c = chunk >> 1;
      const bool is_v = chunk & 1;
      __syncthreads();
#pragma unroll
      for (int t4 = 0; t4 < D / 16; ++t4)
        *(f32x4*)(red + w * kChunk + n * D + 16 * t4 + 4 * g) = is_v ? cpv[c][t4] : cpk[c][t4];
      __syncthreads();
#pragma unroll
      for (int it = 0; it < kChunk / (4 * 64 * kQWaves); ++it) {
        // elements e .. e + 3 of the chunk: slot 16 c + e / D
        const int e = 4 * tid + 4 * 64 * kQWaves * it;
        f32x4 sum = *(const f32x4*)(red + e);
#pragma unroll
        for (int r = 1; r < kQWaves; ++r) sum += *(const f32x4*)(red + r * kChunk + e);
        if (16 * c + e / D < n_coarse) {
          if (is_v)
            *(f32x4*)(a.part_v + out_base + (long)c * kChunk + e) = sum;
          else
            *(f32x4*)(a.part_k + out_base + (long)c * kChunk + e) = sum * a.scale;
        }
      }
    }
  }
}

// ====================================================================== stage 2: coarse keys
// dK_l[j] = sum over the ancestors a in CSC_l[j] of the partial rows of a's slot holding j, over
// every partial unit under a (2^units_log2 per level-2 group, 16^(l-2) groups per level-l query).
// One launch for all levels l >= 2, 8-wave workgroups (measured against 16-wave ones at 256^2
// b2: 17 us against 21 us per launch):
//  * level 2: one wave per key (8 keys per workgroup); a key sums about K * units rows;
//  * level >= 3: one workgroup per key; its rows (entry, unit) are dealt round-robin to the 8
//    waves and the waves' sums are added in a fixed order.
// Lanes first resolve up to 64 CSC entries into partial-row offsets (lane = entry); every lane
// then sums one channel of the rows, kCgBatch rows per round with all their loads in flight
// (buffer loads: rows of missing entries read offset kNoRow, i.e. zeros); with 128 channels
// a lane sums channels lane and lane + 64.  Deterministic.
constexpr int kCgWaves = 8;
constexpr int kCgBatch = 16;

struct CoarseGradArgs {
  int first_block[kMaxLv + 1];   // level l's workgroups start at first_block[l - 1]
};

// Sums over this wave's share (rows i = part, part + nparts, ...) of key j's partial rows:
// sk[h], sv[h] for channel lane + 64 h.
template <int D>
__device__ __forceinline__ void coarse_key_sum(const BwdArgs& a, int l, int head, int j,
                                               int part, int nparts, int lane,
                                               float (&sk)[D / 64], float (&sv)[D / 64]) {
  constexpr int H = D / 64;
  constexpr int kBatch = kCgBatch / H;   // rows in flight per round (registers: 4 H kBatch)
  const int K = a.topk;
  const int nl = a.n >> (a.bshift * l);
  const int n2 = a.n >> (2 * kBlockShift);   // 256-token groups (the partials' layout)
  const int n_coarse = a.coarse_levels * K;
  // partial units (of 256 / units tokens) under one level-l ancestor
  const int span = 1 << (a.bshift * l - 2 * kBlockShift + a.units_log2);
  const uint32_t row_bytes = (uint32_t)n_coarse * D * 4;   // one unit's partial rows
  const uint32_t head_bytes = ((uint32_t)n2 << a.units_log2) * row_bytes;
  const long head_floats = ((long)n2 << a.units_log2) * n_coarse * D;
  const rsrc_t rk = make_rsrc_uniform(a.part_k + head * head_floats, head_bytes);
  const rsrc_t rv = make_rsrc_uniform(a.part_v + head * head_floats, head_bytes);
  const int32_t* off = a.csc_off[l - 1] + (long)head * (nl + 1);
  const int32_t* rows = a.csc_rows[l - 1] + (long)head * nl * K;
  const int32_t* sel = a.sel[l - 1] + (long)head * nl * K;
  const int e0 = uniform(off[j]);
  const int e1 = uniform(off[j + 1]);
  float ak[H][kBatch], av[H][kBatch];
#pragma unroll
  for (int h = 0; h < H; ++h)
#pragma unroll
    for (int u = 0; u < kBatch; ++u) ak[h][u] = av[h][u] = 0.f;
  for (int base = e0; base < e1; base += 64) {
    const int cnt = min(64, e1 - base);
    // lane e: byte offset of entry e's row in unit 0 under its ancestor (kNoRow if none)
    uint32_t src = kNoRow;
    if (lane < cnt) {
      const int anc = rows[base + lane];
      if (anc >= 0 && anc < nl) {
        int slot = -1;
        for (int s = 0; s < K; ++s)
          if (sel[(long)anc * K + s] == j) slot = s;
        if (slot >= 0)
          src = (uint32_t)anc * span * row_bytes + (uint32_t)((l - 2) * K + slot) * D * 4;
      }
    }
    const int total = cnt * span;
    for (int i0 = part; i0 < total; i0 += nparts * kBatch) {
      float xk[H][kBatch], xv[H][kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int i = i0 + u * nparts;
        const int e = i < total ? i / span : 0;
        const uint32_t r = (uint32_t)__builtin_amdgcn_readlane((int)src, e);
        const uint32_t o = (i < total && r != kNoRow)
                               ? r + (uint32_t)(i - e * span) * row_bytes + 4 * lane
                               : kNoRow;
#pragma unroll
        for (int h = 0; h < H; ++h) {
          const uint32_t oh = o == kNoRow ? kNoRow : o + 256 * h;
          xk[h][u] =
              __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rk, oh, 0, 0));
          xv[h][u] =
              __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rv, oh, 0, 0));
        }
      }
#pragma unroll
      for (int h = 0; h < H; ++h)
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          ak[h][u] += xk[h][u];
          av[h][u] += xv[h][u];
        }
    }
  }
#pragma unroll
  for (int h = 0; h < H; ++h) {
#pragma unroll
    for (int w = kBatch / 2; w >= 1; w >>= 1)
#pragma unroll
      for (int u = 0; u < w; ++u) {
        ak[h][u] += ak[h][u + w];
        av[h][u] += av[h][u + w];
      }
    sk[h] = ak[h][0];
    sv[h] = av[h][0];
  }
}

template <int D>
__global__ __launch_bounds__(64 * kCgWaves) void coarse_grad_kernel(BwdArgs a,
                                                                    CoarseGradArgs cg) {
  constexpr int H = D / 64;
  __shared__ float red[2][kCgWaves][D];
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int bid = blockIdx.x;
  if (bid < cg.first_block[2]) {   // level 2: one wave per key
    const int n2 = a.n >> (2 * a.bshift);
    const int f = bid * kCgWaves + w;
    if (f >= a.bh * n2) return;
    const int head = uniform(f / n2);
    const int j = uniform(f - head * n2);
    float sk[H], sv[H];
    coarse_key_sum<D>(a, 2, head, j, 0, 1, lane, sk, sv);
#pragma unroll
    for (int h = 0; h < H; ++h) {
      a.dk_lv[1][((long)head * n2 + j) * D + lane + 64 * h] = sk[h];
      a.dv_lv[1][((long)head * n2 + j) * D + lane + 64 * h] = sv[h];
    }
    return;
  }
  int l = 3;
  while (l < a.levels && bid >= cg.first_block[l]) ++l;
  const int nl = a.n >> (a.bshift * l);
  const int idx = bid - cg.first_block[l - 1];
  const int head = uniform(idx / nl);
  const int j = uniform(idx - head * nl);
  float sk[H], sv[H];
  coarse_key_sum<D>(a, l, head, j, w, kCgWaves, lane, sk, sv);
#pragma unroll
  for (int h = 0; h < H; ++h) {
    red[0][w][lane + 64 * h] = sk[h];
    red[1][w][lane + 64 * h] = sv[h];
  }
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int h = 0; h < H; ++h) {
      float tk = 0.f, tv = 0.f;
#pragma unroll
      for (int x = 0; x < kCgWaves; ++x) {
        tk += red[0][x][lane + 64 * h];
        tv += red[1][x][lane + 64 * h];
      }
      a.dk_lv[l - 1][((long)head * nl + j) * D + lane + 64 * h] = tk;
      a.dv_lv[l - 1][((long)head * nl + j) * D + lane + 64 * h] = tv;
    }
  }
}

// ====================================================================== stage 3: key-major
// One wave per workgroup: key blocks differ widely in how many query blocks picked them, so a
// wave that finishes early frees its slot at once.  A key block takes at most kKeyChunk CSC_1
// entries itself; the rest of a popular block (a block every query block picks, as a key
// with a large norm becomes under random weights) is cut into chunks of kKeyChunk that
// overflow waves run, each writing raw partial sums that the key block's wave adds in chunk
// order: the work stays balanced and the result deterministic.  With 64 channels the overflow
// waves lead the key-major launch and count each written chunk per key block (a device-scope
// release); a key block with chunks waits for its count (an acquire) before adding them, so an
// empty plan costs nothing beyond a few idle waves.  With 128 channels they have a launch of
// their own (one wave per SIMD: two would spill), and the count is complete before the key
// blocks start.
// Modes:
//  * kKeyCsc: the key block's first chunk of CSC_1[j], plus its overflow partials, then store;
//  * kKeyOverflow: overflow chunks (numbered by the plan), partial sums only; a head's
//    kOvWaves waves take its chunks in turn;
//  * kKeyMask: the comparator of a mask-based backward -- the query blocks of key block j are
//    found by scanning column j of the dense block mask (all n_1 query blocks) instead of
//    reading CSC_1[j]; the scan yields them in ascending order, the order of the CSC rows, and
//    they are processed in the same batches of 64 (no chunking), so both variants give
//    bit-identical dK and dV when no key block has more than kKeyChunk picks.
constexpr int kKeyChunk = 128;
constexpr int kKeyCsc = 0, kKeyMask = 1, kKeyOverflow = 2;
constexpr int kOvWaves = 64;   // overflow waves per head (each loops over chunks)

// Overflow plan of one head, run by one 256-thread workgroup: a key block with c > kKeyChunk
// entries has (c - 1) / kKeyChunk overflow chunks, numbered by an exclusive scan over the key
// blocks.  Rounds of 256 blocks (thread t takes block 256 r + t, coalesced), each scanned with
// wave shuffles plus four wave totals in LDS; the next round's offsets load during the scan.
__device__ void key_plan(const BwdArgs& a, int head, int* wsum) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int n1 = a.n >> kBlockShift;
  const int32_t* off = a.csc_off[0] + (long)head * (n1 + 1);
  int32_t* ovs = a.ov_start + (long)head * n1;
  int32_t* ovc = a.ov_count + (long)head * n1;
  int32_t* tab = a.ov_table + (long)head * a.ov_cap;
  int32_t* done = a.ov_done + (long)head * n1;
  auto entries = [&](int c) { return c < n1 ? off[c + 1] - off[c] : 0; };
  int cnt = entries(t);
  int base = 0;
  for (int c0 = 0; c0 < n1; c0 += 256) {
    const int c = c0 + t;
    const int next = entries(c + 256);
    const int ov = cnt > 0 ? (cnt - 1) / kKeyChunk : 0;
    int x = ov;   // inclusive scan over the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d, 64);
      if (lane >= d) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int start = base + x - ov;
    for (int u = 0; u < w; ++u) start += wsum[u];
    base += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();   // the totals are rewritten by the next round
    if (c < n1) {
      ovs[c] = start;
      ovc[c] = ov;
      done[c] = 0;
      for (int m = 1; m <= ov; ++m) tab[start + m - 1] = (c << 16) | m;
    }
    cnt = next;
  }
  if (t == 0) a.ov_total[head] = base;
}

// One key block's share of the key-major pass: chunk `chunk` of CSC_1[j] (kKeyCsc: chunk 0
// plus the overflow partials, then the store; kKeyOverflow: partial sums into slot ov_t), or
// the whole mask column j (kKeyMask).
template <int MODE, int D>
__device__ __forceinline__ void key_block(const BwdArgs& a, int head, int j, int chunk, int ov_t,
                                          bf16* stQ, bf16* stO, float* pdown, float* stL,
                                          int* pend) {
  constexpr bool MASK = MODE == kKeyMask;
  constexpr int H = D / 64;               // channels per lane in the push-down
  constexpr int kStride = bstride(D);
  constexpr int PPR = D / 8;              // 16-byte pieces per row
  constexpr int RPI = 64 / PPR;           // rows per load instruction
  constexpr int NINS = 32 / RPI;          // load instructions for a pair's 32 rows
  const int lane = threadIdx.x;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int n1 = a.n >> kBlockShift;
  const long tok_base = (long)head * a.n;

  // pooled-key gradients pushed down to this block (lane = channel, + 64 h), loaded first so
  // that they arrive during the CSC lookups instead of after the pair loop
  float pk_sum[H], pv_sum[H];
#pragma unroll
  for (int h = 0; h < H; ++h) pk_sum[h] = pv_sum[h] = 0.f;
  if (MODE != kKeyOverflow && a.enrich) {
    for (int l = 2; l <= 1 + a.coarse_levels; ++l) {
      const int nl = a.n >> (a.bshift * l);
      const int anc = (j << kBlockShift) >> (a.bshift * l);
      const float f = 1.0f / (float)(1 << (a.bshift * l));
#pragma unroll
      for (int h = 0; h < H; ++h) {
        pk_sum[h] += a.dk_lv[l - 1][((long)head * nl + anc) * D + lane + 64 * h] * f;
        pv_sum[h] += a.dv_lv[l - 1][((long)head * nl + anc) * D + lane + 64 * h] * f;
      }
    }
  }

  const uint32_t head_bytes = (uint32_t)a.n * D * 2;
  const rsrc_t rq = make_rsrc_uniform((const char*)a.q + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rk = make_rsrc_uniform((const char*)a.k + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rv = make_rsrc_uniform((const char*)a.v + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rdo =
      make_rsrc_uniform((const char*)a.dout + (size_t)head * head_bytes, head_bytes);
  const float* lse_h = a.lse + tok_base;   // the head's LSE and D
  const float* dd_h = a.dd + tok_base;

  // keys of this block as B operands: lane (n, g) holds row n, channels 32s + 8g .. +7
  const int krow = block_corner(j, a.grid) + tile_offset(n, a.grid);
  // (the key-major pass over CSC_1 loads them once it knows the block has picks: below)
  bf16x8 kh[D / 32], vh[D / 32];
  if constexpr (MODE != kKeyCsc) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      kh[s] = buf_load8(rk, (uint32_t)(krow * D + 32 * s + 8 * g) * 2);
      vh[s] = buf_load8(rv, (uint32_t)(krow * D + 32 * s + 8 * g) * 2);
    }
  }

  // lane-constant offsets: staged rows (bytes) and this lane's 4 queries per tile (tokens)
  const int srow0 = lane / PPR;
  const int piece = lane % PPR;
  uint32_t st_off[NINS];
#pragma unroll
  for (int ins = 0; ins < NINS; ++ins)
    st_off[ins] = (uint32_t)(tile_offset((ins * RPI + srow0) & 15, a.grid) * D * 2 + 16 * piece);
  const bool lane_second = g >= 2;   // this lane's queries come from the second block

  struct PairLd {
    i32x4 q[NINS], d[NINS];   // staged Q and dO rows
    float ld;           // lane < 32: lse of pair query lane; else D of pair query lane - 32
    int okA, okB;
  };
  // The query blocks of CSC_1[j] in batches of 64: lane i holds entry base + i as the byte
  // offset of its first Q/dO row (qtab) and of its first LSE/D value (ttab), kNoRow past the
  // batch or for an invalid id.  Pairs take them with v_readlane.
  uint32_t qtab = kNoRow, ttab = kNoRow;
  int cnt = 0;
  // Pair k of the batch (entries 2k, 2k+1).  Every call issues the same loads, also past the
  // batch end (kNoRow: zeros, no memory access), so waiting for a pair never drains the
  // prefetch queued behind it.
  auto load_pair = [&](int k) -> PairLd {
    PairLd f;
    const int idx = min(2 * k, 62);
    uint32_t bA = (uint32_t)__builtin_amdgcn_readlane((int)qtab, idx);
    uint32_t bB = (uint32_t)__builtin_amdgcn_readlane((int)qtab, idx + 1);
    uint32_t tA = (uint32_t)__builtin_amdgcn_readlane((int)ttab, idx);
    uint32_t tB = (uint32_t)__builtin_amdgcn_readlane((int)ttab, idx + 1);
    if (2 * k >= cnt) bA = tA = kNoRow;
    if (2 * k + 1 >= cnt) bB = tB = kNoRow;
    f.okA = bA != kNoRow;
    f.okB = bB != kNoRow;
    // lanes 0..31 read the LSE, lanes 32..63 D, in one load through a per-lane pointer (an
    // absent block reads its lane's query of block 0: its P is 0), issued before the rows.
    // One load into one register: two loads whose sum the compiler formed where it liked
    // made it wait for every load in flight there, the next pair's rows included.
    const uint32_t tl = (((lane >> 4) & 1) ? tB : tA);
    f.ld = *(const float*)((const char*)(lane < 32 ? lse_h : dd_h) + (tl == kNoRow ? 0u : tl) +
                           n * 4);
#pragma unroll
    for (int ins = 0; ins < NINS; ++ins) {
      const uint32_t o = (ins >= NINS / 2 ? bB : bA) + st_off[ins];
      f.q[ins] = __builtin_amdgcn_raw_buffer_load_b128(rq, o, 0, 0);
      f.d[ins] = __builtin_amdgcn_raw_buffer_load_b128(rdo, o, 0, 0);
    }
    return f;
  };

  f32x4 dka[D / 16], dva[D / 16];
#pragma unroll
  for (int t4 = 0; t4 < D / 16; ++t4) dka[t4] = dva[t4] = f32x4{0.f, 0.f, 0.f, 0.f};
  int ovc = 0, ovs = 0;   // the key block's overflow chunks (CSC pass)

  auto pair = [&](const PairLd& f) {
#pragma unroll
    for (int ins = 0; ins < NINS; ++ins) {
      *(i32x4*)(stQ + (ins * RPI + srow0) * kStride + 8 * piece) = f.q[ins];
      *(i32x4*)(stO + (ins * RPI + srow0) * kStride + 8 * piece) = f.d[ins];
    }
    stL[lane] = f.ld;
    wave_lds_sync();
    // S and dP tiles (queries x keys): lane (n, g) holds queries 8g + i + 4t, key n
    const float madd = (lane_second ? f.okB : f.okA) ? 0.f : -INFINITY;
    float p[2][4], dsv[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int arow = chunk_key(n, t);
      const f32x4 l4 = *(const f32x4*)(stL + 8 * g + 4 * t);
      const f32x4 d4 = *(const f32x4*)(stL + 32 + 8 * g + 4 * t);
      f32x4 st = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < D / 32; ++s) st = mfma_bf16_k32(lds_row8<D>(stQ, arow, s, g), kh[s], st);
#pragma unroll
      for (int s = 0; s < D / 32; ++s) dp = mfma_bf16_k32(lds_row8<D>(stO, arow, s, g), vh[s], dp);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = fast_exp2(fmaf(st[i], a.c2, madd - l4[i] * kLog2e));
        p[t][i] = pv;
        dsv[t][i] = pv * (dp[i] - d4[i]);
      }
    }
    bf16x8 p_hi, p_lo, ds_hi, ds_lo;
    split8(p, p_hi, p_lo);
    split8(dsv, ds_hi, ds_lo);
    // dV^T += dO^T P, dK^T += Q^T dS  (contract over the pair's 32 queries)
#pragma unroll
    for (int t4 = 0; t4 < D / 16; ++t4) {
      const bf16x8 ot = lds_tr8<D>(stO, t4, lane);
      const bf16x8 qt = lds_tr8<D>(stQ, t4, lane);
      dva[t4] = mfma_bf16_k32(ot, p_hi, dva[t4]);
      dva[t4] = mfma_bf16_k32(ot, p_lo, dva[t4]);
      dka[t4] = mfma_bf16_k32(qt, ds_hi, dka[t4]);
      dka[t4] = mfma_bf16_k32(qt, ds_lo, dka[t4]);
    }
    wave_lds_sync();
  };

  // ---- one batch of up to 64 query blocks (lane i: block p_lane of entry i), in pairs with
  // two load buffers used in turn
  auto batch = [&](int count, int p_lane) {
    cnt = count;
    qtab = ttab = kNoRow;
    if (lane < cnt && p_lane >= 0 && p_lane < n1) {
      qtab = (uint32_t)block_corner(p_lane, a.grid) * D * 2;
      ttab = (uint32_t)p_lane * kBlock * 4;
    }
    const int npairs = (cnt + 1) >> 1;
    PairLd fa = load_pair(0), fb;
    // whole pairs of pairs in the loop, an odd last pair after it (a break inside the loop
    // body gives the loop head a second entry whose wait counts drain every load in flight)
    int k = 0;
    for (; k + 1 < npairs; k += 2) {
      fb = load_pair(k + 1);
      pair(fa);
      fa = load_pair(k + 2);
      pair(fb);
    }
    if (k < npairs) {
      fb = load_pair(k + 1);
      pair(fa);
    }
  };
  if constexpr (!MASK) {
    // this wave's chunk of CSC_1[j]: entries [chunk, chunk + 1) * kKeyChunk
    const int32_t* off = a.csc_off[0] + (long)head * (n1 + 1);
    const int32_t* rows = a.csc_rows[0] + (long)head * n1 * a.fine_k;
    const int e0 = uniform(off[j] + chunk * kKeyChunk);
    const int e1 = uniform(min(off[j + 1], e0 + kKeyChunk));
    if constexpr (MODE == kKeyCsc) {
      // requested with the offsets, so that no wave ends on a round trip for them
      ovc = uniform(a.ov_count[(long)head * n1 + j]);
      ovs = uniform(a.ov_start[(long)head * n1 + j]);
    }
    int first_rows = -1;
    if constexpr (MODE == kKeyCsc) {
      // A third of the key blocks have no picks and need no key rows.  The others load them
      // as whole 128-byte lines (lane l: row l / 8 + 8 m, piece l % 8; the vector memory path
      // pays per line, and the B-operand layout would touch 16 half lines per load), request
      // the first batch's CSC rows before waiting for them, and rearrange them through the
      // still unused staging tiles into the B-operand layout (row n, channels 32 s + 8 g).
      if (e1 > e0) {
        i32x4 kl[D / 32], vl[D / 32];
        const uint32_t kbase = (uint32_t)block_corner(j, a.grid) * D * 2;
#pragma unroll
        for (int m = 0; m < D / 32; ++m) {
          const int r = lane / PPR + RPI * m;
          const uint32_t o =
              kbase + (uint32_t)tile_offset(r, a.grid) * D * 2 + 16 * (lane % PPR);
          kl[m] = __builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, 0);
          vl[m] = __builtin_amdgcn_raw_buffer_load_b128(rv, o, 0, 0);
        }
        first_rows = lane < min(64, e1 - e0) ? rows[e0 + lane] : -1;
#pragma unroll
        for (int m = 0; m < D / 32; ++m) {
          const int at = (lane / PPR + RPI * m) * kStride + 8 * (lane % PPR);
          *(i32x4*)(stQ + at) = kl[m];
          *(i32x4*)(stO + at) = vl[m];
        }
        wave_lds_sync();
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
          kh[s] = lds_row8<D>(stQ, n, s, g);
          vh[s] = lds_row8<D>(stO, n, s, g);
        }
        wave_lds_sync();
      }
    }
    for (int base = e0; base < e1; base += 64) {
      const int count = min(64, e1 - base);
      const int pl = MODE == kKeyCsc && base == e0 ? first_rows
                                                   : (lane < count ? rows[base + lane] : -1);
      batch(count, pl);
    }
  } else {
    // column j of the mask, 64 query blocks per step; hits are appended to pend in order and
    // run 64 at a time
    const uint8_t* col = a.mask + (long)head * n1 * n1 + j;
    int npend = 0;
    for (int scan = 0; scan < n1; scan += 64) {
      const int p = scan + lane;
      const bool hit = p < n1 && col[(long)p * n1] != 0;
      const uint64_t bal = __builtin_amdgcn_ballot_w64(hit);
      if (hit) pend[npend + __builtin_popcountll(bal & ((1ull << lane) - 1))] = p;
      npend += __builtin_popcountll(bal);
      if (npend >= 64) {
        wave_lds_sync();
        batch(64, pend[lane]);
        const int rest = npend - 64;
        const int moved = lane < rest ? pend[64 + lane] : 0;
        wave_lds_sync();
        if (lane < rest) pend[lane] = moved;
        npend = rest;
      }
    }
    if (npend > 0) {
      wave_lds_sync();
      batch(npend, lane < npend ? pend[lane] : -1);
    }
  }

  if constexpr (MODE == kKeyOverflow) {   // raw partial sums, lane-major
    float* dst = a.ov_part + (((long)head * a.ov_cap + ov_t) * 64 + lane) * (D / 2);
#pragma unroll
    for (int t4 = 0; t4 < D / 16; ++t4) {
      *(f32x4*)(dst + 4 * t4) = dka[t4];
      *(f32x4*)(dst + D / 4 + 4 * t4) = dva[t4];
    }
    // the chunk is written: one count for its key block (a release at device scope, after
    // every store of the wave)
    if (lane == 0)
      __hip_atomic_fetch_add(a.ov_done + (long)head * n1 + j, 1, __ATOMIC_RELEASE,
                             __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if constexpr (MODE == kKeyCsc) {   // the overflow chunks' partial sums, in chunk order
    if (ovc > 0) {
      // With 64 channels the overflow chunks run in this launch, ahead of the key blocks:
      // wait until all of this block's are written.  Only key blocks with overflow chunks wait,
      // a few per head, and the chunks' waves wait for nothing, so the wait ends; it is also
      // bounded (about 0.2 s) so that no fault elsewhere can turn it into a hang.
      // Polls are relaxed loads (an acquire at device scope invalidates this XCD's L2, which
      // the other waves' gathers live in); one acquire fence follows the last poll.
      const int32_t* done = a.ov_done + (long)head * n1 + j;
      for (int spin = 0; spin < (1 << 22); ++spin) {
        if (__hip_atomic_load(done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= ovc) break;
        __builtin_amdgcn_s_sleep(2);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    for (int m = 0; m < ovc; ++m) {
      const float* src = a.ov_part + (((long)head * a.ov_cap + ovs + m) * 64 + lane) * (D / 2);
#pragma unroll
      for (int t4 = 0; t4 < D / 16; ++t4) {
        dka[t4] += *(const f32x4*)(src + 4 * t4);
        dva[t4] += *(const f32x4*)(src + D / 4 + 4 * t4);
      }
    }
  }

  // ---- push-down of pooled-key gradients and store (lane holds key n, channels 16t4+4g+i)
#pragma unroll
  for (int h = 0; h < H; ++h) {
    pdown[lane + 64 * h] = pk_sum[h];
    pdown[D + lane + 64 * h] = pv_sum[h];
  }
  wave_lds_sync();
  bf16* dkp = a.dk + (tok_base + krow) * D;
  bf16* dvp = a.dv + (tok_base + krow) * D;
#pragma unroll
  for (int t4 = 0; t4 < D / 16; ++t4) {
    const f32x4 pk = *(const f32x4*)(pdown + 16 * t4 + 4 * g);
    const f32x4 pv = *(const f32x4*)(pdown + D + 16 * t4 + 4 * g);
    f32x4 rk4, rv4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rk4[i] = dka[t4][i] * a.scale + pk[i];
      rv4[i] = dva[t4][i] + pv[i];
    }
    *(bf16x4*)(dkp + 16 * t4 + 4 * g) = pack4_bf16(rk4);
    *(bf16x4*)(dvp + 16 * t4 + 4 * g) = pack4_bf16(rv4);
  }
}

// Two waves per SIMD (at most 256 registers): with 128 channels the compiler fits the CSC pass
// in 254 without spilling (it takes 264 unconstrained, one wave per SIMD; 500 -> 403 us per
// launch at 256x256 b2), while the overflow pass keeps one wave per SIMD (two would spill 17).
template <int MODE, int D>
__global__ __launch_bounds__(64)
__attribute__((amdgpu_waves_per_eu(D == 64 || MODE == kKeyCsc ? 2 : 1)))
void bwd_key_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 stQ[32 * bstride(D)];
  __shared__ __attribute__((aligned(16))) bf16 stO[32 * bstride(D)];   // dO rows
  __shared__ __attribute__((aligned(16))) float pdown[2 * D];          // pushed-down dK, dV
  __shared__ __attribute__((aligned(16))) float stL[64];            // lse (0..31), D (32..63)
  __shared__ int pend[MODE == kKeyMask ? 128 : 1];                  // mask hits not yet run
  const int kb = uniform(xcd_block(blockIdx.x, gridDim.x));
  if constexpr (MODE == kKeyOverflow) {
    const int head = uniform(kb / a.ov_waves);
    const int total = uniform(a.ov_total[head]);
    for (int t = uniform(kb - head * a.ov_waves); t < total; t += a.ov_waves) {
      const int packed = uniform(a.ov_table[(long)head * a.ov_cap + t]);
      key_block<MODE, D>(a, head, packed >> 16, packed & 0xffff, t, stQ, stO, pdown, stL,
                         pend);
    }
  } else {
    int kbi = kb;
    if constexpr (MODE == kKeyCsc && D == 64) {
      if ((int)blockIdx.x < a.ov_blocks) {   // leading workgroups: the overflow chunks
        const int ob = uniform(xcd_block(blockIdx.x, a.ov_blocks));
        const int head = uniform(ob / a.ov_waves);
        if (head >= a.bh) return;   // padding to a multiple of 8 workgroups
        const int total = uniform(a.ov_total[head]);
        for (int t = uniform(ob - head * a.ov_waves); t < total; t += a.ov_waves) {
          const int packed = uniform(a.ov_table[(long)head * a.ov_cap + t]);
          key_block<kKeyOverflow, D>(a, head, packed >> 16, packed & 0xffff, t, stQ, stO,
                                     pdown, stL, pend);
        }
        return;
      }
      // key blocks: numbered without the leading workgroups (a multiple of 8, so each XCD
      // keeps its contiguous range)
      kbi = uniform(xcd_block(blockIdx.x - a.ov_blocks, gridDim.x - a.ov_blocks));
    }
    const int n1 = a.n >> kBlockShift;
    const int head = uniform(kbi / n1);
    key_block<MODE, D>(a, head, uniform(kbi - head * n1), 0, 0, stQ, stO, pdown, stL, pend);
  }
}

// ====================================================================== host side
struct BwdLayout {
  size_t dd, part_k, part_v, dk_lv[kMaxLv], dv_lv[kMaxLv];
  size_t ov_start, ov_count, ov_table, ov_total, ov_done, ov_part;
  int ov_cap;
  size_t total;
};

// Overflow chunks per head never exceed (N/16) * fine_k / kKeyChunk: a block with c entries
// has floor((c - 1) / kKeyChunk) of them and the entries sum to (N/16) * fine_k.
static int key_overflow_cap(const Shape& s) {
  return std::max(1, (int)(((long)(s.n >> kBlockShift) * s.fine_k) / kKeyChunk));
}

static BwdLayout bwd_layout(const Shape& s) {
  BwdLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) & ~(size_t)255;
    return at;
  };
  L.dd = take(sizeof(float) * (size_t)s.bh * s.n);
  if (s.coarse_levels > 0) {
    const size_t n2 = (size_t)s.n >> (2 * kBlockShift);   // 256-token groups
    const size_t nc = (size_t)s.coarse_levels * s.topk;
    const size_t units = (size_t)q_units(s.d);
    L.part_k = take(sizeof(float) * s.bh * n2 * units * nc * s.d);
    L.part_v = take(sizeof(float) * s.bh * n2 * units * nc * s.d);
    for (int l = 2; l <= 1 + s.coarse_levels; ++l) {
      const size_t nl = (size_t)s.n_level(l);
      L.dk_lv[l - 1] = take(sizeof(float) * s.bh * nl * s.d);
      L.dv_lv[l - 1] = take(sizeof(float) * s.bh * nl * s.d);
    }
  }
  const size_t n1 = (size_t)s.n >> kBlockShift;
  L.ov_cap = key_overflow_cap(s);
  L.ov_start = take(sizeof(int32_t) * s.bh * n1);
  L.ov_count = take(sizeof(int32_t) * s.bh * n1);
  L.ov_table = take(sizeof(int32_t) * s.bh * (size_t)L.ov_cap);
  L.ov_total = take(sizeof(int32_t) * s.bh);
  L.ov_done = take(sizeof(int32_t) * s.bh * n1);
  L.ov_part = take(sizeof(float) * s.bh * (size_t)L.ov_cap * 64 * (s.d / 2));
  L.total = off;
  return L;
}

size_t bwd_workspace_bytes(const Shape& s) { return bwd_layout(s).total; }

hipError_t launch_attn_bwd(const Shape& s, const void* q, const void* k, const void* v,
                           const void* dout, const float* lse,
                           const float* const* k_lv, const float* const* v_lv,
                           const int32_t* const* sel, const int32_t* const* csc_off,
                           const int32_t* const* csc_rows, const uint8_t* mask, void* dq,
                           void* dk, void* dv, void* ws, hipStream_t stream) {
  const BwdLayout L = bwd_layout(s);
  char* base = (char*)ws;
  BwdArgs a{};
  a.q = (const bf16*)q;
  a.k = (const bf16*)k;
  a.v = (const bf16*)v;
  a.dout = (const bf16*)dout;
  a.lse = lse;
  for (int l = 0; l < s.levels; ++l) {
    a.k_lv[l] = k_lv ? k_lv[l] : nullptr;
    a.v_lv[l] = v_lv ? v_lv[l] : nullptr;
    a.sel[l] = sel[l];
    a.csc_off[l] = csc_off[l];
    a.csc_rows[l] = csc_rows[l];
  }
  a.dq = (bf16*)dq;
  a.dk = (bf16*)dk;
  a.dv = (bf16*)dv;
  a.dd = (float*)(base + L.dd);
  a.ov_start = (int32_t*)(base + L.ov_start);
  a.ov_count = (int32_t*)(base + L.ov_count);
  a.ov_table = (int32_t*)(base + L.ov_table);
  a.ov_total = (int32_t*)(base + L.ov_total);
  a.ov_done = (int32_t*)(base + L.ov_done);
  a.ov_part = (float*)(base + L.ov_part);
  a.ov_cap = L.ov_cap;
  const bool coarse = s.coarse_levels > 0;
  const int top = 1 + s.coarse_levels;   // the coarsest level with coarse keys
  if (coarse) {
    a.part_k = (float*)(base + L.part_k);
    a.part_v = (float*)(base + L.part_v);
    for (int l = 2; l <= top; ++l) {
      a.dk_lv[l - 1] = (float*)(base + L.dk_lv[l - 1]);
      a.dv_lv[l - 1] = (float*)(base + L.dv_lv[l - 1]);
    }
  }
  a.bh = s.bh;
  a.n = s.n;
  a.grid = Grid{s.hbits, s.wbits, s.raster};
  a.levels = s.levels;
  a.units_log2 = q_units(s.d) == 2 ? 1 : 2;
  a.topk = s.topk;
  a.fine_k = s.fine_k;
  a.bshift = s.bshift;
  a.enrich = coarse ? 1 : 0;
  a.coarse_levels = s.coarse_levels;
  a.lbias = s.coarse_lbias;
  a.exclude = s.exclude_overlap && coarse;
  a.scale = s.scale;
  a.c2 = s.scale * kLog2e;

  // the overflow plan of the key-major pass reads only the CSC_1 offsets: its workgroups lead
  // the query-major launch (a multiple of 8, so the XCD of every query unit is unchanged)
  static_assert(kQWaves == 4, "the plan runs on 256-thread workgroups");
  a.plan_blocks = mask ? 0 : (s.bh + 7) / 8 * 8;
  a.ov_waves = std::min(a.ov_cap, kOvWaves);
  const int n2 = s.n >> (2 * kBlockShift);
  const unsigned qblocks = (unsigned)(a.plan_blocks + s.bh * n2 * q_units(s.d));
  const int n_coarse = s.coarse_levels * s.topk;
  const size_t qlds = bwd_query_lds_bytes(s.d, n_coarse, s.exclude_overlap && coarse);
  const auto launch_query = [&](auto kernel) -> hipError_t {
    if (qlds > 65536) {
      const hipError_t e = hipFuncSetAttribute((const void*)kernel,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)qlds);
      if (e != hipSuccess) return e;
    }
    LLSA_LAUNCH("bwd_query_kernel", kernel, dim3(qblocks), dim3(64 * kQWaves), qlds, stream, a);
    return hipGetLastError();
  };
  const int nct = n_coarse == 0 ? 0 : n_coarse <= 16 ? 1 : 2;
  hipError_t err;
  if (s.d == 64)
    err = nct == 0 ? launch_query(bwd_query_kernel<0, 64>)
        : nct == 1 ? launch_query(bwd_query_kernel<1, 64>) : launch_query(bwd_query_kernel<2, 64>);
  else
    err = nct == 0 ? launch_query(bwd_query_kernel<0, 128>)
        : nct == 1 ? launch_query(bwd_query_kernel<1, 128>)
                   : launch_query(bwd_query_kernel<2, 128>);
  if (err != hipSuccess) return err;
  if (coarse) {
    CoarseGradArgs cg{};
    long blocks = 0;
    for (int l = 2; l <= top; ++l) {   // level 2: kCgWaves keys per workgroup
      cg.first_block[l - 1] = (int)blocks;
      const long keys = (long)s.bh * s.n_level(l);
      blocks += l == 2 ? (keys + kCgWaves - 1) / kCgWaves : keys;
    }
    for (int l = top; l <= kMaxLv; ++l) cg.first_block[l] = (int)blocks;
    if (s.d == 64)
      LLSA_LAUNCH("coarse_grad_kernel", coarse_grad_kernel<64>, dim3((unsigned)blocks),
                  dim3(64 * kCgWaves), 0, stream, a, cg);
    else
      LLSA_LAUNCH("coarse_grad_kernel", coarse_grad_kernel<128>, dim3((unsigned)blocks),
                  dim3(64 * kCgWaves), 0, stream, a, cg);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  const long kwaves = (long)s.bh * (s.n >> kBlockShift);
  const dim3 ovgrid((unsigned)((long)s.bh * a.ov_waves)), kgrid((unsigned)kwaves);
  if (mask) {   // the comparator: 64 channels only (checked by the caller)
    a.mask = mask;
    LLSA_LAUNCH("bwd_key_mask_kernel", (bwd_key_kernel<kKeyMask, 64>), kgrid, dim3(64), 0,
                stream, a);
  } else if (s.d == 64) {
    // the overflow chunks lead the key-major launch (no launch of their own)
    a.ov_blocks = (int)(((long)s.bh * a.ov_waves + 7) / 8 * 8);
    LLSA_LAUNCH("bwd_key_kernel", (bwd_key_kernel<kKeyCsc, 64>),
                dim3((unsigned)(a.ov_blocks + kwaves)), dim3(64), 0, stream, a);
  } else {
    LLSA_LAUNCH("bwd_key_overflow_kernel", (bwd_key_kernel<kKeyOverflow, 128>), ovgrid,
                dim3(64), 0, stream, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    LLSA_LAUNCH("bwd_key_kernel", (bwd_key_kernel<kKeyCsc, 128>), kgrid, dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

// ====================================================================== allocation-free entry
// The backward's workspace as a file-scope device array, for callers that cannot allocate.
// Each device the library runs on holds its own copy (for the life of the process); in host
// code `scratch` only names the symbol, so its device address is looked up once per device
// with hipGetSymbolAddress and kept.  Every call on a device uses that device's copy, and
// nothing in it has to start at zero (each launch writes what a later one reads), so calls
// that overlap on one device race and must be serialised by the caller.
static __device__ __align__(256) char scratch[LLSA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace llsa
