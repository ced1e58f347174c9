// Sparse attention forward with hierarchical KV enrichment (paper summary sec. 四; article
// sec. 三/四: the forward gathers the selected key blocks directly, no dense mask).
//
// One workgroup owns one level-2 group (the 16 level-1 query blocks of a 16x16-pixel tile,
// which share their ancestors and so their coarse keys), or half of one when K > 16; each of
// its 4 waves owns QB consecutive query blocks (QB = 4, or 2 when K > 16, so that the wave's
// QB K picks fit its 64 lanes) and works on its own, without workgroup barriers:
//  1. its QB K picks are ranked in LDS (keys (id, owner)) into the ascending list U of distinct
//     key blocks, with a QB-bit mask per entry of the blocks that picked it.  Neighbouring
//     query blocks choose among the same candidates, so U is much shorter than QB K;
//  2. the wave streams U: each key block's 16 K rows and 16 V rows are loaded row-major (each
//     4-lane quad reads 64 contiguous bytes: the vector memory pipeline charges a quad per
//     distinct cache line, so MFMA-operand-shaped loads cost 4x as much), two blocks ahead of
//     use in registers, and staged in the wave's LDS tile;
//  3. for every block of U, each of the wave's query blocks that picked it gets one 16 x 16
//     tile: S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (lane (n, g): scores of query n against
//     keys 4g..4g+3, the B-operand layout of the next product), online softmax, and
//     O^T += V^T P^T on v_mfma_f32_16x16x16_bf16 with V^T read by ds_read_b64_tr_b16;
//  4. the coarse keys Sel_l[ancestor], l = 2..L, staged once per workgroup in LDS (fp32 pooled
//     values as bf16 hi + lo parts, weight 16^l as the log2-domain bias 4l), then O and LSE.
//     Each wave stages a share of them before its stream and counts it in LDS; a wave waits for
//     the count only when it reads them, so no wave waits for the slowest one's staging.
// fp32 tensors use v_mfma_f32_16x16x4f32 with the same data flow.  Workgroups are renumbered
// so that each XCD (and its L2) works on one contiguous spatial range of level-2 groups.
// D (head_dim) is 64 or 128 (bf16 only): rows, MFMA contraction chains and accumulators scale
// with it; with 128 channels a wave owns 2 query blocks (its accumulators double).
#include "common.hpp"
#include "kernels.hpp"

namespace llsa {

constexpr int kMaxLevels = 6;
constexpr int kFwdWaves = 4;
// LDS row strides: D + 8 bf16 (144 bytes for 64 channels: 16-byte aligned, staggered banks),
// D + 4 floats
__host__ __device__ constexpr int stride_bf16(int D) { return D + 8; }
__host__ __device__ constexpr int stride_f32(int D) { return D + 4; }
constexpr float kMinusBig = -1e30f;     // running-max floor: keeps exp2 arguments finite

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* k_lv[kMaxLevels];
  const float* v_lv[kMaxLevels];
  const int32_t* sel[kMaxLevels];
  void* o;
  float* lse;
  int bh;
  int n;
  Grid grid;
  int levels;
  int topk;            // K: coarse keys per level
  int fine_k;          // picks per 16-token query block (rows of sel[0]): K B / 16
  int bshift;          // log2(B) of the coarse levels: 4 or 6
  int coarse_levels;   // coarse keys of levels 2 .. 1 + coarse_levels
  float lbias;         // log2-domain bias per level: log2(B) (weight B^l) or 0 (weight 1)
  int exclude;         // 1: a coarse key over a key selected one level finer is dropped
  float c2;            // scale * log2(e)
};

__device__ __forceinline__ void split_bf16(f32x4 a, f32x4 b, bf16x8& hi, bf16x8& lo) {
  split8_bf16(a, b, hi, lo);
}

constexpr int kWavePicks = 64;     // QB query blocks x K (QB K <= 64)
constexpr int kSentinel = 0x7f000000;

template <bool BF16, int D>
struct FwdCfg {
  static constexpr int ES = BF16 ? 2 : 4;               // element bytes
  static constexpr int kStride = BF16 ? stride_bf16(D) : stride_f32(D);
  static constexpr int kRowBytes = D * ES;
  static constexpr int PPR = kRowBytes / 16;            // 16-byte pieces per row
  static constexpr int kTile = 16 * kStride;            // one 16-row tile (elements)
  static constexpr int NB = BF16 ? 4 : 2;               // coarse buffers: K(hi,lo), V(hi,lo)
  static constexpr int kBlockPieces = 16 * PPR;         // pieces of one block's rows per tensor
  static constexpr int kLoads = kBlockPieces / 64;      // row-major loads per lane per tensor
};

// Dynamic LDS: per wave a K/V tile pair and its pick lists; per workgroup the coarse tiles
// [ctiles][NB][16][stride] and their biases.
__host__ __device__ constexpr int fwd_wave_lds_bytes(bool bf16, int D) {
  return 2 * 16 * (bf16 ? stride_bf16(D) * 2 : stride_f32(D) * 4) +
         (int)sizeof(int) * 4 * kWavePicks;
}
// ... then each slot's bias and key id, with overlap exclusion per-block biases
// [waves][4 blocks][ctiles * 16], and the count of waves that have staged their share.
static size_t fwd_lds_bytes(bool bf16, int D, int n_coarse, bool exclude) {
  const int es = bf16 ? 2 : 4;
  const int stride = bf16 ? stride_bf16(D) : stride_f32(D);
  const int nb = bf16 ? 4 : 2;
  const int ctiles = (n_coarse + 15) / 16;
  return kFwdWaves * fwd_wave_lds_bytes(bf16, D) + (size_t)ctiles * nb * 16 * stride * es +
         (sizeof(float) + sizeof(int)) * 16 * ctiles +
         (exclude ? sizeof(float) * kFwdWaves * 4 * 16 * ctiles : 0) + 16;
}

// QB: query blocks per wave (4, or 2 for K > 16 or 128 channels); D: head_dim
template <bool BF16, int QB, int D>
__global__ __launch_bounds__(64 * kFwdWaves)
__attribute__((amdgpu_waves_per_eu(BF16 && D == 64 ? 3 : 2))) void attn_fwd_kernel(FwdArgs a) {
  constexpr int PS = kWavePicks / QB;                     // pick slots per query block
  constexpr int kUnitsPerGroup = kBlock / (kFwdWaves * QB);   // workgroups per level-2 group
  static_assert(BF16 || D == 64, "fp32 tokens: 64 channels");
  using C = FwdCfg<BF16, D>;
  typedef typename std::conditional<BF16, bf16, float>::type T;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int n1 = a.n >> kBlockShift;
  const int n2 = n1 >> kBlockShift;
  const int wg = uniform(xcd_block(blockIdx.x, gridDim.x));
  const int head = uniform(wg / (kUnitsPerGroup * n2));   // scalar: buffer descriptors must
  const int rem = uniform(wg - head * kUnitsPerGroup * n2);   // be wave-uniform
  const int a2 = rem / kUnitsPerGroup;
  const int K = a.topk;
  const int KF = a.fine_k;
  const long tok_base = (long)head * a.n;
  const int n_coarse = a.coarse_levels * K;
  const int ctiles = (n_coarse + 15) >> 4;

  char* wbase = smem + w * fwd_wave_lds_bytes(BF16, D);
  T* kt = (T*)wbase;                          // the staged key block: K rows, then V rows
  T* vt = kt + C::kTile;
  int* keys = (int*)(vt + C::kTile);          // [64] pick keys (id << 8 | index)
  int* sorted = keys + kWavePicks;            // [64] ascending
  int* uoff = sorted + kWavePicks;            // [64] first-row byte offset of U[u]
  int* umask = uoff + kWavePicks;             // [64] blocks of the wave that picked U[u]
  T* ctile = (T*)(smem + kFwdWaves * fwd_wave_lds_bytes(BF16, D));
  float* cbias = (float*)(ctile + ctiles * C::NB * C::kTile);
  int* cid = (int*)(cbias + 16 * ctiles);       // key id of each coarse slot (-1: none)
  float* xbias = (float*)(cid + 16 * ctiles);   // with exclusion: [w][bb][slot] biases
  int* staged = (int*)(xbias + (a.exclude ? kFwdWaves * 4 * 16 * ctiles : 0));
  if (tid == 0) *staged = 0;
  __syncthreads();   // the count is zero (the waves start together, so this costs little)

  const uint32_t head_bytes = (uint32_t)a.n * C::kRowBytes;
  const rsrc_t rq = make_rsrc_uniform((const char*)a.q + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rk = make_rsrc_uniform((const char*)a.k + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rv = make_rsrc_uniform((const char*)a.v + (size_t)head * head_bytes, head_bytes);
  // the wave's first query block
  const int pb_first = a2 * kBlock + (rem % kUnitsPerGroup) * (kFwdWaves * QB) + QB * w;

  // ---- the wave's picks (lane PS b + i: pick i of block b) and its query operands
  int key = kSentinel | lane;   // sentinels sort after every pick and stay distinct
  if ((lane % PS) < KF) {
    const int j = a.sel[0][((long)head * n1 + pb_first + lane / PS) * KF + (lane % PS)];
    if (j >= 0 && j < n1) key = (j << 8) | lane;
  }
  // B operand of S^T for block bb: lane (n, g) holds query row n, channels 32s + 8g .. +7
  // (bf16) or 16g + 4c .. +3 (fp32)
  bf16x8 qh[QB][D / 32];
  f32x4 qf[QB][D / 16];
#pragma unroll
  for (int bb = 0; bb < QB; ++bb) {
    const uint32_t qrow =
        (uint32_t)(block_corner(pb_first + bb, a.grid) + tile_offset(n, a.grid)) * C::kRowBytes;
    if constexpr (BF16) {
#pragma unroll
      for (int s2 = 0; s2 < D / 32; ++s2)
        qh[bb][s2] = buf_load8(rq, qrow + (32 * s2 + 8 * g) * 2);
    } else {
#pragma unroll
      for (int c = 0; c < D / 16; ++c) qf[bb][c] = buf_load4f(rq, qrow + (16 * g + 4 * c) * 4);
    }
  }

  // ---- coarse keys of the group (slot e / (D/8) of 16 ctiles, channels 8 (e % (D/8)) ..
  // +7): fp32 pooled values as bf16 hi + lo parts (fp32 tensors: as they are) and the bias.
  // First each item's key id and bias (their loads overlap the ranking of the picks below),
  // then, beside the first key blocks' loads, the rows themselves.
  const int pb0 = a2 * kBlock;
  constexpr int kCItems = (2 * 16 * (D / 8) + 64 * kFwdWaves - 1) / (64 * kFwdWaves);
  const int citems = ctiles * 16 * (D / 8);
  int cit_id[kCItems];
  float cit_bias[kCItems];
#pragma unroll
  for (int it = 0; it < kCItems; ++it) {
    const int e = tid + 64 * kFwdWaves * it;
    const int cslot = e / (D / 8), c8 = (e % (D / 8)) * 8;
    cit_id[it] = -1;
    cit_bias[it] = -INFINITY;
    if (e < citems && cslot < n_coarse) {
      const int l = 2 + cslot / K;
      const int nl = a.n >> (a.bshift * l);
      const int anc = (pb0 << kBlockShift) >> (a.bshift * l);   // the group's level-l ancestor
      const int id = a.sel[l - 1][((long)head * nl + anc) * K + (cslot - (l - 2) * K)];
      if (id >= 0 && id < nl) {
        cit_id[it] = id;
        cit_bias[it] = a.lbias * (float)l;   // log2(B^l), or 0 for unit weights
        if (a.exclude && l >= 3 && c8 == 0) {
          // level >= 3: dropped for the whole group if it is the parent of one of the keys
          // selected at level l - 1 for the group's level-(l-1) ancestor
          const int nf = a.n >> (a.bshift * (l - 1));
          const int ancf = (pb0 << kBlockShift) >> (a.bshift * (l - 1));
          for (int i = 0; i < K; ++i)
            if ((a.sel[l - 2][((long)head * nf + ancf) * K + i] >> a.bshift) == id)
              cit_bias[it] = -INFINITY;
        }
      }
    }
  }

  // ---- U: rank of each pick key among the wave's 64, distinct ids, owner masks
  keys[lane] = key;
  umask[lane] = 0;
  wave_lds_sync();
  {
    int r = 0;
#pragma unroll 4
    for (int u = 0; u < kWavePicks; u += 4) {
      const i32x4 kk = *(const i32x4*)(keys + u);
#pragma unroll
      for (int e = 0; e < 4; ++e) r += kk[e] < key ? 1 : 0;
    }
    sorted[r] = key;
  }
  wave_lds_sync();
  const int sk = sorted[lane];
  const bool valid = sk < kSentinel;
  const int prev = sorted[lane > 0 ? lane - 1 : 0];
  const bool first = valid && (lane == 0 || (prev >> 8) != (sk >> 8));
  const uint64_t fm = __builtin_amdgcn_ballot_w64(first);
  const int n_u = uniform(__builtin_popcountll(fm));
  {
    const int u = __builtin_popcountll(fm & (~0ull >> (63 - lane))) - 1;
    if (first) {   // the run of this key block: one entry per block that picked it
      int m = 0;
      for (int r = lane; r < min(lane + QB, kWavePicks); ++r) {
        const int o = sorted[r];
        if ((o >> 8) != (sk >> 8)) break;
        m |= 1 << ((o & 63) / PS);
      }
      uoff[u] = block_corner(sk >> 8, a.grid) * C::kRowBytes;
      umask[u] = m;
    }
  }
  wave_lds_sync();

  // ---- the stream of U: row-major loads (lane l: pieces l + 64 m of the block's 16 rows),
  // two blocks ahead of use; past the end kNoRow (zeros, no memory access)
  uint32_t piece_off[C::kLoads];
#pragma unroll
  for (int m = 0; m < C::kLoads; ++m) {
    const int e = lane + 64 * m;
    piece_off[m] = (uint32_t)tile_offset(e / C::PPR, a.grid) * C::kRowBytes + 16 * (e % C::PPR);
  }
  struct BlockLd {
    i32x4 k[C::kLoads], v[C::kLoads];
  };
  auto load_u = [&](int u) -> BlockLd {
    BlockLd f;
    const uint32_t b = u < n_u ? (uint32_t)uniform(uoff[min(u, kWavePicks - 1)]) : kNoRow;
#pragma unroll
    for (int m = 0; m < C::kLoads; ++m) {
      f.k[m] = __builtin_amdgcn_raw_buffer_load_b128(rk, b + piece_off[m], 0, 0);
      f.v[m] = __builtin_amdgcn_raw_buffer_load_b128(rv, b + piece_off[m], 0, 0);
    }
    return f;
  };
  // the coarse rows (loaded before the first key blocks, so they are waited for first)
  f32x4 ck[kCItems][2], cv[kCItems][2];
#pragma unroll
  for (int it = 0; it < kCItems; ++it) {
    const int e = tid + 64 * kFwdWaves * it;
    const int cslot = e / (D / 8), c8 = (e % (D / 8)) * 8;
    ck[it][0] = ck[it][1] = cv[it][0] = cv[it][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (e < citems && cit_id[it] >= 0) {
      const int l = 2 + cslot / K;
      const int nl = a.n >> (a.bshift * l);
      const float* kp = a.k_lv[l - 1] + ((long)head * nl + cit_id[it]) * D + c8;
      const float* vp = a.v_lv[l - 1] + ((long)head * nl + cit_id[it]) * D + c8;
      ck[it][0] = *(const f32x4*)kp;
      ck[it][1] = *(const f32x4*)(kp + 4);
      cv[it][0] = *(const f32x4*)vp;
      cv[it][1] = *(const f32x4*)(vp + 4);
    }
  }
  BlockLd fa = load_u(0), fb = load_u(1);
#pragma unroll
  for (int it = 0; it < kCItems; ++it) {
    const int e = tid + 64 * kFwdWaves * it;
    if (e >= citems) continue;
    const int cslot = e / (D / 8), c8 = (e % (D / 8)) * 8;
    T* base = ctile + (cslot >> 4) * C::NB * C::kTile + (cslot & 15) * C::kStride + c8;
    if constexpr (BF16) {
      bf16x8 hi, lo;
      split_bf16(ck[it][0], ck[it][1], hi, lo);
      *(bf16x8*)base = hi;
      *(bf16x8*)(base + C::kTile) = lo;
      split_bf16(cv[it][0], cv[it][1], hi, lo);
      *(bf16x8*)(base + 2 * C::kTile) = hi;
      *(bf16x8*)(base + 3 * C::kTile) = lo;
    } else {
      *(f32x4*)base = ck[it][0];
      *(f32x4*)(base + 4) = ck[it][1];
      *(f32x4*)(base + C::kTile) = cv[it][0];
      *(f32x4*)(base + C::kTile + 4) = cv[it][1];
    }
    if (c8 == 0) {
      cbias[cslot] = cit_bias[it];
      cid[cslot] = cit_id[it];
    }
  }
  // This wave's share of the coarse tiles is staged.  The tiles are read only after the wave's
  // stream (or by the exclusion biases below), so a wave counts its share and goes on instead
  // of waiting at a barrier for the slowest one; a reader waits for the count.  The waves of a
  // workgroup are resident together and stage without waiting for anything, so the wait ends.
  if (lane == 0) __hip_atomic_fetch_add(staged, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  auto wait_staged = [&]() {
    while (__hip_atomic_load(staged, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < kFwdWaves)
      __builtin_amdgcn_s_sleep(1);
  };

  // with overlap exclusion, per-block biases: a level-2 slot is dropped for block bb if one of
  // bb's fine picks lies in its span (the 16-token block j is in key (16 j) >> 2 log2(B))
  const int cslots = 16 * ctiles;
  float* wxb = xbias + w * QB * cslots;
  if (a.exclude) {
    wait_staged();
    for (int sl = lane; sl < cslots; sl += 64) {
      const int id = cid[sl];
      const bool lv2 = sl < K && id >= 0;
#pragma unroll
      for (int bb = 0; bb < QB; ++bb) {
        bool hit = false;
        if (lv2)
          for (int i = 0; i < KF; ++i) {
            const int kk = keys[PS * bb + i];
            hit |= kk < kSentinel && (((kk >> 8) << kBlockShift) >> (2 * a.bshift)) == id;
          }
        wxb[bb * cslots + sl] = hit ? -INFINITY : cbias[sl];
      }
    }
    wave_lds_sync();
  }

  float m_run[QB], l_run[QB];   // running max (log2 domain) and this lane's partial sums
  f32x4 acc[QB][D / 16];        // O^T of each block: lane (n, g) holds d = 16 t4 + 4g + i
#pragma unroll
  for (int bb = 0; bb < QB; ++bb) {
    m_run[bb] = kMinusBig;
    l_run[bb] = 0.f;
#pragma unroll
    for (int t4 = 0; t4 < D / 16; ++t4) acc[bb][t4] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One 16-key tile for block bb: scores x = st * c2 + bias (log2 domain), online softmax,
  // O^T += V^T P^T.  The running max moves only when some score exceeds it by more than
  // 2^kLazy (a wave vote): below that exp2(x - m_run) <= 2^kLazy is exact in fp32 and within
  // bf16's range, and O = acc / l is unchanged, so most tiles skip the cross-lane max and the
  // rescaling.  ktl/vtl: K and V rows (16 x stride); klo/vlo: their lo parts (coarse keys).
  constexpr float kLazy = 8.f;
  auto tile = [&](auto bbc, const T* ktl, const T* klo, const T* vtl, const T* vlo,
                  const float* kbias) {
    constexpr int bb = decltype(bbc)::value;
    f32x4 st = {0.f, 0.f, 0.f, 0.f};
    if constexpr (BF16) {
#pragma unroll
      for (int s2 = 0; s2 < D / 32; ++s2) {
        st = mfma_bf16_k32(*(const bf16x8*)(ktl + n * C::kStride + 32 * s2 + 8 * g), qh[bb][s2],
                           st);
        if (klo)
          st = mfma_bf16_k32(*(const bf16x8*)(klo + n * C::kStride + 32 * s2 + 8 * g),
                             qh[bb][s2], st);
      }
    } else {
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const f32x4 kf = *(const f32x4*)(ktl + n * C::kStride + 16 * g + 4 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) st = mfma_f32_k4(kf[e], qf[bb][c][e], st);
      }
    }
    float x[4];
    if (kbias) {
      const f32x4 b4 = *(const f32x4*)(kbias + 4 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = fmaf(st[i], a.c2, b4[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = st[i] * a.c2;
    }
    const float mloc = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    if (__builtin_amdgcn_ballot_w64(mloc > m_run[bb] + kLazy)) {   // wave-uniform
      const float m_new = fmaxf(m_run[bb], group4_max(mloc));
      const float alpha = fast_exp2(m_run[bb] - m_new);
      l_run[bb] *= alpha;
#pragma unroll
      for (int t4 = 0; t4 < D / 16; ++t4)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[bb][t4][i] *= alpha;
      m_run[bb] = m_new;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = fast_exp2(x[i] - m_run[bb]);
      l_run[bb] += p[i];
    }
    if constexpr (BF16) {
      const bf16x4 pb = pack4_bf16(p[0], p[1], p[2], p[3]);
      const int r = (lane & 15) >> 2;
      const int c = lane & 3;
#pragma unroll
      for (int t4 = 0; t4 < D / 16; ++t4) {
        const int off = (4 * g + r) * C::kStride + 16 * t4 + 4 * c;
        if (vlo)
          acc[bb][t4] = mfma_bf16_k16x2(lds_read_tr16(vtl + off), pb, lds_read_tr16(vlo + off),
                                        pb, acc[bb][t4]);
        else
          acc[bb][t4] = mfma_bf16_k16(lds_read_tr16(vtl + off), pb, acc[bb][t4]);
      }
    } else {
#pragma unroll
      for (int t4 = 0; t4 < D / 16; ++t4)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[bb][t4] =
              mfma_f32_k4(vtl[(4 * g + i) * C::kStride + 16 * t4 + n], p[i], acc[bb][t4]);
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  auto for_blocks = [&](auto&& fn) {
    fn(I0{});
    fn(I1{});
    if constexpr (QB > 2) {
      fn(I2{});
      fn(I3{});
    }
  };

  // one block of U: its rows from their loads to the wave's LDS tile (after which the load
  // registers take the block two ahead, so that two blocks stay in flight while this one is
  // computed), then the tiles of the blocks that picked it
  auto stage_u = [&](const BlockLd& f) {
#pragma unroll
    for (int m = 0; m < C::kLoads; ++m) {
      const int e = lane + 64 * m;
      const int at = (e / C::PPR) * C::kStride + (e % C::PPR) * (16 / C::ES);
      *(i32x4*)(kt + at) = f.k[m];
      *(i32x4*)(vt + at) = f.v[m];
    }
  };
  auto compute_u = [&](int u) {
    wave_lds_sync();
    const int mask = uniform(umask[u]);
    for_blocks([&](auto bbc) {
      if (mask & (1 << decltype(bbc)::value)) tile(bbc, kt, nullptr, vt, nullptr, nullptr);
    });
    wave_lds_sync();
  };
  // Whole pairs in the loop and an odd last block after it: with a break inside the loop
  // body, one path into the loop head has only the first block's loads in flight, and the
  // head then waits for every load (the next block's too) instead of the first block's.
  int u = 0;
  for (; u + 1 < n_u; u += 2) {
    stage_u(fa);
    fa = load_u(u + 2);
    compute_u(u);
    stage_u(fb);
    fb = load_u(u + 3);
    compute_u(u + 1);
  }
  if (u < n_u) {
    stage_u(fa);
    compute_u(u);
  }

  // ---- coarse keys, then O and the LSE of each block
  wait_staged();
  for (int ct = 0; ct < ctiles; ++ct) {
    const T* cb0 = ctile + ct * C::NB * C::kTile;
    for_blocks([&](auto bbc) {
      constexpr int bb = decltype(bbc)::value;
      const float* cb = (a.exclude ? wxb + bb * cslots : cbias) + 16 * ct;
      if constexpr (BF16)
        tile(bbc, cb0, cb0 + C::kTile, cb0 + 2 * C::kTile, cb0 + 3 * C::kTile, cb);
      else
        tile(bbc, cb0, nullptr, cb0 + C::kTile, nullptr, cb);
    });
  }
  for_blocks([&](auto bbc) {
    constexpr int bb = decltype(bbc)::value;
    const int pb = pb_first + bb;
    const int qrow = block_corner(pb, a.grid) + tile_offset(n, a.grid);
    const float l_tot = group4_sum(l_run[bb]);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;   // 0 only if every key was skipped
    if constexpr (BF16) {
      bf16* op = (bf16*)a.o + (tok_base + qrow) * D;
#pragma unroll
      for (int t4 = 0; t4 < D / 16; ++t4) {
        f32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = acc[bb][t4][i] * inv;
        *(bf16x4*)(op + 16 * t4 + 4 * g) = pack4_bf16(r);
      }
    } else {
      float* op = (float*)a.o + (tok_base + qrow) * D;
#pragma unroll
      for (int t4 = 0; t4 < D / 16; ++t4) {
        f32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = acc[bb][t4][i] * inv;
        *(f32x4*)(op + 16 * t4 + 4 * g) = r;
      }
    }
    if (g == 0) a.lse[tok_base + pb * kBlock + n] = (m_run[bb] + log2f(l_tot)) * kLn2;
  });
}

hipError_t launch_attn_fwd(const Shape& s, const void* q, const void* k, const void* v,
                           const float* const* k_lv, const float* const* v_lv,
                           const int32_t* const* sel, void* o, float* lse, hipStream_t stream) {
  FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  for (int l = 0; l < s.levels; ++l) {
    a.k_lv[l] = k_lv ? k_lv[l] : nullptr;
    a.v_lv[l] = v_lv ? v_lv[l] : nullptr;
    a.sel[l] = sel[l];
  }
  a.o = o;
  a.lse = lse;
  a.bh = s.bh;
  a.n = s.n;
  a.grid = Grid{s.hbits, s.wbits, s.raster};
  a.levels = s.levels;
  a.topk = s.topk;
  a.fine_k = s.fine_k;
  a.bshift = s.bshift;
  a.coarse_levels = s.coarse_levels;
  a.lbias = s.coarse_lbias;
  a.exclude = s.exclude_overlap && s.coarse_levels > 0;
  a.c2 = s.scale * kLog2e;
  const int n_coarse = s.coarse_levels * s.topk;
  const size_t lds = fwd_lds_bytes(s.bf16, s.d, n_coarse, s.exclude_overlap != 0);
  // one workgroup per level-2 group (N is a multiple of 16^2), two when a wave owns 2 query
  // blocks (K > 16, so that its 2 K picks fit 64 lanes; or 128 channels)
  const bool wide = s.fine_k > kWavePicks / 4 || s.d == 128;
  const unsigned blocks = (unsigned)((long)s.bh * (s.n >> (2 * kBlockShift)) * (wide ? 2 : 1));
  const dim3 grid(blocks), block(64 * kFwdWaves);
  const auto launch = [&](auto kernel) -> hipError_t {
    if (lds > 65536) {
      const hipError_t e = hipFuncSetAttribute((const void*)kernel,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)lds);
      if (e != hipSuccess) return e;
    }
    LLSA_LAUNCH("attn_fwd_kernel", kernel, grid, block, lds, stream, a);
    return hipGetLastError();
  };
  if (s.d == 128) return launch(attn_fwd_kernel<true, 2, 128>);   // bf16 only (checked)
  if (s.bf16)
    return wide ? launch(attn_fwd_kernel<true, 2, 64>) : launch(attn_fwd_kernel<true, 4, 64>);
  return wide ? launch(attn_fwd_kernel<false, 2, 64>) : launch(attn_fwd_kernel<false, 4, 64>);
}

}  // namespace llsa
