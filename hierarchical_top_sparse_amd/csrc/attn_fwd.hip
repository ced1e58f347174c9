// Sparse attention forward with hierarchical KV enrichment (paper summary sec. 四; article
// sec. 三/四: the forward gathers the selected key blocks directly, no dense mask).
//
// One wave owns one level-1 query block p (16 queries).  Its keys are processed in chunks of
// 32: first the 16 tokens of each pair of fine blocks in Sel_1[p], then the coarse keys
// Sel_l[p / 16^(l-1)] of levels l = 2..L (weight 16^l, i.e. a log2-domain bias of 4l).
//
// Orientation S^T = K Q^T: the MFMA result gives lane (n, g) the scores of query n against
// keys 8g..8g+7 of the chunk (two 16x16 tiles whose rows are interleaved so that this holds),
// so the online-softmax max needs two cross-lane steps and the exponentials already sit in
// the B-operand layout of O^T += V^T P^T.  V^T comes from the chunk's V rows staged row-major
// in LDS and read with ds_read_b64_tr_b16.  fp32 online softmax in the exp2 domain.
// Pooled (fp32) keys/values and the probabilities enter the bf16 MFMA as hi + lo pairs, so
// the only bf16 rounding is that of the inputs themselves.
// fp32 tensors use v_mfma_f32_16x16x4f32 with the same data flow.
// Workgroups are renumbered so that each XCD (and its L2) works on one contiguous spatial
// range of query blocks: neighbouring blocks select overlapping key blocks.
#include "common.hpp"
#include "kernels.hpp"

namespace llsa {

constexpr int kMaxLevels = 6;
constexpr int kFwdWaves = 4;
constexpr int kStageStrideBf16 = kDim + 8;   // 144-byte rows: 16-byte aligned, staggered banks
constexpr int kStageStrideF32 = kDim + 4;

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
  int topk;
  int enrich;
  float c2;   // scale * log2(e)
};

// Row of chunk position kk within S^T tile t: tile row r <-> kk = 8*(r/4) + r%4 + 4t.
__device__ __forceinline__ int tile_row_key(int r, int t) { return 8 * (r >> 2) + (r & 3) + 4 * t; }

__device__ __forceinline__ void split_bf16(f32x4 a, f32x4 b, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16 ha = (bf16)a[i], hb = (bf16)b[i];
    hi[i] = ha;
    hi[i + 4] = hb;
    lo[i] = (bf16)(a[i] - (float)ha);
    lo[i + 4] = (bf16)(b[i] - (float)hb);
  }
}

template <bool BF16>
__global__ __launch_bounds__(64 * kFwdWaves) void attn_fwd_kernel(FwdArgs a) {
  constexpr int kStride = BF16 ? kStageStrideBf16 : kStageStrideF32;
  typedef typename std::conditional<BF16, bf16, float>::type T;
  // [wave][hi/lo][32 rows]; the lo half is used by bf16 coarse chunks only
  __shared__ __attribute__((aligned(16))) T stage_all[kFwdWaves][BF16 ? 2 : 1][32 * kStride];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  T* stage = stage_all[w][0];
  T* stage_lo = stage_all[w][BF16 ? 1 : 0];
  const int n1 = a.n >> kBlockShift;
  const long qb = (long)xcd_block(blockIdx.x, gridDim.x) * kFwdWaves + w;
  if (qb >= (long)a.bh * n1) return;
  const int head = (int)(qb / n1);
  const int pb = (int)(qb - (long)head * n1);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int K = a.topk;
  const long tok_base = (long)head * a.n;

  // ---- queries: B operand of S^T
  const int qrow = token_row(pb * kBlock + n, a.grid);
  bf16x8 qh[2];
  f32x4 qf[4];
  if constexpr (BF16) {
    const bf16* qp = (const bf16*)a.q + (tok_base + qrow) * kDim;
    qh[0] = *(const bf16x8*)(qp + 8 * g);
    qh[1] = *(const bf16x8*)(qp + 32 + 8 * g);
  } else {
    const float* qp = (const float*)a.q + (tok_base + qrow) * kDim + 16 * g;
#pragma unroll
    for (int c = 0; c < 4; ++c) qf[c] = *(const f32x4*)(qp + 4 * c);
  }

  const int32_t* sel1 = a.sel[0] + ((long)head * n1 + pb) * K;
  const int n_fine_chunks = (K + 1) >> 1;
  const int n_coarse = a.enrich ? (a.levels - 1) * K : 0;
  const int n_chunks = n_fine_chunks + ((n_coarse + 31) >> 5);

  float m_run = -INFINITY;   // running max (log2 domain) of query n
  float l_run = 0.f;         // this lane's partial sum of exp2
  f32x4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int ch = 0; ch < n_chunks; ++ch) {
    const bool fine = ch < n_fine_chunks;
    // ---- per chunk: lane kk (< 32) resolves key kk: its row and level; validity as a mask
    int j0 = -1, j1 = -1;
    long my_row = 0;
    bool my_ok = false;
    if (fine) {
      j0 = sel1[2 * ch];
      j1 = (2 * ch + 1 < K) ? sel1[2 * ch + 1] : -1;
      const int kk = lane & 31;
      const int j = kk < 16 ? j0 : j1;
      my_ok = j >= 0 && j < n1;
      my_row = my_ok ? tok_base + token_row(j * kBlock + (kk & 15), a.grid) : 0;
    } else {
      const int slot = (ch - n_fine_chunks) * 32 + (lane & 31);
      if (slot < n_coarse) {
        const int l = 2 + slot / K;
        const int nl = a.n >> (kBlockShift * l);
        const int anc = pb >> (kBlockShift * (l - 1));
        const int id = a.sel[l - 1][((long)head * nl + anc) * K + (slot % K)];
        my_ok = id >= 0 && id < nl;
        my_row = my_ok ? (long)head * nl + id : 0;
      }
    }
    const uint64_t valid = __ballot(my_ok) & 0xffffffffull;
    auto row_of = [&](int kk) -> long { return __shfl(my_row, kk, 64); };
    // level of chunk position kk (coarse chunks): arithmetic on its slot, clamped to a level
    // that exists, so no cross-lane read is needed and a pointer index is always in range
    auto level_of = [&](int kk) -> int {
      const int slot = (ch - n_fine_chunks) * 32 + kk;
      const int l = 2 + (slot > 0 ? slot : 0) / K;
      return l < a.levels ? l : a.levels;
    };

    // ---- stage this chunk's V rows (row-major, 32 x 64) into LDS
#pragma unroll
    for (int ins = 0; ins < (BF16 ? 4 : 8); ++ins) {
      const int per_row = BF16 ? 8 : 16;                   // 16-byte pieces per row
      const int row = ins * (64 / per_row) + lane / per_row;
      const int piece = lane % per_row;
      const long r = row_of(row);
      const int lvl = level_of(row);
      const bool ok = (valid >> row) & 1;
      if constexpr (BF16) {
        if (fine) {
          bf16x8 val;
          if (ok) {
            val = *(const bf16x8*)((const bf16*)a.v + r * kDim + 8 * piece);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) val[e] = (bf16)0.f;
          }
          *(bf16x8*)(stage + row * kStride + 8 * piece) = val;
        } else {
          f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
          if (ok) {
            const float* vp = a.v_lv[lvl - 1] + r * kDim + 8 * piece;
            v0 = *(const f32x4*)vp;
            v1 = *(const f32x4*)(vp + 4);
          }
          bf16x8 hi, lo;
          split_bf16(v0, v1, hi, lo);
          *(bf16x8*)(stage + row * kStride + 8 * piece) = hi;
          *(bf16x8*)(stage_lo + row * kStride + 8 * piece) = lo;
        }
      } else {
        f32x4 val = {0.f, 0.f, 0.f, 0.f};
        if (ok) {
          const float* vp = (fine ? (const float*)a.v : a.v_lv[lvl - 1]) + r * kDim + 4 * piece;
          val = *(const f32x4*)vp;
        }
        *(f32x4*)(stage + row * kStride + 4 * piece) = val;
      }
    }

    // ---- S^T tiles and scores
    float sc[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int akk = tile_row_key(n, t);   // A-operand row owned by this lane
      const long r = row_of(akk);
      const int lvl = level_of(akk);
      const bool ok = (valid >> akk) & 1;
      f32x4 st = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BF16) {
        if (fine) {
          bf16x8 ka0, ka1;
          if (ok) {
            const bf16* kp = (const bf16*)a.k + r * kDim;
            ka0 = *(const bf16x8*)(kp + 8 * g);
            ka1 = *(const bf16x8*)(kp + 32 + 8 * g);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) ka0[e] = ka1[e] = (bf16)0.f;
          }
          st = mfma_bf16_k32(ka0, qh[0], st);
          st = mfma_bf16_k32(ka1, qh[1], st);
        } else {
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            f32x4 k0 = {0.f, 0.f, 0.f, 0.f}, k1 = {0.f, 0.f, 0.f, 0.f};
            if (ok) {
              const float* kp = a.k_lv[lvl - 1] + r * kDim + 32 * s + 8 * g;
              k0 = *(const f32x4*)kp;
              k1 = *(const f32x4*)(kp + 4);
            }
            bf16x8 hi, lo;
            split_bf16(k0, k1, hi, lo);
            st = mfma_bf16_k32(hi, qh[s], st);
            st = mfma_bf16_k32(lo, qh[s], st);
          }
        }
      } else {
        f32x4 kf[4];
        const float* kp = ok ? (fine ? (const float*)a.k : a.k_lv[lvl - 1]) + r * kDim + 16 * g
                             : nullptr;
#pragma unroll
        for (int c = 0; c < 4; ++c) kf[c] = kp ? *(const f32x4*)(kp + 4 * c) : f32x4{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) st = mfma_f32_k4(kf[c][e], qf[c][e], st);
      }
      // this lane's results: keys kk = 8g + i + 4t
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = 8 * g + i + 4 * t;
        const float bias = fine ? 0.f : 4.0f * (float)level_of(kk);   // log2(16^l)
        sc[t][i] = ((valid >> kk) & 1) ? st[i] * a.c2 + bias : -INFINITY;
      }
    }

    // ---- online softmax (log2 domain)
    float mloc = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, sc[t][i]);
    const float m_new = fmaxf(m_run, group4_max(mloc));
    const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - m_new);
    float p[2][4];
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[t][i] = (sc[t][i] == -INFINITY) ? 0.f : exp2f(sc[t][i] - m_new);
        psum += p[t][i];
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t4][i] *= alpha;

    wave_lds_sync();
    // ---- O^T += V^T P^T
    if constexpr (BF16) {
      bf16x8 p_hi, p_lo;
      split_bf16(f32x4{p[0][0], p[0][1], p[0][2], p[0][3]},
                 f32x4{p[1][0], p[1][1], p[1][2], p[1][3]}, p_hi, p_lo);
      const int r = (lane & 15) >> 2;
      const int c = lane & 3;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const int off = (8 * g + r) * kStride + 16 * t4 + 4 * c;
        const bf16x4 lo4 = lds_read_tr16(stage + off);
        const bf16x4 hi4 = lds_read_tr16(stage + off + 4 * kStride);
        bf16x8 vt;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vt[e] = lo4[e];
          vt[e + 4] = hi4[e];
        }
        acc[t4] = mfma_bf16_k32(vt, p_hi, acc[t4]);
        acc[t4] = mfma_bf16_k32(vt, p_lo, acc[t4]);
        if (!fine) {
          const bf16x4 a4 = lds_read_tr16(stage_lo + off);
          const bf16x4 b4 = lds_read_tr16(stage_lo + off + 4 * kStride);
          bf16x8 vl;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            vl[e] = a4[e];
            vl[e + 4] = b4[e];
          }
          acc[t4] = mfma_bf16_k32(vl, p_hi, acc[t4]);
        }
      }
    } else {
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float vv = stage[(8 * g + i + 4 * t) * kStride + 16 * t4 + n];
            acc[t4] = mfma_f32_k4(vv, p[t][i], acc[t4]);
          }
    }
    wave_lds_sync();
  }

  // ---- finalize
  const float l_tot = group4_sum(l_run);
  const float inv = 1.0f / l_tot;
  if constexpr (BF16) {
    bf16* op = (bf16*)a.o + (tok_base + qrow) * kDim;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      bf16x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = (bf16)(acc[t4][i] * inv);
      *(bf16x4*)(op + 16 * t4 + 4 * g) = r;
    }
  } else {
    float* op = (float*)a.o + (tok_base + qrow) * kDim;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      f32x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = acc[t4][i] * inv;
      *(f32x4*)(op + 16 * t4 + 4 * g) = r;
    }
  }
  if (g == 0) a.lse[tok_base + pb * kBlock + n] = (m_run + log2f(l_tot)) * kLn2;
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
  a.enrich = s.enrich;
  a.c2 = s.scale * kLog2e;
  const long waves = (long)s.bh * (s.n >> kBlockShift);
  const unsigned blocks = (unsigned)((waves + kFwdWaves - 1) / kFwdWaves);
  if (s.bf16)
    hipLaunchKernelGGL(attn_fwd_kernel<true>, dim3(blocks), dim3(64 * kFwdWaves), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<false>, dim3(blocks), dim3(64 * kFwdWaves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace llsa
