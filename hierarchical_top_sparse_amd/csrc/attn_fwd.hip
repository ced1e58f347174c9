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
// fp32 tensors use v_mfma_f32_16x16x4f32 with the same data flow.
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

// Source of key kk (0..31) of a chunk.
struct KeySrc {
  long row;     // row index into the token tensor or the level array (head offset included)
  int level;    // 0: fine token, l >= 2: pooled level l
  bool valid;
};

// Row of chunk position kk within S^T tile t: tile row r <-> kk = 8*(r/4) + r%4 + 4t.
__device__ __forceinline__ int tile_row_key(int r, int t) { return 8 * (r >> 2) + (r & 3) + 4 * t; }

template <bool BF16>
__global__ __launch_bounds__(64 * kFwdWaves) void attn_fwd_kernel(FwdArgs a) {
  constexpr int kStride = BF16 ? kStageStrideBf16 : kStageStrideF32;
  typedef typename std::conditional<BF16, bf16, float>::type T;
  __shared__ __attribute__((aligned(16))) T stage_all[kFwdWaves][32 * kStride];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  T* stage = stage_all[w];
  const int n1 = a.n >> kBlockShift;
  const long qb = (long)blockIdx.x * kFwdWaves + w;
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
    int j0 = -1, j1 = -1;
    if (fine) {
      j0 = sel1[2 * ch];
      j1 = (2 * ch + 1 < K) ? sel1[2 * ch + 1] : -1;
    }
    const int cbase = (ch - n_fine_chunks) * 32;   // first coarse slot of a coarse chunk
    auto src = [&](int kk) -> KeySrc {
      KeySrc s;
      if (fine) {
        const int j = kk < 16 ? j0 : j1;
        s.valid = j >= 0 && j < n1;
        s.level = 0;
        s.row = s.valid ? tok_base + token_row(j * kBlock + (kk & 15), a.grid) : 0;
      } else {
        const int slot = cbase + kk;
        s.valid = slot < n_coarse;
        const int l = s.valid ? 2 + slot / K : 2;
        s.level = l;
        s.row = 0;
        if (s.valid) {
          const int nl = a.n >> (kBlockShift * l);
          const int anc = pb >> (kBlockShift * (l - 1));
          const int id = a.sel[l - 1][((long)head * nl + anc) * K + (slot % K)];
          s.valid = id >= 0 && id < nl;
          s.row = s.valid ? (long)head * nl + id : 0;
        }
      }
      return s;
    };

    // ---- stage this chunk's V rows (row-major, 32 x 64) into LDS
#pragma unroll
    for (int ins = 0; ins < (BF16 ? 4 : 8); ++ins) {
      const int per_row = BF16 ? 8 : 16;                   // 16-byte pieces per row
      const int row = ins * (64 / per_row) + lane / per_row;
      const int piece = lane % per_row;
      const KeySrc s = src(row);
      if constexpr (BF16) {
        bf16x8 val;
        if (!s.valid) {
#pragma unroll
          for (int e = 0; e < 8; ++e) val[e] = (bf16)0.f;
        } else if (s.level == 0) {
          val = *(const bf16x8*)((const bf16*)a.v + s.row * kDim + 8 * piece);
        } else {
          const float* vp = a.v_lv[s.level - 1] + s.row * kDim + 8 * piece;
          val = cvt8_bf16(*(const f32x4*)vp, *(const f32x4*)(vp + 4));
        }
        *(bf16x8*)(stage + row * kStride + 8 * piece) = val;
      } else {
        f32x4 val = {0.f, 0.f, 0.f, 0.f};
        if (s.valid) {
          const float* vp = (s.level == 0 ? (const float*)a.v : a.v_lv[s.level - 1]) +
                            s.row * kDim + 4 * piece;
          val = *(const f32x4*)vp;
        }
        *(f32x4*)(stage + row * kStride + 4 * piece) = val;
      }
    }

    // ---- S^T tiles and scores
    float sc[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const KeySrc s = src(tile_row_key(n, t));   // A-operand row owned by this lane
      f32x4 st = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BF16) {
        bf16x8 ka[2];
        if (!s.valid) {
#pragma unroll
          for (int e = 0; e < 8; ++e) ka[0][e] = ka[1][e] = (bf16)0.f;
        } else if (s.level == 0) {
          const bf16* kp = (const bf16*)a.k + s.row * kDim;
          ka[0] = *(const bf16x8*)(kp + 8 * g);
          ka[1] = *(const bf16x8*)(kp + 32 + 8 * g);
        } else {
          const float* kp = a.k_lv[s.level - 1] + s.row * kDim;
          ka[0] = cvt8_bf16(*(const f32x4*)(kp + 8 * g), *(const f32x4*)(kp + 8 * g + 4));
          ka[1] = cvt8_bf16(*(const f32x4*)(kp + 32 + 8 * g),
                            *(const f32x4*)(kp + 32 + 8 * g + 4));
        }
        st = mfma_bf16_k32(ka[0], qh[0], st);
        st = mfma_bf16_k32(ka[1], qh[1], st);
      } else {
        f32x4 kf[4];
        const float* kp = s.valid ? (s.level == 0 ? (const float*)a.k : a.k_lv[s.level - 1]) +
                                        s.row * kDim + 16 * g
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
        const KeySrc s2 = src(8 * g + i + 4 * t);
        const float bias = s2.level ? 4.0f * s2.level : 0.f;   // log2(16^l)
        sc[t][i] = s2.valid ? st[i] * a.c2 + bias : -INFINITY;
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
      bf16x8 pb8;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb8[i] = (bf16)p[0][i];
        pb8[i + 4] = (bf16)p[1][i];
      }
      const int r = (lane & 15) >> 2;
      const int c = lane & 3;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const bf16* base = stage + (8 * g + r) * kStride + 16 * t4 + 4 * c;
        const bf16x4 lo = lds_read_tr16(base);
        const bf16x4 hi = lds_read_tr16(base + 4 * kStride);
        bf16x8 vt;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vt[e] = lo[e];
          vt[e + 4] = hi[e];
        }
        acc[t4] = mfma_bf16_k32(vt, pb8, acc[t4]);
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
