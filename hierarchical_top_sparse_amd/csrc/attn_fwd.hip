// Sparse attention forward with hierarchical KV enrichment (paper summary sec. 四; article
// sec. 三/四: the forward gathers the selected key blocks directly, no dense mask).
//
// One wave owns one level-1 query block p (16 queries); a workgroup holds the 4 consecutive
// blocks of one 8x8-pixel tile, which share their ancestors at every level >= 2.
//  * Fine keys: the 16 tokens of each pair of blocks in Sel_1[p] form a 32-key chunk.  The
//    picks' first-row offsets are computed once into a lane-held table and taken into scalar
//    registers with v_readlane; every lane's row offset inside a 4x4 tile is a constant, so a
//    chunk's 16-byte loads need one add each.  The next chunk's loads are always issued before
//    the current chunk is computed (register double buffering, no data-dependent branch around
//    the prefetch, so the wait for a chunk never drains the loads queued behind it).
//  * Coarse keys: the keys Sel_l[p / 16^(l-1)], l = 2..L, are staged once per workgroup in LDS
//    (fp32 pooled values split into bf16 hi + lo parts, so the MFMA sees them at ~16 bits),
//    together with each slot's log2-domain weight bias 4l (weight 16^l).
//
// Orientation S^T = K Q^T: the MFMA result gives lane (n, g) the scores of query n against
// keys 8g..8g+7 of the chunk (two 16x16 tiles whose rows are interleaved so that this holds),
// so the online-softmax max needs two cross-lane steps and the exponentials already sit in
// the B-operand layout of O^T += V^T P^T.  V^T comes from V rows staged row-major in LDS and
// read with ds_read_b64_tr_b16.  fp32 online softmax in the exp2 domain.
// fp32 tensors use v_mfma_f32_16x16x4f32 with the same data flow.
// Workgroups are renumbered so that each XCD (and its L2) works on one contiguous spatial
// range of query blocks: neighbouring blocks select overlapping key blocks.
#include "common.hpp"
#include "kernels.hpp"

namespace llsa {

constexpr int kMaxLevels = 6;
constexpr int kFwdWaves = 4;
constexpr int kStrideBf16 = kDim + 8;   // 144-byte LDS rows: 16-byte aligned, staggered banks
constexpr int kStrideF32 = kDim + 4;
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
struct FwdCfg {
  static constexpr int ES = BF16 ? 2 : 4;              // element bytes
  static constexpr int kStride = BF16 ? kStrideBf16 : kStrideF32;
  static constexpr int PPR = kDim * ES / 16;           // 16-byte pieces per row
  static constexpr int RPI = 64 / PPR;                 // rows staged per load instruction
  static constexpr int NINS = 32 / RPI;                // load instructions per 32-row chunk
  static constexpr int KLD = BF16 ? 2 : 4;             // 16-byte loads per A-operand row
  static constexpr int NB = BF16 ? 4 : 2;              // coarse buffers: K(hi,lo), V(hi,lo)
  static constexpr int kChunkElems = 32 * kStride;
};

static size_t fwd_lds_bytes(bool bf16, int n_coarse) {
  const int es = bf16 ? 2 : 4;
  const int stride = bf16 ? kStrideBf16 : kStrideF32;
  const int nb = bf16 ? 4 : 2;
  const int cchunks = (n_coarse + 31) / 32;
  return (size_t)es * 32 * stride * (kFwdWaves + cchunks * nb) + sizeof(float) * 32 * cchunks;
}

template <bool BF16>
__global__ __launch_bounds__(64 * kFwdWaves) void attn_fwd_kernel(FwdArgs a) {
  using C = FwdCfg<BF16>;
  typedef typename std::conditional<BF16, bf16, float>::type T;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int n1 = a.n >> kBlockShift;
  const int qb = uniform(xcd_block(blockIdx.x, gridDim.x) * kFwdWaves) + w;
  const int head = uniform(qb / n1);   // scalar: buffer descriptors must be wave-uniform
  const int pb = uniform(qb - head * n1);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int K = a.topk;
  const long tok_base = (long)head * a.n;
  const int n_coarse = a.enrich ? (a.levels - 1) * K : 0;
  const int n_cchunks = (n_coarse + 31) >> 5;
  T* stage = (T*)smem + w * C::kChunkElems;
  T* cstage = (T*)smem + kFwdWaves * C::kChunkElems;
  float* cbias = (float*)(cstage + n_cchunks * C::NB * C::kChunkElems);

  const uint32_t head_bytes = (uint32_t)a.n * kDim * C::ES;
  const rsrc_t rq = make_rsrc_uniform((const char*)a.q + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rk = make_rsrc_uniform((const char*)a.k + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rv = make_rsrc_uniform((const char*)a.v + (size_t)head * head_bytes, head_bytes);

  // ---- the picks of Sel_1[p] as a lane-held table: lane i < K holds the byte offset of pick
  // i's first row (kNoRow for an invalid id and for lanes >= K); chunks read it by v_readlane.
  const int32_t* sel1 = a.sel[0] + ((long)head * n1 + pb) * K;
  uint32_t pick_off = kNoRow;
  if (lane < K) {
    const int j = sel1[lane];
    if (j >= 0 && j < n1) pick_off = (uint32_t)block_corner(j, a.grid) * kDim * C::ES;
  }

  // ---- queries: B operand of S^T
  const int qrow = block_corner(pb, a.grid) + tile_offset(n, a.grid);
  bf16x8 qh[2];
  f32x4 qf[4];
  if constexpr (BF16) {
    qh[0] = buf_load8(rq, (uint32_t)(qrow * kDim + 8 * g) * 2);
    qh[1] = buf_load8(rq, (uint32_t)(qrow * kDim + 32 + 8 * g) * 2);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) qf[c] = buf_load4f(rq, (uint32_t)(qrow * kDim + 16 * g + 4 * c) * 4);
  }

  // ---- lane-constant byte offsets inside a block: staged rows and A-operand rows
  const int srow0 = lane / C::PPR;
  const int piece = lane % C::PPR;
  uint32_t st_off[C::NINS];
#pragma unroll
  for (int ins = 0; ins < C::NINS; ++ins)
    st_off[ins] = (uint32_t)(tile_offset((ins * C::RPI + srow0) & 15, a.grid) * kDim * C::ES +
                             16 * piece);
  uint32_t ka_off[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
    ka_off[t] = (uint32_t)(tile_offset(tile_row_key(n, t) & 15, a.grid) * kDim * C::ES) +
                (BF16 ? 16 * g : 64 * g);
  const bool ka_second = n >= 8;    // A rows 8..15 of both tiles come from the second block
  const bool lane_second = g >= 2;  // this lane's 8 keys come from the second block
  const int n_fine = (K + 1) >> 1;

  // loads of fine chunk ch (blocks 2ch, 2ch+1 of the table), issued one chunk ahead of use.
  // Every call issues the same loads, also past the last chunk (kNoRow: zeros, no memory
  // access), so the wait before a chunk's use never has to drain the prefetch behind it.
  struct FineLd {
    i32x4 v[C::NINS];
    i32x4 k[2][C::KLD];
    int ok0, ok1;
  };
  auto load_fine = [&](int ch) -> FineLd {
    FineLd f;
    const uint32_t b0 = (uint32_t)__builtin_amdgcn_readlane((int)pick_off, 2 * ch);
    const uint32_t b1 = (uint32_t)__builtin_amdgcn_readlane((int)pick_off, 2 * ch + 1);
    f.ok0 = b0 != kNoRow;
    f.ok1 = b1 != kNoRow;
#pragma unroll
    for (int ins = 0; ins < C::NINS; ++ins)
      f.v[ins] = __builtin_amdgcn_raw_buffer_load_b128(rv, (ins * C::RPI >= 16 ? b1 : b0) +
                                                           st_off[ins], 0, 0);
    const uint32_t kb = ka_second ? b1 : b0;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int c = 0; c < C::KLD; ++c)
        f.k[t][c] = __builtin_amdgcn_raw_buffer_load_b128(
            rk, kb + ka_off[t] + (BF16 ? 64 * c : 16 * c), 0, 0);
    return f;
  };
  FineLd fa = load_fine(0), fb;

  // ---- the workgroup's coarse keys and values, shared by its four query blocks (their loads
  // overlap the first fine chunk's)
  if (n_coarse > 0) {
    const int pb0 = pb & ~(kFwdWaves - 1);
    for (int e = threadIdx.x; e < n_cchunks * 32 * 8; e += 64 * kFwdWaves) {
      const int slot = e >> 3;
      const int c8 = (e & 7) * 8;
      f32x4 k0 = {0.f, 0.f, 0.f, 0.f}, k1 = k0, v0 = k0, v1 = k0;
      float bias = -INFINITY;
      if (slot < n_coarse) {
        const int l = 2 + slot / K;
        const int nl = a.n >> (kBlockShift * l);
        const int anc = pb0 >> (kBlockShift * (l - 1));
        const int id = a.sel[l - 1][((long)head * nl + anc) * K + (slot - (l - 2) * K)];
        if (id >= 0 && id < nl) {
          const float* kp = a.k_lv[l - 1] + ((long)head * nl + id) * kDim + c8;
          const float* vp = a.v_lv[l - 1] + ((long)head * nl + id) * kDim + c8;
          k0 = *(const f32x4*)kp;
          k1 = *(const f32x4*)(kp + 4);
          v0 = *(const f32x4*)vp;
          v1 = *(const f32x4*)(vp + 4);
          bias = 4.0f * (float)l;   // log2(16^l)
        }
      }
      T* base = cstage + (slot >> 5) * C::NB * C::kChunkElems + (slot & 31) * C::kStride + c8;
      if constexpr (BF16) {
        bf16x8 hi, lo;
        split_bf16(k0, k1, hi, lo);
        *(bf16x8*)base = hi;
        *(bf16x8*)(base + C::kChunkElems) = lo;
        split_bf16(v0, v1, hi, lo);
        *(bf16x8*)(base + 2 * C::kChunkElems) = hi;
        *(bf16x8*)(base + 3 * C::kChunkElems) = lo;
      } else {
        *(f32x4*)base = k0;
        *(f32x4*)(base + 4) = k1;
        *(f32x4*)(base + C::kChunkElems) = v0;
        *(f32x4*)(base + C::kChunkElems + 4) = v1;
      }
      if (c8 == 0) cbias[slot] = bias;
    }
    __syncthreads();
  }

  float m_run = kMinusBig;   // running max (log2 domain) of query n
  float l_run = 0.f;         // this lane's partial sum of exp2
  f32x4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // online softmax over one chunk's scores, then O^T += V^T P^T from the row-major V rows at
  // vbuf (and the lo parts at vlo, if any)
  auto absorb = [&](float (&sc)[2][4], const T* vbuf, const T* vlo) {
    float mloc = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                       fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    const float m_new = fmaxf(m_run, group4_max(mloc));
    const float alpha = fast_exp2(m_run - m_new);
    float p[2][4];
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[t][i] = fast_exp2(sc[t][i] - m_new);
        psum += p[t][i];
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t4][i] *= alpha;
    wave_lds_sync();
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
        const int off = (8 * g + r) * C::kStride + 16 * t4 + 4 * c;
        const bf16x4 x0 = lds_read_tr16(vbuf + off);
        const bf16x4 x1 = lds_read_tr16(vbuf + off + 4 * C::kStride);
        bf16x8 vt;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vt[e] = x0[e];
          vt[e + 4] = x1[e];
        }
        acc[t4] = mfma_bf16_k32(vt, pb8, acc[t4]);
        if (vlo) {
          const bf16x4 y0 = lds_read_tr16(vlo + off);
          const bf16x4 y1 = lds_read_tr16(vlo + off + 4 * C::kStride);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            vt[e] = y0[e];
            vt[e + 4] = y1[e];
          }
          acc[t4] = mfma_bf16_k32(vt, pb8, acc[t4]);
        }
      }
    } else {
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float vv = vbuf[(8 * g + i + 4 * t) * C::kStride + 16 * t4 + n];
            acc[t4] = mfma_f32_k4(vv, p[t][i], acc[t4]);
          }
    }
    wave_lds_sync();
  };

  // one fine chunk from its loads: V rows to LDS, S^T on the MFMA, softmax and PV
  auto fine_chunk = [&](const FineLd& f) {
#pragma unroll
    for (int ins = 0; ins < C::NINS; ++ins)
      *(i32x4*)(stage + (ins * C::RPI + srow0) * C::kStride + piece * (16 / C::ES)) = f.v[ins];
    float sc[2][4];
    const float madd = (lane_second ? f.ok1 : f.ok0) ? 0.f : -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x4 st = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BF16) {
        st = mfma_bf16_k32(*(const bf16x8*)&f.k[t][0], qh[0], st);
        st = mfma_bf16_k32(*(const bf16x8*)&f.k[t][1], qh[1], st);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const f32x4 kf = *(const f32x4*)&f.k[t][c];
#pragma unroll
          for (int e = 0; e < 4; ++e) st = mfma_f32_k4(kf[e], qf[c][e], st);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[t][i] = fmaf(st[i], a.c2, madd);
    }
    absorb(sc, stage, nullptr);
  };

  // ---- fine chunks: two load buffers used in turn, each refilled while the other computes
  for (int ch = 0; ch < n_fine; ch += 2) {
    fb = load_fine(ch + 1);
    fine_chunk(fa);
    if (ch + 1 >= n_fine) break;
    fa = load_fine(ch + 2);
    fine_chunk(fb);
  }

  // ---- coarse chunks from the workgroup's LDS copy
  for (int cc = 0; cc < n_cchunks; ++cc) {
    const T* kb = cstage + cc * C::NB * C::kChunkElems;
    float sc[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = tile_row_key(n, t);
      f32x4 st = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BF16) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16* rp = kb + row * C::kStride + 32 * s + 8 * g;
          st = mfma_bf16_k32(*(const bf16x8*)rp, qh[s], st);
          st = mfma_bf16_k32(*(const bf16x8*)(rp + C::kChunkElems), qh[s], st);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const f32x4 kf = *(const f32x4*)(kb + row * C::kStride + 16 * g + 4 * c);
#pragma unroll
          for (int e = 0; e < 4; ++e) st = mfma_f32_k4(kf[e], qf[c][e], st);
        }
      }
      const f32x4 b4 = *(const f32x4*)(cbias + cc * 32 + 8 * g + 4 * t);
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[t][i] = fmaf(st[i], a.c2, b4[i]);
    }
    absorb(sc, kb + (BF16 ? 2 : 1) * C::kChunkElems, BF16 ? kb + 3 * C::kChunkElems : nullptr);
  }

  // ---- finalize
  const float l_tot = group4_sum(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;   // 0 only if every key was skipped
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
  const int n_coarse = s.enrich ? (s.levels - 1) * s.topk : 0;
  const size_t lds = fwd_lds_bytes(s.bf16, n_coarse);
  // every workgroup holds 4 whole query blocks of one head (N / 16 is a multiple of 4)
  const long waves = (long)s.bh * (s.n >> kBlockShift);
  const unsigned blocks = (unsigned)(waves / kFwdWaves);
  const void* fn = s.bf16 ? (const void*)attn_fwd_kernel<true> : (const void*)attn_fwd_kernel<false>;
  if (lds > 65536) {
    const hipError_t e =
        hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (s.bf16)
    LLSA_LAUNCH("attn_fwd_kernel", attn_fwd_kernel<true>, dim3(blocks), dim3(64 * kFwdWaves), lds, stream, a);
  else
    LLSA_LAUNCH("attn_fwd_kernel", attn_fwd_kernel<false>, dim3(blocks), dim3(64 * kFwdWaves), lds, stream, a);
  return hipGetLastError();
}

}  // namespace llsa
