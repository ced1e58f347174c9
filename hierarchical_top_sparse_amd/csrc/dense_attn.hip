// Dense softmax attention, forward and backward, on bf16 MFMA: the full-attention baseline
// the sparse method is measured against (the pages compare against a dense FlashAttention
// kernel at the same sequence lengths; paper summary sec. 5.4, Figure 3).
//
// Tokens form a plain sequence [bh, N, 64] (attention over all N keys does not depend on the
// token order).  Flash-style tiling, fp32 accumulation and softmax, no T x T matrix in memory:
//  * dense_fwd_kernel: a workgroup owns 128 queries (4 waves x 32); K and V blocks of 64 rows
//    are staged in LDS (double-buffered, one barrier per block) and every wave streams them:
//    S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with the key rows of the two 16-row tiles of a
//    32-key chunk interleaved, so that each lane ends up with query n's scores for keys
//    8g .. 8g + 7 -- the B-operand layout of O^T += V^T P^T, whose V^T is read from the V rows
//    with ds_read_b64_tr_b16.  Online softmax in the exp2 domain with a lazily moved max.
//  * dense_bwd_dq_kernel: same streaming; per chunk S^T and dP^T = V dO^T, P = exp2(S c2 -
//    lse2); D = sum P dP and dQ = scale (sum P dP k - D sum P k) in one pass (D exact, the
//    stored O is not needed); writes D.
//  * dense_bwd_dkv_kernel: a workgroup owns 128 keys (4 waves x 32) and streams 64-query
//    blocks of Q, dO, LSE and D through LDS: S = Q K^T, dP = dO V^T (query rows interleaved
//    the same way), dV^T += dO^T P and dK^T += Q^T dS.
// P enters the MFMA rounded to bf16 (the usual flash-attention choice); dS, whose terms cancel,
// enters as a bf16 hi + lo pair, as in the sparse backward.  All sums are in a fixed order:
// deterministic, no atomics.
#include "common.hpp"
#include "kernels.hpp"

namespace llsa {

constexpr int kDnWaves = 4;
constexpr int kDnRows = 32;              // queries (fwd, dQ) or keys (dK/dV) per wave
constexpr int kDnBlock = 64;             // streamed rows per LDS block
constexpr int kDnStride = kDim + 8;      // LDS row stride (bf16 elements): 144 bytes
constexpr int kDnTile = kDnBlock * kDnStride;
constexpr float kDnLazy = 8.f;
constexpr float kDnMinusBig = -1e30f;

// MFMA row r of tile t of a 32-row chunk holds chunk row 8 (r / 4) + r % 4 + 4 t, so that the
// output rows 4g + i of tiles 0 and 1 are chunk rows 8g + i and 8g + 4 + i.
__device__ __forceinline__ int dn_chunk_row(int r, int t) { return 8 * (r >> 2) + (r & 3) + 4 * t; }

__device__ __forceinline__ bf16x8 dn_row8(const bf16* st, int row, int s, int g) {
  return *(const bf16x8*)(st + row * kDnStride + 32 * s + 8 * g);
}
// Transposed operand: chunk rows 8g .. 8g + 7 at columns 16 t4 .. + 15 (lane gets its column).
__device__ __forceinline__ bf16x8 dn_tr8(const bf16* st, int t4, int lane) {
  const int g = lane >> 4;
  const int r = (lane & 15) >> 2;
  const int c = lane & 3;
  const bf16* base = st + (8 * g + r) * kDnStride + 16 * t4 + 4 * c;
  const bf16x4 lo = lds_read_tr16(base);
  const bf16x4 hi = lds_read_tr16(base + 4 * kDnStride);
  bf16x8 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    out[e] = lo[e];
    out[e + 4] = hi[e];
  }
  return out;
}

// x = hi + lo, both bf16: dS sums values of both signs to ~0 per query, so its products keep
// ~16 mantissa bits this way (a single bf16 rounding of dS costs ~2^-9 of every term).
__device__ __forceinline__ void dn_split(float x, bf16x8& hi, bf16x8& lo, int e) {
  const bf16 h = (bf16)x;
  hi[e] = h;
  lo[e] = (bf16)(x - (float)h);
}

struct DenseArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* dout;
  float* lse;    // [bh, N] natural log
  float* dd;     // [bh, N] D = rowsum(dO o O)
  bf16* out;     // fwd: O; bwd: dQ
  bf16* dk;
  bf16* dv;
  int n;
  float scale;
  float c2;      // scale * log2(e)
};

// Stages rows [row0, row0 + 64) of two [N, 64] bf16 tensors: thread tid owns pieces tid and
// tid + 256 (16 bytes each) of each.
struct DnStage {
  i32x4 a[2], b[2];
};
__device__ __forceinline__ DnStage dn_load(rsrc_t ra, rsrc_t rb, int row0, int tid) {
  DnStage s;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int e = tid + 256 * m;
    const uint32_t off = (uint32_t)((row0 + (e >> 3)) * kDim + 8 * (e & 7)) * 2;
    s.a[m] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
    s.b[m] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
  }
  return s;
}
__device__ __forceinline__ void dn_store(const DnStage& s, bf16* ta, bf16* tb, int tid) {
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int e = tid + 256 * m;
    const int at = (e >> 3) * kDnStride + 8 * (e & 7);
    *(i32x4*)(ta + at) = s.a[m];
    *(i32x4*)(tb + at) = s.b[m];
  }
}

// ----------------------------------------------------------------------------------- forward
__global__ __launch_bounds__(64 * kDnWaves) __attribute__((amdgpu_waves_per_eu(2)))
void dense_fwd_kernel(DenseArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 sk[2][kDnTile];
  __shared__ __attribute__((aligned(16))) bf16 sv[2][kDnTile];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int per_head = a.n / (kDnWaves * kDnRows);
  const int wg = uniform(xcd_block(blockIdx.x, gridDim.x));
  const int head = uniform(wg / per_head);
  const int q0 = uniform((wg - head * per_head) * kDnWaves * kDnRows + kDnRows * w);
  const uint32_t head_bytes = (uint32_t)a.n * kDim * 2;
  const rsrc_t rq = make_rsrc_uniform((const char*)a.q + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rk = make_rsrc_uniform((const char*)a.k + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rv = make_rsrc_uniform((const char*)a.v + (size_t)head * head_bytes, head_bytes);

  bf16x8 qh[2][2];   // B operand of S^T: lane (n, g) holds query q0 + 16 qt + n, ch 32 s + 8 g
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int s = 0; s < 2; ++s)
      qh[qt][s] = buf_load8(rq, (uint32_t)((q0 + 16 * qt + n) * kDim + 32 * s + 8 * g) * 2);

  float m_run[2] = {kDnMinusBig, kDnMinusBig}, l_run[2] = {0.f, 0.f};
  f32x4 acc[2][4];   // O^T: lane (n, g) holds dims 16 t4 + 4 g + i of query n
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) acc[qt][t4] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nblocks = a.n / kDnBlock;
  DnStage st = dn_load(rk, rv, 0, tid);
  for (int kb = 0; kb < nblocks; ++kb) {
    const int buf = kb & 1;
    dn_store(st, sk[buf], sv[buf], tid);
    __syncthreads();
    if (kb + 1 < nblocks) st = dn_load(rk, rv, (kb + 1) * kDnBlock, tid);
#pragma unroll
    for (int c = 0; c < kDnBlock / 32; ++c) {
      const bf16* kc = sk[buf] + 32 * c * kDnStride;
      const bf16* vc = sv[buf] + 32 * c * kDnStride;
      bf16x8 ka[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int s = 0; s < 2; ++s) ka[t][s] = dn_row8(kc, dn_chunk_row(n, t), s, g);
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        float x[2][4];
        float mloc = kDnMinusBig;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f32x4 sc = {0.f, 0.f, 0.f, 0.f};
          sc = mfma_bf16_k32(ka[t][0], qh[qt][0], sc);
          sc = mfma_bf16_k32(ka[t][1], qh[qt][1], sc);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[t][i] = sc[i] * a.c2;
            mloc = fmaxf(mloc, x[t][i]);
          }
        }
        if (__builtin_amdgcn_ballot_w64(mloc > m_run[qt] + kDnLazy)) {   // wave-uniform
          const float m_new = fmaxf(m_run[qt], group4_max(mloc));
          const float alpha = fast_exp2(m_run[qt] - m_new);
          l_run[qt] *= alpha;
#pragma unroll
          for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[qt][t4][i] *= alpha;
          m_run[qt] = m_new;
        }
        bf16x8 pb;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = fast_exp2(x[t][i] - m_run[qt]);
            l_run[qt] += p;
            pb[4 * t + i] = (bf16)p;
          }
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4)
          acc[qt][t4] = mfma_bf16_k32(dn_tr8(vc, t4, lane), pb, acc[qt][t4]);
      }
    }
  }
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int qrow = q0 + 16 * qt + n;
    const float l_tot = group4_sum(l_run[qt]);
    const float inv = 1.0f / l_tot;
    bf16* op = a.out + ((long)head * a.n + qrow) * kDim;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      bf16x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = (bf16)(acc[qt][t4][i] * inv);
      *(bf16x4*)(op + 16 * t4 + 4 * g) = r;
    }
    if (g == 0) a.lse[(long)head * a.n + qrow] = (m_run[qt] + log2f(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------- backward: dQ
// D = sum_j P_ij dP_ij is accumulated with the rest in one pass (exact, unlike rowsum(dO o O)
// with the bf16-rounded O): with A = sum_j P_ij dP_ij k_j and Bv = sum_j P_ij k_j,
// dq_i = scale sum_j P_ij (dP_ij - D_i) k_j = scale (A - D_i Bv).  P dP and P enter the MFMA
// as bf16 hi + lo pairs.  D is written for the dK/dV kernel.
__global__ __launch_bounds__(64 * kDnWaves) __attribute__((amdgpu_waves_per_eu(2)))
void dense_bwd_dq_kernel(DenseArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 sk[2][kDnTile];
  __shared__ __attribute__((aligned(16))) bf16 sv[2][kDnTile];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int per_head = a.n / (kDnWaves * kDnRows);
  const int wg = uniform(xcd_block(blockIdx.x, gridDim.x));
  const int head = uniform(wg / per_head);
  const int q0 = uniform((wg - head * per_head) * kDnWaves * kDnRows + kDnRows * w);
  const long tok = (long)head * a.n;
  const uint32_t head_bytes = (uint32_t)a.n * kDim * 2;
  const rsrc_t rq = make_rsrc_uniform((const char*)a.q + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rk = make_rsrc_uniform((const char*)a.k + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rv = make_rsrc_uniform((const char*)a.v + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rdo =
      make_rsrc_uniform((const char*)a.dout + (size_t)head * head_bytes, head_bytes);

  bf16x8 qh[2][2], dh[2][2];
  float lse2[2], dpart[2] = {0.f, 0.f};
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int qrow = q0 + 16 * qt + n;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint32_t off = (uint32_t)(qrow * kDim + 32 * s + 8 * g) * 2;
      qh[qt][s] = buf_load8(rq, off);
      dh[qt][s] = buf_load8(rdo, off);
    }
    lse2[qt] = a.lse[tok + qrow] * kLog2e;
  }

  f32x4 ac[2][4], bv[2][4];   // A^T, Bv^T: lane (n, g) holds dims 16 t4 + 4 g + i of query n
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) ac[qt][t4] = bv[qt][t4] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nblocks = a.n / kDnBlock;
  DnStage st = dn_load(rk, rv, 0, tid);
  for (int kb = 0; kb < nblocks; ++kb) {
    const int buf = kb & 1;
    dn_store(st, sk[buf], sv[buf], tid);
    __syncthreads();
    if (kb + 1 < nblocks) st = dn_load(rk, rv, (kb + 1) * kDnBlock, tid);
#pragma unroll
    for (int c = 0; c < kDnBlock / 32; ++c) {
      const bf16* kc = sk[buf] + 32 * c * kDnStride;
      const bf16* vc = sv[buf] + 32 * c * kDnStride;
      bf16x8 ka[2][2], va[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          ka[t][s] = dn_row8(kc, dn_chunk_row(n, t), s, g);
          va[t][s] = dn_row8(vc, dn_chunk_row(n, t), s, g);
        }
      bf16x8 kt8[4];
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) kt8[t4] = dn_tr8(kc, t4, lane);
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        bf16x8 w_hi, w_lo, p_hi, p_lo;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f32x4 sc = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
          sc = mfma_bf16_k32(ka[t][0], qh[qt][0], sc);
          sc = mfma_bf16_k32(ka[t][1], qh[qt][1], sc);
          dp = mfma_bf16_k32(va[t][0], dh[qt][0], dp);
          dp = mfma_bf16_k32(va[t][1], dh[qt][1], dp);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = fast_exp2(fmaf(sc[i], a.c2, -lse2[qt]));
            const float w1 = p * dp[i];
            dpart[qt] += w1;
            dn_split(w1, w_hi, w_lo, 4 * t + i);
            dn_split(p, p_hi, p_lo, 4 * t + i);
          }
        }
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
          ac[qt][t4] = mfma_bf16_k32(kt8[t4], w_hi, ac[qt][t4]);
          ac[qt][t4] = mfma_bf16_k32(kt8[t4], w_lo, ac[qt][t4]);
          bv[qt][t4] = mfma_bf16_k32(kt8[t4], p_hi, bv[qt][t4]);
          bv[qt][t4] = mfma_bf16_k32(kt8[t4], p_lo, bv[qt][t4]);
        }
      }
    }
  }
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int qrow = q0 + 16 * qt + n;
    const float dd = group4_sum(dpart[qt]);   // D of query qrow, in every lane of column n
    if (g == 0) a.dd[tok + qrow] = dd;
    bf16* op = a.out + (tok + qrow) * kDim;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      bf16x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = (bf16)(a.scale * (ac[qt][t4][i] - dd * bv[qt][t4][i]));
      *(bf16x4*)(op + 16 * t4 + 4 * g) = r;
    }
  }
}

// ------------------------------------------------------------------------ backward: dK, dV
__global__ __launch_bounds__(64 * kDnWaves) __attribute__((amdgpu_waves_per_eu(2)))
void dense_bwd_dkv_kernel(DenseArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 sq[2][kDnTile];
  __shared__ __attribute__((aligned(16))) bf16 so[2][kDnTile];   // dO rows
  __shared__ __attribute__((aligned(16))) float sl[2][kDnBlock];   // lse2 of the block
  __shared__ __attribute__((aligned(16))) float sd[2][kDnBlock];   // D of the block
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int per_head = a.n / (kDnWaves * kDnRows);
  const int wg = uniform(xcd_block(blockIdx.x, gridDim.x));
  const int head = uniform(wg / per_head);
  const int k0 = uniform((wg - head * per_head) * kDnWaves * kDnRows + kDnRows * w);
  const long tok = (long)head * a.n;
  const uint32_t head_bytes = (uint32_t)a.n * kDim * 2;
  const rsrc_t rq = make_rsrc_uniform((const char*)a.q + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rk = make_rsrc_uniform((const char*)a.k + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rv = make_rsrc_uniform((const char*)a.v + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rdo =
      make_rsrc_uniform((const char*)a.dout + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rl = make_rsrc_uniform(a.lse + tok, (uint32_t)a.n * 4);
  const rsrc_t rd = make_rsrc_uniform(a.dd + tok, (uint32_t)a.n * 4);

  bf16x8 kh[2][2], vh[2][2];   // B operands: lane (n, g) holds key k0 + 16 kt + n, ch 32 s + 8g
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint32_t off = (uint32_t)((k0 + 16 * kt + n) * kDim + 32 * s + 8 * g) * 2;
      kh[kt][s] = buf_load8(rk, off);
      vh[kt][s] = buf_load8(rv, off);
    }
  f32x4 dka[2][4], dva[2][4];   // dK^T, dV^T: lane (n, g) holds dims 16 t4 + 4g + i of key n
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) dka[kt][t4] = dva[kt][t4] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nblocks = a.n / kDnBlock;
  DnStage st = dn_load(rq, rdo, 0, tid);
  float ld = 0.f;
  if (tid < 2 * kDnBlock)
    ld = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                       tid < kDnBlock ? rl : rd, (uint32_t)(tid & 63) * 4, 0, 0));
  for (int qb = 0; qb < nblocks; ++qb) {
    const int buf = qb & 1;
    dn_store(st, sq[buf], so[buf], tid);
    if (tid < kDnBlock) sl[buf][tid] = ld * kLog2e;
    else if (tid < 2 * kDnBlock) sd[buf][tid - kDnBlock] = ld;
    __syncthreads();
    if (qb + 1 < nblocks) {
      st = dn_load(rq, rdo, (qb + 1) * kDnBlock, tid);
      if (tid < 2 * kDnBlock)
        ld = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(
                       tid < kDnBlock ? rl : rd,
                       (uint32_t)((qb + 1) * kDnBlock + (tid & 63)) * 4, 0, 0));
    }
#pragma unroll
    for (int c = 0; c < kDnBlock / 32; ++c) {
      const bf16* qc = sq[buf] + 32 * c * kDnStride;
      const bf16* oc = so[buf] + 32 * c * kDnStride;
      bf16x8 qa[2][2], oa[2][2];
      f32x4 l4[2], d4[2];   // lse2 and D of chunk rows 8g + 4t + i
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          qa[t][s] = dn_row8(qc, dn_chunk_row(n, t), s, g);
          oa[t][s] = dn_row8(oc, dn_chunk_row(n, t), s, g);
        }
        l4[t] = *(const f32x4*)(&sl[buf][32 * c + 8 * g + 4 * t]);
        d4[t] = *(const f32x4*)(&sd[buf][32 * c + 8 * g + 4 * t]);
      }
      bf16x8 qt8[4], ot8[4];
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        qt8[t4] = dn_tr8(qc, t4, lane);
        ot8[t4] = dn_tr8(oc, t4, lane);
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        bf16x8 pb, ds_hi, ds_lo;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f32x4 sc = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
          sc = mfma_bf16_k32(qa[t][0], kh[kt][0], sc);
          sc = mfma_bf16_k32(qa[t][1], kh[kt][1], sc);
          dp = mfma_bf16_k32(oa[t][0], vh[kt][0], dp);
          dp = mfma_bf16_k32(oa[t][1], vh[kt][1], dp);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = fast_exp2(fmaf(sc[i], a.c2, -l4[t][i]));
            pb[4 * t + i] = (bf16)p;
            dn_split(p * (dp[i] - d4[t][i]), ds_hi, ds_lo, 4 * t + i);
          }
        }
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
          dva[kt][t4] = mfma_bf16_k32(ot8[t4], pb, dva[kt][t4]);
          dka[kt][t4] = mfma_bf16_k32(qt8[t4], ds_hi, dka[kt][t4]);
          dka[kt][t4] = mfma_bf16_k32(qt8[t4], ds_lo, dka[kt][t4]);
        }
      }
    }
  }
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const long row = tok + k0 + 16 * kt + n;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      bf16x4 rk4, rv4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rk4[i] = (bf16)(dka[kt][t4][i] * a.scale);
        rv4[i] = (bf16)dva[kt][t4][i];
      }
      *(bf16x4*)(a.dk + row * kDim + 16 * t4 + 4 * g) = rk4;
      *(bf16x4*)(a.dv + row * kDim + 16 * t4 + 4 * g) = rv4;
    }
  }
}

hipError_t launch_dense_fwd(int bh, int n, float scale, const void* q, const void* k,
                            const void* v, void* o, float* lse, hipStream_t stream) {
  DenseArgs a{};
  a.q = (const bf16*)q;
  a.k = (const bf16*)k;
  a.v = (const bf16*)v;
  a.out = (bf16*)o;
  a.lse = lse;
  a.n = n;
  a.scale = scale;
  a.c2 = scale * kLog2e;
  const unsigned blocks = (unsigned)((long)bh * (n / (kDnWaves * kDnRows)));
  LLSA_LAUNCH("dense_fwd_kernel", dense_fwd_kernel, dim3(blocks), dim3(64 * kDnWaves), 0,
              stream, a);
  return hipGetLastError();
}

hipError_t launch_dense_bwd(int bh, int n, float scale, const void* q, const void* k,
                            const void* v, const void* dout, const float* lse, void* dq,
                            void* dk, void* dv, float* dd, hipStream_t stream) {
  DenseArgs a{};
  a.q = (const bf16*)q;
  a.k = (const bf16*)k;
  a.v = (const bf16*)v;
  a.dout = (const bf16*)dout;
  a.lse = (float*)lse;
  a.dd = dd;
  a.out = (bf16*)dq;
  a.dk = (bf16*)dk;
  a.dv = (bf16*)dv;
  a.n = n;
  a.scale = scale;
  a.c2 = scale * kLog2e;
  const unsigned blocks = (unsigned)((long)bh * (n / (kDnWaves * kDnRows)));
  LLSA_LAUNCH("dense_bwd_dq_kernel", dense_bwd_dq_kernel, dim3(blocks), dim3(64 * kDnWaves), 0,
              stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  LLSA_LAUNCH("dense_bwd_dkv_kernel", dense_bwd_dkv_kernel, dim3(blocks), dim3(64 * kDnWaves),
              0, stream, a);
  return hipGetLastError();
}

}  // namespace llsa
