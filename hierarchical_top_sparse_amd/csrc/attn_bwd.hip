// Sparse attention backward (paper summary sec. 4.1 and Figure 4: the KV gradient is
// computed key-major over a CSR->CSC sparse index transpose, so no T x T mask is formed).
//
// Three stages, all deterministic (no atomics):
//  1. bwd_query_kernel  (query-major, one wave per level-1 query block, one workgroup per
//     level-2 group of 16 blocks): D = sum_e P_e dP_e (exact, from the recomputed scores, so
//     the rounded O is never needed), dQ over the block's fine and coarse keys,
//     and, for the coarse keys, the workgroup's partial dK/dV sums (every query of a level-2
//     group shares the same coarse keys).
//  2. coarse_reduce_kernel / coarse_grad_kernel: partials of levels >= 3 are summed over the
//     level-2 groups of each ancestor, then each coarse key j of level l gathers
//     dK_l[j] = sum over the ancestors a in CSC_l[j] of the partial of a's slot holding j.
//  3. bwd_key_kernel (key-major, one wave per level-1 key block): walks the query blocks in
//     CSC_1[j] two at a time, accumulates dK, dV on the MFMA, and adds the pooled gradients
//     pushed down to the block's tokens (dK_l[ancestor] / 16^l, chain rule of the mean).
//
// MFMA data flow (bf16 16x16x32, fp32 accumulation): products that contract over head_dim
// read row-major operands; products that contract over keys or queries read their row-major
// operand from LDS with ds_read_b64_tr_b16.  Chunks of 32 keys (or queries) use the same row
// interleave as the forward, so score tiles come out in the B-operand layout of the next MFMA.
#include "common.hpp"
#include "kernels.hpp"

namespace llsa {

constexpr int kMaxLv = 6;
constexpr int kStride = kDim + 8;   // LDS row stride in bf16 elements (144 bytes)
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
  float* part_k;               // [bh, n2, n_coarse, 64]
  float* part_v;
  float* lvl_part_k[kMaxLv];   // level l >= 3: [bh, n_l, K, 64]
  float* lvl_part_v[kMaxLv];
  float* dk_lv[kMaxLv];        // level l >= 2: [bh, n_l, 64]
  float* dv_lv[kMaxLv];
  int bh;
  int n;
  Grid grid;
  int levels;
  int topk;
  int enrich;
  float scale;
  float c2;   // scale * log2(e)
};

__device__ __forceinline__ int chunk_key(int r, int t) { return 8 * (r >> 2) + (r & 3) + 4 * t; }

// x = hi + lo with both parts in bf16: the pair carries ~16 mantissa bits, so products that
// sum values of both signs (dS sums to zero per query) keep fp32-level accuracy on the MFMA.
__device__ __forceinline__ void split8(const float (&x)[2][4], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16 h = (bf16)x[t][i];
      hi[4 * t + i] = h;
      lo[4 * t + i] = (bf16)(x[t][i] - (float)h);
    }
}

__device__ __forceinline__ void split_f32x8(f32x4 a, f32x4 b, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16 ha = (bf16)a[i], hb = (bf16)b[i];
    hi[i] = ha;
    hi[i + 4] = hb;
    lo[i] = (bf16)(a[i] - (float)ha);
    lo[i + 4] = (bf16)(b[i] - (float)hb);
  }
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (bf16)0.f;
  return z;
}

// A operand (rows of a row-major LDS matrix): lane (m, g) gets row `row`, cols 32s + 8g..+7
__device__ __forceinline__ bf16x8 lds_row8(const bf16* st, int row, int s, int g) {
  return *(const bf16x8*)(st + row * kStride + 32 * s + 8 * g);
}
// Transposed operand: rows k0 + 8g .. +7 (k axis) at column block 16*t4 (lane gets its column)
__device__ __forceinline__ bf16x8 lds_tr8(const bf16* st, int t4, int lane) {
  const int g = lane >> 4;
  const int r = (lane & 15) >> 2;
  const int c = lane & 3;
  const bf16* base = st + (8 * g + r) * kStride + 16 * t4 + 4 * c;
  const bf16x4 lo = lds_read_tr16(base);
  const bf16x4 hi = lds_read_tr16(base + 4 * kStride);
  bf16x8 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    out[e] = lo[e];
    out[e + 4] = hi[e];
  }
  return out;
}

// ====================================================================== stage 1: query-major
template <int NST>   // coarse slot tiles (of 16) kept in registers: 0, 1 or 2
__global__ __launch_bounds__(256) void bwd_query_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 sK[4][32 * kStride];    // K rows (hi part)
  __shared__ __attribute__((aligned(16))) bf16 sKl[4][32 * kStride];   // lo part (pooled keys)
  __shared__ __attribute__((aligned(16))) bf16 sQ[4][16 * kStride];
  __shared__ __attribute__((aligned(16))) bf16 sO[4][16 * kStride];   // dO rows
  __shared__ __attribute__((aligned(16))) bf16 sP[4][2][32 * 16];     // P^T [slot][q], hi/lo
  __shared__ __attribute__((aligned(16))) bf16 sS[4][2][32 * 16];     // dS^T [slot][q], hi/lo
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int n1 = a.n >> kBlockShift;
  const int n2 = n1 >> kBlockShift;
  const int wg = xcd_block(blockIdx.x, gridDim.x);
  const int head = wg / n2;
  const int a2 = wg - head * n2;
  const int K = a.topk;
  const long tok_base = (long)head * a.n;
  const int n_coarse = a.enrich ? (a.levels - 1) * K : 0;
  const int n_fine_chunks = (K + 1) >> 1;
  const int n_chunks = n_fine_chunks + ((n_coarse + 31) >> 5);
  bf16* stK = sK[w];
  bf16* stKl = sKl[w];
  bf16* stQ = sQ[w];
  bf16* stO = sO[w];
  bf16* stP = sP[w][0];
  bf16* stPl = sP[w][1];
  bf16* stS = sS[w][0];
  bf16* stSl = sS[w][1];

  f32x4 cpk[NST > 0 ? NST : 1][4];   // coarse partial dK (unscaled): [slot tile][d tile]
  f32x4 cpv[NST > 0 ? NST : 1][4];
#pragma unroll
  for (int st = 0; st < (NST > 0 ? NST : 1); ++st)
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) cpk[st][t4] = cpv[st][t4] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int it = 0; it < 4; ++it) {
    const int pb = a2 * kBlock + w * 4 + it;
    const int qrow = token_row(pb * kBlock + n, a.grid);
    const bf16* qp = a.q + (tok_base + qrow) * kDim;
    const bf16* dop = a.dout + (tok_base + qrow) * kDim;
    bf16x8 qh[2], dh[2];
    qh[0] = *(const bf16x8*)(qp + 8 * g);
    qh[1] = *(const bf16x8*)(qp + 32 + 8 * g);
    dh[0] = *(const bf16x8*)(dop + 8 * g);
    dh[1] = *(const bf16x8*)(dop + 32 + 8 * g);
    const float lse2 = a.lse[tok_base + pb * kBlock + n] * kLog2e;
    if (NST > 0) {
      // stage this block's Q and dO rows for the coarse partial sums (k = query axis)
      const int row = lane >> 2;            // 16 rows, 4 lanes x 32 bytes each
      const int part = (lane & 3) * 16;
      const int prow = token_row(pb * kBlock + row, a.grid);
      const bf16* qs = a.q + (tok_base + prow) * kDim + part;
      const bf16* ds = a.dout + (tok_base + prow) * kDim + part;
      *(bf16x8*)(stQ + row * kStride + part) = *(const bf16x8*)qs;
      *(bf16x8*)(stQ + row * kStride + part + 8) = *(const bf16x8*)(qs + 8);
      *(bf16x8*)(stO + row * kStride + part) = *(const bf16x8*)ds;
      *(bf16x8*)(stO + row * kStride + part + 8) = *(const bf16x8*)(ds + 8);
    }

    const int32_t* sel1 = a.sel[0] + ((long)head * n1 + pb) * K;
    // dQ = scale * sum_e P_e (dP_e - D) k_e = scale * (A - D * Bv) with A = sum P dP k and
    // Bv = sum P k, so D = sum_e P_e dP_e is exact (no bf16 O) and one pass suffices.
    f32x4 acc_a[4], acc_b[4];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) acc_a[t4] = acc_b[t4] = f32x4{0.f, 0.f, 0.f, 0.f};
    float dpart = 0.f;           // this lane's share of D
    float pc[2][4], dpc[2][4];   // P and dP of the coarse chunk (the last one)

    for (int ch = 0; ch < n_chunks; ++ch) {
      const bool fine = ch < n_fine_chunks;
      // ---- lane kk (< 32) resolves key kk of the chunk: row, level, validity (as a mask)
      long my_row = 0;
      bool my_ok = false;
      if (fine) {
        const int kk = lane & 31;
        const int j = kk < 16 ? sel1[2 * ch] : ((2 * ch + 1 < K) ? sel1[2 * ch + 1] : -1);
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
      // ---- stage the chunk's K rows (32 rows x 128 B; pooled keys as hi + lo)
#pragma unroll
      for (int ins = 0; ins < 4; ++ins) {
        const int row = ins * 8 + (lane >> 3);
        const int piece = (lane & 7) * 8;
        const long r = row_of(row);   // cross-lane read: uniform control flow only
        const int lvl = level_of(row);
        const bool ok = (valid >> row) & 1;
        if (fine) {
          const bf16x8 kv = ok ? *(const bf16x8*)(a.k + r * kDim + piece) : zero8();
          *(bf16x8*)(stK + row * kStride + piece) = kv;
        } else {
          f32x4 k0 = {0.f, 0.f, 0.f, 0.f}, k1 = {0.f, 0.f, 0.f, 0.f};
          if (ok) {
            const float* kp = a.k_lv[lvl - 1] + r * kDim + piece;
            k0 = *(const f32x4*)kp;
            k1 = *(const f32x4*)(kp + 4);
          }
          bf16x8 hi, lo;
          split_f32x8(k0, k1, hi, lo);
          *(bf16x8*)(stK + row * kStride + piece) = hi;
          *(bf16x8*)(stKl + row * kStride + piece) = lo;
        }
      }
      wave_lds_sync();
      // ---- S^T and dP^T tiles (V rows are read straight from memory as A operands)
      float p[2][4], w1[2][4];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int arow = chunk_key(n, t);
        const bool aok = (valid >> arow) & 1;
        const long vr = row_of(arow);   // cross-lane read: uniform control flow only
        const int alvl = level_of(arow);
        f32x4 st = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
        st = mfma_bf16_k32(lds_row8(stK, arow, 0, g), qh[0], st);
        st = mfma_bf16_k32(lds_row8(stK, arow, 1, g), qh[1], st);
        if (fine) {
          bf16x8 v0 = zero8(), v1 = zero8();
          if (aok) {
            v0 = *(const bf16x8*)(a.v + vr * kDim + 8 * g);
            v1 = *(const bf16x8*)(a.v + vr * kDim + 32 + 8 * g);
          }
          dp = mfma_bf16_k32(v0, dh[0], dp);
          dp = mfma_bf16_k32(v1, dh[1], dp);
        } else {
          st = mfma_bf16_k32(lds_row8(stKl, arow, 0, g), qh[0], st);
          st = mfma_bf16_k32(lds_row8(stKl, arow, 1, g), qh[1], st);
#pragma unroll
          for (int sidx = 0; sidx < 2; ++sidx) {
            f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
            if (aok) {
              const float* vp = a.v_lv[alvl - 1] + vr * kDim + 32 * sidx + 8 * g;
              x0 = *(const f32x4*)vp;
              x1 = *(const f32x4*)(vp + 4);
            }
            bf16x8 hi, lo;
            split_f32x8(x0, x1, hi, lo);
            dp = mfma_bf16_k32(hi, dh[sidx], dp);
            dp = mfma_bf16_k32(lo, dh[sidx], dp);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kk = 8 * g + i + 4 * t;
          const bool ok = (valid >> kk) & 1;
          const float bias = fine ? 0.f : 4.0f * (float)level_of(kk);
          const float pv = ok ? exp2f(st[i] * a.c2 + bias - lse2) : 0.f;
          p[t][i] = pv;
          w1[t][i] = pv * dp[i];
          dpart += w1[t][i];
          pc[t][i] = pv;
          dpc[t][i] = dp[i];
        }
      }
      // ---- A^T += K^T (P dP)^T, Bv^T += K^T P^T  (weights as hi + lo pairs)
      bf16x8 a_hi, a_lo, b_hi, b_lo;
      split8(w1, a_hi, a_lo);
      split8(p, b_hi, b_lo);
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const bf16x8 kt = lds_tr8(stK, t4, lane);
        acc_a[t4] = mfma_bf16_k32(kt, a_hi, acc_a[t4]);
        acc_a[t4] = mfma_bf16_k32(kt, a_lo, acc_a[t4]);
        acc_b[t4] = mfma_bf16_k32(kt, b_hi, acc_b[t4]);
        acc_b[t4] = mfma_bf16_k32(kt, b_lo, acc_b[t4]);
        if (!fine) {
          const bf16x8 ktl = lds_tr8(stKl, t4, lane);
          acc_a[t4] = mfma_bf16_k32(ktl, a_hi, acc_a[t4]);
          acc_b[t4] = mfma_bf16_k32(ktl, b_hi, acc_b[t4]);
        }
      }
      wave_lds_sync();
    }
    const float Dn = group4_sum(dpart);
    if (g == 0) a.dd[tok_base + pb * kBlock + n] = Dn;
    // ---- write dQ (lane holds dQ[n][16 t4 + 4g + i])
    bf16* dqp = a.dq + (tok_base + qrow) * kDim;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      bf16x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = (bf16)((acc_a[t4][i] - Dn * acc_b[t4][i]) * a.scale);
      *(bf16x4*)(dqp + 16 * t4 + 4 * g) = r;
    }

    if (NST > 0) {
      // ---- coarse partials over this block's 16 queries: dV_c += P^T dO, dK_c += dS^T Q,
      // with dS = P (dP - D) of the coarse chunk (the last chunk, still in registers)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kk = 8 * g + i + 4 * t;
          const float dsv = pc[t][i] * (dpc[t][i] - Dn);
          const bf16 ph = (bf16)pc[t][i];
          const bf16 sh = (bf16)dsv;
          stP[kk * 16 + n] = ph;
          stPl[kk * 16 + n] = (bf16)(pc[t][i] - (float)ph);
          stS[kk * 16 + n] = sh;
          stSl[kk * 16 + n] = (bf16)(dsv - (float)sh);
        }
      wave_lds_sync();
      const int r = (lane & 15) >> 2;
      const int c = lane & 3;
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const int at = (16 * st + n) * 16 + 4 * g;
        const bf16x4 pa = *(const bf16x4*)(stP + at);
        const bf16x4 pl = *(const bf16x4*)(stPl + at);
        const bf16x4 sa = *(const bf16x4*)(stS + at);
        const bf16x4 sl = *(const bf16x4*)(stSl + at);
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
          const bf16x4 dob = lds_read_tr16(stO + (4 * g + r) * kStride + 16 * t4 + 4 * c);
          const bf16x4 qbt = lds_read_tr16(stQ + (4 * g + r) * kStride + 16 * t4 + 4 * c);
          cpv[st][t4] = mfma_bf16_k16(pa, dob, cpv[st][t4]);
          cpv[st][t4] = mfma_bf16_k16(pl, dob, cpv[st][t4]);
          cpk[st][t4] = mfma_bf16_k16(sa, qbt, cpk[st][t4]);
          cpk[st][t4] = mfma_bf16_k16(sl, qbt, cpk[st][t4]);
        }
      }
      wave_lds_sync();
    }
  }

  if (NST > 0) {
    // ---- reduce the four waves' coarse partials (in wave order 0..3) and store them for this
    // level-2 group.  cp*[st][t4][i] at lane (n, g) is slot 16 st + 4g + i, channel 16 t4 + n.
    float* red = (float*)&sK[0][0];   // reuses the K staging: 2 x NST x 16 x 64 floats <= 16 KB
    const int half = NST * 16 * kDim;
    for (int turn = 0; turn < 4; ++turn) {
      __syncthreads();
      if (w == turn) {
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
          for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int e = (16 * st + 4 * g + i) * kDim + 16 * t4 + n;
              red[e] = (turn ? red[e] : 0.f) + cpk[st][t4][i];
              red[half + e] = (turn ? red[half + e] : 0.f) + cpv[st][t4][i];
            }
      }
    }
    __syncthreads();
    const long out_base = ((long)head * n2 + a2) * n_coarse * kDim;
    for (int e = threadIdx.x; e < half; e += 256) {
      if (e / kDim >= n_coarse) continue;
      a.part_k[out_base + e] = red[e] * a.scale;
      a.part_v[out_base + e] = red[half + e];
    }
  }
}

// ====================================================================== stage 2: coarse keys
// Level l >= 3: sum the level-2 group partials of the 16^(l-2) groups under each ancestor.
__global__ __launch_bounds__(256) void coarse_reduce_kernel(BwdArgs a, int l) {
  const int K = a.topk;
  const int n2 = a.n >> (2 * kBlockShift);
  const int nl = a.n >> (kBlockShift * l);
  const int span = 1 << (kBlockShift * (l - 2));
  const int n_coarse = (a.levels - 1) * K;
  const long total = (long)a.bh * nl * K * kDim;
  const long e = (long)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  const int ch = (int)(e % kDim);
  const long rest = e / kDim;
  const int slot = (int)(rest % K);
  const long anc_g = rest / K;            // head * nl + anc
  const int head = (int)(anc_g / nl);
  const int anc = (int)(anc_g - (long)head * nl);
  const int pslot = (l - 2) * K + slot;
  float sk = 0.f, sv = 0.f;
  for (int c = 0; c < span; ++c) {
    const long src = (((long)head * n2 + anc * span + c) * n_coarse + pslot) * kDim + ch;
    sk += a.part_k[src];
    sv += a.part_v[src];
  }
  a.lvl_part_k[l - 1][e] = sk;
  a.lvl_part_v[l - 1][e] = sv;
}

// dK_l[j] = sum over ancestors a in CSC_l[j] of partial(a, slot of j in Sel_l[a]).
// One wave per coarse key; lane = channel.
__global__ __launch_bounds__(256) void coarse_grad_kernel(BwdArgs a, int l) {
  const int K = a.topk;
  const int nl = a.n >> (kBlockShift * l);
  const long wave = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int ch = threadIdx.x & 63;
  if (wave >= (long)a.bh * nl) return;
  const int head = (int)(wave / nl);
  const int j = (int)(wave - (long)head * nl);
  const int n_coarse = (a.levels - 1) * K;
  const int32_t* off = a.csc_off[l - 1] + (long)head * (nl + 1);
  const int32_t* rows = a.csc_rows[l - 1] + (long)head * nl * K;
  const int32_t* sel = a.sel[l - 1] + (long)head * nl * K;
  const int e0 = off[j], e1 = off[j + 1];
  float sk = 0.f, sv = 0.f;
  for (int e = e0; e < e1; ++e) {
    const int anc = rows[e];
    if (anc < 0 || anc >= nl) continue;
    int slot = -1;
    for (int s = 0; s < K; ++s)
      if (sel[(long)anc * K + s] == j) slot = s;
    if (slot < 0) continue;
    long src;
    const float* pk;
    const float* pv;
    if (l == 2) {
      src = (((long)head * nl + anc) * n_coarse + slot) * kDim + ch;
      pk = a.part_k;
      pv = a.part_v;
    } else {
      src = (((long)head * nl + anc) * K + slot) * kDim + ch;
      pk = a.lvl_part_k[l - 1];
      pv = a.lvl_part_v[l - 1];
    }
    sk += pk[src];
    sv += pv[src];
  }
  a.dk_lv[l - 1][((long)head * nl + j) * kDim + ch] = sk;
  a.dv_lv[l - 1][((long)head * nl + j) * kDim + ch] = sv;
}

// ====================================================================== stage 3: key-major
__global__ __launch_bounds__(256) void bwd_key_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 sQ[4][32 * kStride];
  __shared__ __attribute__((aligned(16))) bf16 sO[4][32 * kStride];   // dO rows
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int n1 = a.n >> kBlockShift;
  const long kb = (long)xcd_block(blockIdx.x, gridDim.x) * 4 + w;
  if (kb >= (long)a.bh * n1) return;
  const int head = (int)(kb / n1);
  const int j = (int)(kb - (long)head * n1);
  const long tok_base = (long)head * a.n;
  bf16* stQ = sQ[w];
  bf16* stO = sO[w];

  // keys of this block as B operands: lane (n, g) holds row n, channels 32s + 8g .. +7
  const int krow = token_row(j * kBlock + n, a.grid);
  const bf16* kp = a.k + (tok_base + krow) * kDim;
  const bf16* vp = a.v + (tok_base + krow) * kDim;
  bf16x8 kh[2], vh[2];
  kh[0] = *(const bf16x8*)(kp + 8 * g);
  kh[1] = *(const bf16x8*)(kp + 32 + 8 * g);
  vh[0] = *(const bf16x8*)(vp + 8 * g);
  vh[1] = *(const bf16x8*)(vp + 32 + 8 * g);

  const int32_t* off = a.csc_off[0] + (long)head * (n1 + 1);
  const int32_t* rows = a.csc_rows[0] + (long)head * n1 * a.topk;
  const int e0 = off[j], e1 = off[j + 1];
  f32x4 dka[4], dva[4];
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4) dka[t4] = dva[t4] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int e = e0; e < e1; e += 2) {
    const int pA = rows[e];
    const int pB = (e + 1 < e1) ? rows[e + 1] : -1;
    const bool okA = pA >= 0 && pA < n1;
    const bool okB = pB >= 0 && pB < n1;
    // ---- stage the pair's Q and dO rows: query position qq = 16*(which) + token
#pragma unroll
    for (int ins = 0; ins < 4; ++ins) {
      const int row = ins * 8 + (lane >> 3);
      const int piece = (lane & 7) * 8;
      const int pblk = row < 16 ? pA : pB;
      const bool ok = row < 16 ? okA : okB;
      bf16x8 qv = zero8(), dv = zero8();
      if (ok) {
        const long r = tok_base + token_row(pblk * kBlock + (row & 15), a.grid);
        qv = *(const bf16x8*)(a.q + r * kDim + piece);
        dv = *(const bf16x8*)(a.dout + r * kDim + piece);
      }
      *(bf16x8*)(stQ + row * kStride + piece) = qv;
      *(bf16x8*)(stO + row * kStride + piece) = dv;
    }
    wave_lds_sync();
    // ---- S and dP tiles (queries x keys): lane (n, g) holds queries 8g + i + 4t, key n
    float p[2][4], dsv[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int arow = chunk_key(n, t);
      f32x4 st = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
      st = mfma_bf16_k32(lds_row8(stQ, arow, 0, g), kh[0], st);
      st = mfma_bf16_k32(lds_row8(stQ, arow, 1, g), kh[1], st);
      dp = mfma_bf16_k32(lds_row8(stO, arow, 0, g), vh[0], dp);
      dp = mfma_bf16_k32(lds_row8(stO, arow, 1, g), vh[1], dp);
      // queries 8g + 4t + i, i = 0..3: four consecutive tokens of one block
      const int qq = 8 * g + 4 * t;
      const int pblk = qq < 16 ? pA : pB;
      const bool ok = qq < 16 ? okA : okB;
      f32x4 l4 = {0.f, 0.f, 0.f, 0.f}, d4 = {0.f, 0.f, 0.f, 0.f};
      if (ok) {
        const long mpos = tok_base + pblk * kBlock + (qq & 15);
        l4 = *(const f32x4*)(a.lse + mpos);
        d4 = *(const f32x4*)(a.dd + mpos);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = ok ? exp2f(st[i] * a.c2 - l4[i] * kLog2e) : 0.f;
        p[t][i] = pv;
        dsv[t][i] = pv * (dp[i] - d4[i]);
      }
    }
    bf16x8 p_hi, p_lo, ds_hi, ds_lo;
    split8(p, p_hi, p_lo);
    split8(dsv, ds_hi, ds_lo);
    // ---- dV^T += dO^T P, dK^T += Q^T dS  (contract over the pair's 32 queries)
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      const bf16x8 ot = lds_tr8(stO, t4, lane);
      const bf16x8 qt = lds_tr8(stQ, t4, lane);
      dva[t4] = mfma_bf16_k32(ot, p_hi, dva[t4]);
      dva[t4] = mfma_bf16_k32(ot, p_lo, dva[t4]);
      dka[t4] = mfma_bf16_k32(qt, ds_hi, dka[t4]);
      dka[t4] = mfma_bf16_k32(qt, ds_lo, dka[t4]);
    }
    wave_lds_sync();
  }

  // ---- push-down of pooled-key gradients and store (lane holds key n, channels 16t4+4g+i)
  float pdk[4][4], pdv[4][4];
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
    for (int i = 0; i < 4; ++i) pdk[t4][i] = pdv[t4][i] = 0.f;
  if (a.enrich) {
    for (int l = 2; l <= a.levels; ++l) {
      const int nl = a.n >> (kBlockShift * l);
      const int anc = j >> (kBlockShift * (l - 1));
      const float f = 1.0f / (float)(1 << (kBlockShift * l));
      const float* gk = a.dk_lv[l - 1] + ((long)head * nl + anc) * kDim;
      const float* gv = a.dv_lv[l - 1] + ((long)head * nl + anc) * kDim;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const f32x4 k4 = *(const f32x4*)(gk + 16 * t4 + 4 * g);
        const f32x4 v4 = *(const f32x4*)(gv + 16 * t4 + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pdk[t4][i] += k4[i] * f;
          pdv[t4][i] += v4[i] * f;
        }
      }
    }
  }
  bf16* dkp = a.dk + (tok_base + krow) * kDim;
  bf16* dvp = a.dv + (tok_base + krow) * kDim;
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4) {
    bf16x4 rk, rv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rk[i] = (bf16)(dka[t4][i] * a.scale + pdk[t4][i]);
      rv[i] = (bf16)(dva[t4][i] + pdv[t4][i]);
    }
    *(bf16x4*)(dkp + 16 * t4 + 4 * g) = rk;
    *(bf16x4*)(dvp + 16 * t4 + 4 * g) = rv;
  }
}

// ====================================================================== host side
struct BwdLayout {
  size_t dd, part_k, part_v, lvl_k[kMaxLv], lvl_v[kMaxLv], dk_lv[kMaxLv], dv_lv[kMaxLv], total;
};

static BwdLayout bwd_layout(const Shape& s) {
  BwdLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) & ~(size_t)255;
    return at;
  };
  L.dd = take(sizeof(float) * (size_t)s.bh * s.n);
  if (s.enrich && s.levels >= 2) {
    const size_t n2 = (size_t)s.n_level(2);
    const size_t nc = (size_t)(s.levels - 1) * s.topk;
    L.part_k = take(sizeof(float) * s.bh * n2 * nc * kDim);
    L.part_v = take(sizeof(float) * s.bh * n2 * nc * kDim);
    for (int l = 2; l <= s.levels; ++l) {
      const size_t nl = (size_t)s.n_level(l);
      if (l >= 3) {
        L.lvl_k[l - 1] = take(sizeof(float) * s.bh * nl * s.topk * kDim);
        L.lvl_v[l - 1] = take(sizeof(float) * s.bh * nl * s.topk * kDim);
      }
      L.dk_lv[l - 1] = take(sizeof(float) * s.bh * nl * kDim);
      L.dv_lv[l - 1] = take(sizeof(float) * s.bh * nl * kDim);
    }
  }
  L.total = off;
  return L;
}

size_t bwd_workspace_bytes(const Shape& s) { return bwd_layout(s).total; }

hipError_t launch_attn_bwd(const Shape& s, const void* q, const void* k, const void* v,
                           const void* dout, const float* lse,
                           const float* const* k_lv, const float* const* v_lv,
                           const int32_t* const* sel, const int32_t* const* csc_off,
                           const int32_t* const* csc_rows, void* dq, void* dk, void* dv,
                           void* ws, hipStream_t stream) {
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
  const bool coarse = s.enrich && s.levels >= 2;
  if (coarse) {
    a.part_k = (float*)(base + L.part_k);
    a.part_v = (float*)(base + L.part_v);
    for (int l = 2; l <= s.levels; ++l) {
      if (l >= 3) {
        a.lvl_part_k[l - 1] = (float*)(base + L.lvl_k[l - 1]);
        a.lvl_part_v[l - 1] = (float*)(base + L.lvl_v[l - 1]);
      }
      a.dk_lv[l - 1] = (float*)(base + L.dk_lv[l - 1]);
      a.dv_lv[l - 1] = (float*)(base + L.dv_lv[l - 1]);
    }
  }
  a.bh = s.bh;
  a.n = s.n;
  a.grid = Grid{s.hbits, s.wbits, s.raster};
  a.levels = s.levels;
  a.topk = s.topk;
  a.enrich = coarse ? 1 : 0;
  a.scale = s.scale;
  a.c2 = s.scale * kLog2e;

  const int n2 = s.n >> (2 * kBlockShift);
  const unsigned qblocks = (unsigned)(s.bh * n2);
  const int n_coarse = coarse ? (s.levels - 1) * s.topk : 0;
  if (n_coarse == 0)
    hipLaunchKernelGGL(bwd_query_kernel<0>, dim3(qblocks), dim3(256), 0, stream, a);
  else if (n_coarse <= 16)
    hipLaunchKernelGGL(bwd_query_kernel<1>, dim3(qblocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(bwd_query_kernel<2>, dim3(qblocks), dim3(256), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (coarse) {
    for (int l = 3; l <= s.levels; ++l) {
      const long total = (long)s.bh * s.n_level(l) * s.topk * kDim;
      hipLaunchKernelGGL(coarse_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256),
                         0, stream, a, l);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    for (int l = 2; l <= s.levels; ++l) {
      const long waves = (long)s.bh * s.n_level(l);
      hipLaunchKernelGGL(coarse_grad_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                         stream, a, l);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
  }
  const long kwaves = (long)s.bh * (s.n >> kBlockShift);
  hipLaunchKernelGGL(bwd_key_kernel, dim3((unsigned)((kwaves + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace llsa
