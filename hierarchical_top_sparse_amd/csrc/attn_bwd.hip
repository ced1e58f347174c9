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
//  3. bwd_key_kernel (key-major, one one-wave workgroup per level-1 key block): walks the
//     query blocks in CSC_1[j] two at a time, accumulates dK, dV on the MFMA, and adds the
//     pooled gradients pushed down to the block's tokens (dK_l[ancestor] / 16^l, chain rule
//     of the mean).
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
// LDS layout (bf16 elements): per wave, a 32-row staging tile (K rows of a fine chunk; after the
// chunk loop the block's Q and dO rows for the coarse partial sums) and four 32x16 tiles (P^T,
// dS^T as hi + lo); then, shared by the workgroup, the coarse keys/values of its level-2
// group: K hi, K lo, V hi, V lo (32 rows each) and the 32 slot biases (fp32).
constexpr int kQStage = 32 * kStride;
constexpr int kQPd = 4 * 32 * 16;
constexpr int kQPerWave = kQStage + kQPd;
static size_t bwd_query_lds_bytes(bool coarse) {
  return sizeof(bf16) * (size_t)(4 * kQPerWave + (coarse ? 4 * kQStage : 0)) +
         (coarse ? 32 * sizeof(float) : 0);
}

template <int NST>   // coarse slot tiles (of 16) kept in registers: 0, 1 or 2
__global__ __launch_bounds__(256) void bwd_query_kernel(BwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16* lds = (bf16*)smem;
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int n = lane & 15;
  const int g = lane >> 4;
  const int n1 = a.n >> kBlockShift;
  const int n2 = n1 >> kBlockShift;
  const int wg = uniform(xcd_block(blockIdx.x, gridDim.x));
  const int head = uniform(wg / n2);
  const int a2 = uniform(wg - head * n2);
  const int K = a.topk;
  const long tok_base = (long)head * a.n;
  const int n_coarse = NST > 0 ? (a.levels - 1) * K : 0;
  bf16* stK = lds + w * kQPerWave;            // K rows of a chunk / Q and dO rows of a block
  bf16* stP = stK + kQStage;                  // P^T hi, P^T lo, dS^T hi, dS^T lo: [slot][q]
  bf16* cK = lds + 4 * kQPerWave;             // shared coarse K hi (+kQStage: lo)
  bf16* cV = cK + 2 * kQStage;                // shared coarse V hi (+kQStage: lo)
  float* cbias = (float*)(cK + 4 * kQStage);

  const uint32_t head_bytes = (uint32_t)a.n * kDim * 2;
  const rsrc_t rq = make_rsrc_uniform((const char*)a.q + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rk = make_rsrc_uniform((const char*)a.k + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rv = make_rsrc_uniform((const char*)a.v + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rdo =
      make_rsrc_uniform((const char*)a.dout + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rl = make_rsrc_uniform(a.lse + tok_base, (uint32_t)a.n * 4);

  // The wave's four query blocks pb_first + b, b = 0..3, form one stream of 4 * n_fine fine
  // chunks; the loads of the next chunk are always issued before the current one is computed.
  const int pb_first = a2 * kBlock + w * 4;
  const int n_fine = (K + 1) >> 1;
  // picks as a lane-held table: lane 16b + i holds the first-row byte offset of pick i of
  // block b (kNoRow for i >= K and for an invalid id); chunks take them with v_readlane
  uint32_t pick_off = kNoRow;
  if ((lane & 15) < K) {
    const int j = a.sel[0][((long)head * n1 + pb_first + (lane >> 4)) * K + (lane & 15)];
    if (j >= 0 && j < n1) pick_off = (uint32_t)block_corner(j, a.grid) * kDim * 2;
  }

  // lane-constant byte offsets inside a 4x4 block: staged rows and A-operand rows
  const int srow0 = lane >> 3;
  const int piece = lane & 7;
  uint32_t st_off[4];
#pragma unroll
  for (int ins = 0; ins < 4; ++ins)
    st_off[ins] = (uint32_t)(tile_offset((ins * 8 + srow0) & 15, a.grid) * kDim * 2 + 16 * piece);
  uint32_t va_off[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
    va_off[t] = (uint32_t)(tile_offset(chunk_key(n, t) & 15, a.grid) * kDim * 2) + 16 * g;
  const bool a_second = n >= 8;     // A rows 8..15 of both tiles come from the second block
  const bool lane_second = g >= 2;  // this lane's 8 keys come from the second block

  // rows of one query block: Q and dO as B operands (lane (n, g): row n, channels 32s + 8g..)
  // and the row's LSE (natural log, as stored)
  struct BlockLd {
    bf16x8 q[2], d[2];
    float lse;
  };
  auto load_block = [&](int b) -> BlockLd {
    BlockLd r;
    const int pb = pb_first + b;
    const int qrow = block_corner(pb, a.grid) + tile_offset(n, a.grid);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      r.q[s] = buf_load8(rq, (uint32_t)(qrow * kDim + 32 * s + 8 * g) * 2);
      r.d[s] = buf_load8(rdo, (uint32_t)(qrow * kDim + 32 * s + 8 * g) * 2);
    }
    r.lse = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rl, (uint32_t)(pb * kBlock + n) * 4, 0, 0));
    return r;
  };

  struct FineLd {
    i32x4 k[4];      // staged K rows
    i32x4 v[2][2];   // V rows as A operands of dP^T
    int ok0, ok1;
  };
  int lb = 0, lch = 0;   // block and chunk of the next load (lb == 4: past the end)
  // Every call issues the same loads, also past the last chunk (kNoRow: zeros, no memory
  // access), so the wait before a chunk's use never drains the loads queued behind it.
  auto load_next = [&]() -> FineLd {
    FineLd f;
    const int idx = min(16 * lb + 2 * lch, 62);
    uint32_t b0 = (uint32_t)__builtin_amdgcn_readlane((int)pick_off, idx);
    uint32_t b1 = (uint32_t)__builtin_amdgcn_readlane((int)pick_off, idx + 1);
    if (lb >= 4) b0 = b1 = kNoRow;
    f.ok0 = b0 != kNoRow;
    f.ok1 = b1 != kNoRow;
#pragma unroll
    for (int ins = 0; ins < 4; ++ins)
      f.k[ins] = __builtin_amdgcn_raw_buffer_load_b128(rk, (ins >= 2 ? b1 : b0) + st_off[ins],
                                                       0, 0);
    const uint32_t vb = a_second ? b1 : b0;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        f.v[t][s] = __builtin_amdgcn_raw_buffer_load_b128(rv, vb + va_off[t] + 64 * s, 0, 0);
    if (++lch == n_fine) {
      lch = 0;
      ++lb;
    }
    return f;
  };

  BlockLd cur = load_block(0), nxt;
  FineLd fa = load_next(), fb;

  if (NST > 0) {
    // ---- the group's coarse keys/values (all 256 queries of the level-2 group share them);
    // their loads overlap the first chunk's
    const int pb0 = a2 * kBlock;
    const int e = threadIdx.x;             // 32 slots x 8 pieces of 8 channels
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
    bf16x8 hi, lo;
    split_f32x8(k0, k1, hi, lo);
    *(bf16x8*)(cK + slot * kStride + c8) = hi;
    *(bf16x8*)(cK + kQStage + slot * kStride + c8) = lo;
    split_f32x8(v0, v1, hi, lo);
    *(bf16x8*)(cV + slot * kStride + c8) = hi;
    *(bf16x8*)(cV + kQStage + slot * kStride + c8) = lo;
    if (c8 == 0) cbias[slot] = bias;
    __syncthreads();
  }

  f32x4 cpk[NST > 0 ? NST : 1][4];   // coarse partial dK (unscaled): [slot tile][d tile]
  f32x4 cpv[NST > 0 ? NST : 1][4];
#pragma unroll
  for (int st = 0; st < (NST > 0 ? NST : 1); ++st)
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) cpk[st][t4] = cpv[st][t4] = f32x4{0.f, 0.f, 0.f, 0.f};

  // dQ = scale * sum_e P_e (dP_e - D) k_e = scale * (A - D * Bv) with A = sum P dP k and
  // Bv = sum P k, so D = sum_e P_e dP_e is exact (no bf16 O) and one pass suffices.
  f32x4 acc_a[4], acc_b[4];
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4) acc_a[t4] = acc_b[t4] = f32x4{0.f, 0.f, 0.f, 0.f};
  float dpart = 0.f;           // this lane's share of D
  float pc[2][4], dpc[2][4];   // P and dP of the coarse chunk

  // P, P dP of one chunk from its S^T / dP^T tiles; A/B accumulation on the MFMA
  auto absorb = [&](const f32x4 (&st)[2], const f32x4 (&dp)[2], const float (&add)[2][4],
                    const bf16* kt_hi, const bf16* kt_lo, bool keep) {
    float p[2][4], w1[2][4];
    const float lse2 = cur.lse * kLog2e;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = fast_exp2(fmaf(st[t][i], a.c2, add[t][i] - lse2));
        p[t][i] = pv;
        w1[t][i] = pv * dp[t][i];
        dpart += w1[t][i];
        if (keep) {
          pc[t][i] = pv;
          dpc[t][i] = dp[t][i];
        }
      }
    bf16x8 a_hi, a_lo, b_hi, b_lo;
    split8(w1, a_hi, a_lo);
    split8(p, b_hi, b_lo);
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      const bf16x8 kt = lds_tr8(kt_hi, t4, lane);
      acc_a[t4] = mfma_bf16_k32(kt, a_hi, acc_a[t4]);
      acc_a[t4] = mfma_bf16_k32(kt, a_lo, acc_a[t4]);
      acc_b[t4] = mfma_bf16_k32(kt, b_hi, acc_b[t4]);
      acc_b[t4] = mfma_bf16_k32(kt, b_lo, acc_b[t4]);
      if (kt_lo) {
        const bf16x8 ktl = lds_tr8(kt_lo, t4, lane);
        acc_a[t4] = mfma_bf16_k32(ktl, a_hi, acc_a[t4]);
        acc_b[t4] = mfma_bf16_k32(ktl, b_hi, acc_b[t4]);
      }
    }
  };

  auto fine_chunk = [&](const FineLd& f) {
#pragma unroll
    for (int ins = 0; ins < 4; ++ins)
      *(i32x4*)(stK + (ins * 8 + srow0) * kStride + 8 * piece) = f.k[ins];
    wave_lds_sync();
    f32x4 st[2], dp[2];
    float add[2][4];
    const float madd = (lane_second ? f.ok1 : f.ok0) ? 0.f : -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int arow = chunk_key(n, t);
      st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      dp[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      st[t] = mfma_bf16_k32(lds_row8(stK, arow, 0, g), cur.q[0], st[t]);
      st[t] = mfma_bf16_k32(lds_row8(stK, arow, 1, g), cur.q[1], st[t]);
      dp[t] = mfma_bf16_k32(*(const bf16x8*)&f.v[t][0], cur.d[0], dp[t]);
      dp[t] = mfma_bf16_k32(*(const bf16x8*)&f.v[t][1], cur.d[1], dp[t]);
#pragma unroll
      for (int i = 0; i < 4; ++i) add[t][i] = madd;
    }
    absorb(st, dp, add, stK, nullptr, false);
    wave_lds_sync();
  };

  // the end of query block b: its coarse chunk, D, dQ and its share of the coarse partials
  auto block_end = [&](int b) {
    const int pb = pb_first + b;
    const int qrow = block_corner(pb, a.grid) + tile_offset(n, a.grid);
    if (NST > 0) {
      f32x4 st[2], dp[2];
      float add[2][4];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int arow = chunk_key(n, t);
        st[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          st[t] = mfma_bf16_k32(lds_row8(cK, arow, s, g), cur.q[s], st[t]);
          st[t] = mfma_bf16_k32(lds_row8(cK + kQStage, arow, s, g), cur.q[s], st[t]);
          dp[t] = mfma_bf16_k32(lds_row8(cV, arow, s, g), cur.d[s], dp[t]);
          dp[t] = mfma_bf16_k32(lds_row8(cV + kQStage, arow, s, g), cur.d[s], dp[t]);
        }
        const f32x4 b4 = *(const f32x4*)(cbias + 8 * g + 4 * t);
#pragma unroll
        for (int i = 0; i < 4; ++i) add[t][i] = b4[i];
      }
      absorb(st, dp, add, cK, cK + kQStage, true);
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
      // with dS = P (dP - D).  The staging tile takes the block's Q rows (0..15) and dO rows
      // (16..31) from the B-operand registers (lane (n, g) holds row n, channels 32s + 8g..).
      bf16* stQ = stK;
      bf16* stO = stK + 16 * kStride;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        *(bf16x8*)(stQ + n * kStride + 32 * s + 8 * g) = cur.q[s];
        *(bf16x8*)(stO + n * kStride + 32 * s + 8 * g) = cur.d[s];
      }
      bf16* pH = stP;
      bf16* pL = stP + 512;
      bf16* sH = stP + 1024;
      bf16* sL = stP + 1536;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kk = 8 * g + i + 4 * t;
          const float dsv = pc[t][i] * (dpc[t][i] - Dn);
          const bf16 ph = (bf16)pc[t][i];
          const bf16 sh = (bf16)dsv;
          pH[kk * 16 + n] = ph;
          pL[kk * 16 + n] = (bf16)(pc[t][i] - (float)ph);
          sH[kk * 16 + n] = sh;
          sL[kk * 16 + n] = (bf16)(dsv - (float)sh);
        }
      wave_lds_sync();
      const int r = (lane & 15) >> 2;
      const int c = lane & 3;
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const int at = (16 * st + n) * 16 + 4 * g;
        const bf16x4 pa = *(const bf16x4*)(pH + at);
        const bf16x4 pl = *(const bf16x4*)(pL + at);
        const bf16x4 sa = *(const bf16x4*)(sH + at);
        const bf16x4 sl = *(const bf16x4*)(sL + at);
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
    dpart = 0.f;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) acc_a[t4] = acc_b[t4] = f32x4{0.f, 0.f, 0.f, 0.f};
  };

  // one step of the stream: (next block's rows,) next chunk's loads, then chunk `f`; returns
  // false after the last block.  Two call sites alternate the load buffers (no copies).
  int cb = 0, cch = 0;   // block and chunk being computed
  auto step = [&](const FineLd& f, FineLd& refill) -> bool {
    // the next block's rows are loaded before the chunk loads so that waiting for them
    // (conditional loads) never drains the chunk prefetch
    if (lch == 0 && lb > 0 && lb < 4) nxt = load_block(lb);
    refill = load_next();
    fine_chunk(f);
    if (++cch < n_fine) return true;
    block_end(cb);
    cch = 0;
    if (++cb == 4) return false;
    cur = nxt;
    return true;
  };
  while (step(fa, fb) && step(fb, fa)) {
  }

  if (NST > 0) {
    // ---- reduce the four waves' coarse partials (in wave order 0..3) and store them for this
    // level-2 group.  cp*[st][t4][i] at lane (n, g) is slot 16 st + 4g + i, channel 16 t4 + n.
    float* red = (float*)cK;   // the shared coarse copy is no longer needed: 16 KB >= 2 x NST KB x 4
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
// One wave per coarse key.  Lanes first resolve up to 64 CSC entries at once (ancestor and
// slot), then every lane (= channel) sums the partial rows in CSC order.
__global__ __launch_bounds__(256) void coarse_grad_kernel(BwdArgs a, int l) {
  const int K = a.topk;
  const int nl = a.n >> (kBlockShift * l);
  const int wave = uniform((int)(blockIdx.x * 4) + (int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  if (wave >= a.bh * nl) return;
  const int head = uniform(wave / nl);
  const int j = uniform(wave - head * nl);
  const int n_coarse = (a.levels - 1) * K;
  const int32_t* off = a.csc_off[l - 1] + (long)head * (nl + 1);
  const int32_t* rows = a.csc_rows[l - 1] + (long)head * nl * K;
  const int32_t* sel = a.sel[l - 1] + (long)head * nl * K;
  const float* pk = l == 2 ? a.part_k : a.lvl_part_k[l - 1];
  const float* pv = l == 2 ? a.part_v : a.lvl_part_v[l - 1];
  const int row_len = l == 2 ? n_coarse : K;   // slots per ancestor in the partial arrays
  const int e0 = uniform(off[j]);
  const int e1 = uniform(off[j + 1]);
  float sk = 0.f, sv = 0.f;
  for (int base = e0; base < e1; base += 64) {
    const int e = base + lane;
    long src = -1;
    if (e < e1) {
      const int anc = rows[e];
      if (anc >= 0 && anc < nl) {
        int slot = -1;
        for (int s = 0; s < K; ++s)
          if (sel[(long)anc * K + s] == j) slot = s;
        if (slot >= 0) src = (((long)head * nl + anc) * row_len + slot) * kDim;
      }
    }
    const int cnt = min(64, e1 - base);
    for (int i = 0; i < cnt; ++i) {
      const long r = __shfl(src, i, 64);   // uniform control flow
      if (r >= 0) {
        sk += pk[r + lane];
        sv += pv[r + lane];
      }
    }
  }
  a.dk_lv[l - 1][((long)head * nl + j) * kDim + lane] = sk;
  a.dv_lv[l - 1][((long)head * nl + j) * kDim + lane] = sv;
}

// ====================================================================== stage 3: key-major
// One wave per workgroup: key blocks differ widely in how many query blocks picked them, so a
// wave that finishes early frees its slot at once.
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void bwd_key_kernel(
    BwdArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 stQ[32 * kStride];
  __shared__ __attribute__((aligned(16))) bf16 stO[32 * kStride];   // dO rows
  const int lane = threadIdx.x;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int n1 = a.n >> kBlockShift;
  const int kb = uniform(xcd_block(blockIdx.x, gridDim.x));
  const int head = uniform(kb / n1);
  const int j = uniform(kb - head * n1);
  const long tok_base = (long)head * a.n;

  const uint32_t head_bytes = (uint32_t)a.n * kDim * 2;
  const rsrc_t rq = make_rsrc_uniform((const char*)a.q + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rk = make_rsrc_uniform((const char*)a.k + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rv = make_rsrc_uniform((const char*)a.v + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rdo =
      make_rsrc_uniform((const char*)a.dout + (size_t)head * head_bytes, head_bytes);
  const rsrc_t rl = make_rsrc_uniform(a.lse + tok_base, (uint32_t)a.n * 4);
  const rsrc_t rd = make_rsrc_uniform(a.dd + tok_base, (uint32_t)a.n * 4);

  // keys of this block as B operands: lane (n, g) holds row n, channels 32s + 8g .. +7
  const int krow = block_corner(j, a.grid) + tile_offset(n, a.grid);
  bf16x8 kh[2], vh[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    kh[s] = buf_load8(rk, (uint32_t)(krow * kDim + 32 * s + 8 * g) * 2);
    vh[s] = buf_load8(rv, (uint32_t)(krow * kDim + 32 * s + 8 * g) * 2);
  }

  // lane-constant offsets: staged rows (bytes) and this lane's 4 queries per tile (tokens)
  const int srow0 = lane >> 3;
  const int piece = lane & 7;
  uint32_t st_off[4];
#pragma unroll
  for (int ins = 0; ins < 4; ++ins)
    st_off[ins] = (uint32_t)(tile_offset((ins * 8 + srow0) & 15, a.grid) * kDim * 2 + 16 * piece);
  const bool lane_second = g >= 2;   // this lane's queries come from the second block

  const int32_t* off = a.csc_off[0] + (long)head * (n1 + 1);
  const int32_t* rows = a.csc_rows[0] + (long)head * n1 * a.topk;
  const int e0 = uniform(off[j]);
  const int e1 = uniform(off[j + 1]);

  struct PairLd {
    i32x4 q[4], d[4];   // staged Q and dO rows
    f32x4 l4[2], d4[2];  // lse and D of this lane's queries (tile t: tokens 8g+4t .. +3)
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
#pragma unroll
    for (int ins = 0; ins < 4; ++ins) {
      const uint32_t o = (ins >= 2 ? bB : bA) + st_off[ins];
      f.q[ins] = __builtin_amdgcn_raw_buffer_load_b128(rq, o, 0, 0);
      f.d[ins] = __builtin_amdgcn_raw_buffer_load_b128(rdo, o, 0, 0);
    }
    const uint32_t tl = lane_second ? tB : tA;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t o = tl + (uint32_t)(((8 * g + 4 * t) & 15) * 4);
      f.l4[t] = buf_load4f(rl, o);
      f.d4[t] = buf_load4f(rd, o);
    }
    return f;
  };

  f32x4 dka[4], dva[4];
#pragma unroll
  for (int t4 = 0; t4 < 4; ++t4) dka[t4] = dva[t4] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto pair = [&](const PairLd& f) {
#pragma unroll
    for (int ins = 0; ins < 4; ++ins) {
      *(i32x4*)(stQ + (ins * 8 + srow0) * kStride + 8 * piece) = f.q[ins];
      *(i32x4*)(stO + (ins * 8 + srow0) * kStride + 8 * piece) = f.d[ins];
    }
    wave_lds_sync();
    // S and dP tiles (queries x keys): lane (n, g) holds queries 8g + i + 4t, key n
    const float madd = (lane_second ? f.okB : f.okA) ? 0.f : -INFINITY;
    float p[2][4], dsv[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int arow = chunk_key(n, t);
      f32x4 st = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
      st = mfma_bf16_k32(lds_row8(stQ, arow, 0, g), kh[0], st);
      st = mfma_bf16_k32(lds_row8(stQ, arow, 1, g), kh[1], st);
      dp = mfma_bf16_k32(lds_row8(stO, arow, 0, g), vh[0], dp);
      dp = mfma_bf16_k32(lds_row8(stO, arow, 1, g), vh[1], dp);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = fast_exp2(fmaf(st[i], a.c2, madd - f.l4[t][i] * kLog2e));
        p[t][i] = pv;
        dsv[t][i] = pv * (dp[i] - f.d4[t][i]);
      }
    }
    bf16x8 p_hi, p_lo, ds_hi, ds_lo;
    split8(p, p_hi, p_lo);
    split8(dsv, ds_hi, ds_lo);
    // dV^T += dO^T P, dK^T += Q^T dS  (contract over the pair's 32 queries)
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
  };

  // ---- query-block pairs of CSC_1[j]: two load buffers used in turn
  for (int base = e0; base < e1; base += 64) {
    cnt = min(64, e1 - base);
    qtab = ttab = kNoRow;
    if (lane < cnt) {
      const int p = rows[base + lane];
      if (p >= 0 && p < n1) {
        qtab = (uint32_t)block_corner(p, a.grid) * kDim * 2;
        ttab = (uint32_t)p * kBlock * 4;
      }
    }
    const int npairs = (cnt + 1) >> 1;
    PairLd fa = load_pair(0), fb;
    for (int k = 0; k < npairs; k += 2) {
      fb = load_pair(k + 1);
      pair(fa);
      if (k + 1 >= npairs) break;
      fa = load_pair(k + 2);
      pair(fb);
    }
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
    bf16x4 rk4, rv4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rk4[i] = (bf16)(dka[t4][i] * a.scale + pdk[t4][i]);
      rv4[i] = (bf16)(dva[t4][i] + pdv[t4][i]);
    }
    *(bf16x4*)(dkp + 16 * t4 + 4 * g) = rk4;
    *(bf16x4*)(dvp + 16 * t4 + 4 * g) = rv4;
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
  const size_t qlds = bwd_query_lds_bytes(n_coarse > 0);
  if (n_coarse == 0)
    LLSA_LAUNCH("bwd_query_kernel", bwd_query_kernel<0>, dim3(qblocks), dim3(256), qlds, stream, a);
  else if (n_coarse <= 16)
    LLSA_LAUNCH("bwd_query_kernel", bwd_query_kernel<1>, dim3(qblocks), dim3(256), qlds, stream, a);
  else
    LLSA_LAUNCH("bwd_query_kernel", bwd_query_kernel<2>, dim3(qblocks), dim3(256), qlds, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (coarse) {
    for (int l = 3; l <= s.levels; ++l) {
      const long total = (long)s.bh * s.n_level(l) * s.topk * kDim;
      LLSA_LAUNCH("coarse_reduce_kernel", coarse_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256),
                         0, stream, a, l);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    for (int l = 2; l <= s.levels; ++l) {
      const long waves = (long)s.bh * s.n_level(l);
      LLSA_LAUNCH("coarse_grad_kernel", coarse_grad_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                         stream, a, l);
      if ((err = hipGetLastError()) != hipSuccess) return err;
    }
  }
  const long kwaves = (long)s.bh * (s.n >> kBlockShift);
  LLSA_LAUNCH("bwd_key_kernel", bwd_key_kernel, dim3((unsigned)kwaves), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace llsa
