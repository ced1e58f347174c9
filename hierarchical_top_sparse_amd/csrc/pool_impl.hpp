// Device bodies of the pooling kernels, shared by pool.hip and by the selection launches that
// pool V beside the selection (select.hip).  See pool.hip for the design.
#pragma once
#include "common.hpp"

namespace llsa {

struct PoolArgs {
  const void* x[3];
  float* lv1[3];    // 16-token means (B = 16 level 1)
  float* lv2[3];    // 256-token means (B = 16 level 2)
  float* lv64[3];   // 64-token means (B = 64 level 1)
};

// B = 64 level 1 of one 256-token group from its 16 staged 16-token means: thread t writes
// channel t % 64 of 64-token block t / 64 (a workgroup barrier first).
__device__ __forceinline__ void pool64_from_lds(const float (&sh)[kBlock][kDim], float* out,
                                                int head, int n, int group, int t) {
  __syncthreads();
  const int r = t >> 6, c = t & 63;
  const float s = (sh[4 * r][c] + sh[4 * r + 1][c]) + (sh[4 * r + 2][c] + sh[4 * r + 3][c]);
  out[((long)head * (n >> 6) + group * 4 + r) * kDim + c] = s * 0.25f;
}

// bf16 tokens: thread t owns level-1 block t / 16 of the group, half (t / 8) % 2 of its 16
// tokens and the 16-byte channel piece t % 8; its 8 row loads are issued at once (each wave
// instruction reads 8 whole 128-byte rows), the two halves meet by a cross-lane add.
// Workgroup bx of tensor `tensor` (bx = head * groups_per_head + group), 256 threads.
__device__ __forceinline__ void pool12_bf16_group(const PoolArgs& args, int n, Grid grid,
                                                  int groups_per_head, int tensor, int bx,
                                                  float (&sh)[kBlock][kDim]) {
  const int head = bx / groups_per_head;
  const int group = bx - head * groups_per_head;
  const int t = threadIdx.x;
  const int blk = t >> 4;          // level-1 block within the group
  const int half = (t >> 3) & 1;   // tokens 8 half .. 8 half + 7 of the block
  const int cp = t & 7;            // channels 8 cp .. 8 cp + 7
  const int first_tok = (group * kBlock + blk) * kBlock + 8 * half;
  const bf16* x = (const bf16*)args.x[tensor] + (long)head * n * kDim + 8 * cp;
  bf16x8 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = *(const bf16x8*)(x + (long)token_row(first_tok + i, grid) * kDim);
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += (float)v[i][c];
    acc[c] = s + __shfl_xor(s, 8, 64);   // + the other half of the block
  }
  f32x4 l1a, l1b;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    l1a[c] = acc[c] * (1.0f / kBlock);
    l1b[c] = acc[4 + c] * (1.0f / kBlock);
  }
  const int n1 = n >> kBlockShift;
  if (half == 0) {
    if (args.lv1[tensor]) {
      float* out = args.lv1[tensor] + ((long)head * n1 + group * kBlock + blk) * kDim + 8 * cp;
      *(f32x4*)out = l1a;
      *(f32x4*)(out + 4) = l1b;
    }
    *(f32x4*)&sh[blk][8 * cp] = l1a;
    *(f32x4*)&sh[blk][8 * cp + 4] = l1b;
  }
  if (args.lv64[tensor]) pool64_from_lds(sh, args.lv64[tensor], head, n, group, t);
  if (args.lv2[tensor]) {
    __syncthreads();
    if (t < kDim) {
      float s = 0.f;
#pragma unroll
      for (int b = 0; b < kBlock; ++b) s += sh[b][t];
      const int n2 = n1 >> kBlockShift;
      args.lv2[tensor][((long)head * n2 + group) * kDim + t] = s * (1.0f / kBlock);
    }
  }
}

// fp32 tokens: thread t owns block t / 16 and channels 4 (t % 16) .. +3.
__device__ __forceinline__ void pool12_f32_group(const PoolArgs& args, int n, Grid grid,
                                                 int groups_per_head, int tensor, int bx,
                                                 float (&sh)[kBlock][kDim]) {
  const int head = bx / groups_per_head;
  const int group = bx - head * groups_per_head;
  const int t = threadIdx.x;
  const int blk = t >> 4;        // level-1 block within the group
  const int dq = (t & 15) * 4;   // first of 4 channels
  const int first_tok = (group * kBlock + blk) * kBlock;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  const float* x = (const float*)args.x[tensor] + (long)head * n * kDim;
  f32x4 v[kBlock];
#pragma unroll
  for (int i = 0; i < kBlock; ++i) v[i] = *(const f32x4*)(x + (long)token_row(first_tok + i, grid) * kDim + dq);
#pragma unroll
  for (int i = 0; i < kBlock; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] += v[i][c];
  f32x4 l1;
#pragma unroll
  for (int c = 0; c < 4; ++c) l1[c] = acc[c] * (1.0f / kBlock);
  const int n1 = n >> kBlockShift;
  if (args.lv1[tensor]) {
    float* out = args.lv1[tensor] + ((long)head * n1 + group * kBlock + blk) * kDim + dq;
    *(f32x4*)out = l1;
  }
  if (args.lv64[tensor]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) sh[blk][dq + c] = l1[c];
    pool64_from_lds(sh, args.lv64[tensor], head, n, group, t);
  }
  if (args.lv2[tensor]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) sh[blk][dq + c] = l1[c];
    __syncthreads();
    if (t < kDim) {
      float s = 0.f;
#pragma unroll
      for (int b = 0; b < kBlock; ++b) s += sh[b][t];
      const int n2 = n1 >> kBlockShift;
      args.lv2[tensor][((long)head * n2 + group) * kDim + t] = s * (1.0f / kBlock);
    }
  }
}

struct PoolNextArgs {
  const float* in[3];
  float* out[3];
};

// out[j][d] = mean_t in[j*B + t][d] (B = 16 or 64); output element i < total_out.
template <int B>
__device__ __forceinline__ void pool_next_elem(const PoolNextArgs& args, int tensor, long i) {
  const long j = i / kDim;
  const int d = (int)(i - j * kDim);
  const float* src = args.in[tensor] + (j * B) * kDim + d;
  float s = 0.f;
#pragma unroll
  for (int t = 0; t < B; ++t) s += src[t * kDim];
  args.out[tensor][i] = s * (1.0f / B);
}

}  // namespace llsa
