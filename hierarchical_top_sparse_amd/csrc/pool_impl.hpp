// Device bodies of the pooling kernels, shared by pool.hip and by the selection launches that
// pool V beside the selection (select.hip).  See pool.hip for the design.  D: head_dim (64 or
// 128); every body works on 64-channel slices of the rows, one after the other.
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
// channel e % D of 64-token block e / D, e = t, t + 256, ... (a workgroup barrier first).
template <int D>
__device__ __forceinline__ void pool64_from_lds(const float (&sh)[kBlock][D], float* out,
                                                int head, int n, int group, int t) {
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4 * D / 256; ++i) {
    const int e = t + 256 * i;
    const int r = e / D, c = e % D;
    const float s = (sh[4 * r][c] + sh[4 * r + 1][c]) + (sh[4 * r + 2][c] + sh[4 * r + 3][c]);
    out[((long)head * (n >> 6) + group * 4 + r) * D + c] = s * 0.25f;
  }
}

// Level 2 of one group from its 16 staged level-1 means (a workgroup barrier first).
template <int D>
__device__ __forceinline__ void pool2_from_lds(const float (&sh)[kBlock][D], float* out,
                                               int head, int n1, int group, int t) {
  __syncthreads();
  for (int c = t; c < D; c += 256) {
    float s = 0.f;
#pragma unroll
    for (int b = 0; b < kBlock; ++b) s += sh[b][c];
    const int n2 = n1 >> kBlockShift;
    out[((long)head * n2 + group) * D + c] = s * (1.0f / kBlock);
  }
}

// bf16 tokens: thread t owns level-1 block t / 16 of the group, half (t / 8) % 2 of its 16
// tokens and the 16-byte channel piece t % 8 of each 64-channel slice; its 8 row loads of a
// slice are issued at once (each wave instruction reads 8 whole 128-byte row slices), the
// two halves meet by a cross-lane add.  Workgroup bx of tensor `tensor` (bx = head *
// groups_per_head + group), 256 threads.
template <int D>
__device__ __forceinline__ void pool12_bf16_group(const PoolArgs& args, int n, Grid grid,
                                                  int groups_per_head, int tensor, int bx,
                                                  float (&sh)[kBlock][D]) {
  const int head = bx / groups_per_head;
  const int group = bx - head * groups_per_head;
  const int t = threadIdx.x;
  const int blk = t >> 4;          // level-1 block within the group
  const int half = (t >> 3) & 1;   // tokens 8 half .. 8 half + 7 of the block
  const int cp = t & 7;            // channels 8 cp .. 8 cp + 7 of the slice
  const int first_tok = (group * kBlock + blk) * kBlock + 8 * half;
  const int n1 = n >> kBlockShift;
#pragma unroll
  for (int c0 = 0; c0 < D; c0 += 64) {
    const bf16* x = (const bf16*)args.x[tensor] + (long)head * n * D + c0 + 8 * cp;
    bf16x8 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      v[i] = *(const bf16x8*)(x + (long)token_row(first_tok + i, grid) * D);
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
    if (half == 0) {
      if (args.lv1[tensor]) {
        float* out =
            args.lv1[tensor] + ((long)head * n1 + group * kBlock + blk) * D + c0 + 8 * cp;
        *(f32x4*)out = l1a;
        *(f32x4*)(out + 4) = l1b;
      }
      *(f32x4*)&sh[blk][c0 + 8 * cp] = l1a;
      *(f32x4*)&sh[blk][c0 + 8 * cp + 4] = l1b;
    }
  }
  if (args.lv64[tensor]) pool64_from_lds<D>(sh, args.lv64[tensor], head, n, group, t);
  if (args.lv2[tensor]) pool2_from_lds<D>(sh, args.lv2[tensor], head, n1, group, t);
}

// fp32 tokens: thread t owns block t / 16 and channels 4 (t % 16) .. +3 of each 64-channel
// slice.
template <int D>
__device__ __forceinline__ void pool12_f32_group(const PoolArgs& args, int n, Grid grid,
                                                 int groups_per_head, int tensor, int bx,
                                                 float (&sh)[kBlock][D]) {
  const int head = bx / groups_per_head;
  const int group = bx - head * groups_per_head;
  const int t = threadIdx.x;
  const int blk = t >> 4;        // level-1 block within the group
  const int dq = (t & 15) * 4;   // first of 4 channels of the slice
  const int first_tok = (group * kBlock + blk) * kBlock;
  const int n1 = n >> kBlockShift;
  const float* x = (const float*)args.x[tensor] + (long)head * n * D;
#pragma unroll
  for (int c0 = 0; c0 < D; c0 += 64) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    f32x4 v[kBlock];
#pragma unroll
    for (int i = 0; i < kBlock; ++i)
      v[i] = *(const f32x4*)(x + (long)token_row(first_tok + i, grid) * D + c0 + dq);
#pragma unroll
    for (int i = 0; i < kBlock; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] += v[i][c];
    f32x4 l1;
#pragma unroll
    for (int c = 0; c < 4; ++c) l1[c] = acc[c] * (1.0f / kBlock);
    if (args.lv1[tensor]) {
      float* out = args.lv1[tensor] + ((long)head * n1 + group * kBlock + blk) * D + c0 + dq;
      *(f32x4*)out = l1;
    }
    if (args.lv64[tensor] || args.lv2[tensor]) {
#pragma unroll
      for (int c = 0; c < 4; ++c) sh[blk][c0 + dq + c] = l1[c];
    }
  }
  if (args.lv64[tensor]) pool64_from_lds<D>(sh, args.lv64[tensor], head, n, group, t);
  if (args.lv2[tensor]) pool2_from_lds<D>(sh, args.lv2[tensor], head, n1, group, t);
}

struct PoolNextArgs {
  const float* in[3];
  float* out[3];
};

// out[j][d] = mean_t in[j*B + t][d] (B = 16 or 64); output element i < total_out.
template <int B, int D>
__device__ __forceinline__ void pool_next_elem(const PoolNextArgs& args, int tensor, long i) {
  const long j = i / D;
  const int d = (int)(i - j * D);
  const float* src = args.in[tensor] + (j * B) * D + d;
  float s = 0.f;
#pragma unroll
  for (int t = 0; t < B; ++t) s += src[t * D];
  args.out[tensor][i] = s * (1.0f / B);
}

}  // namespace llsa
