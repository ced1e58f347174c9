// Internal launch interface between the C ABI (api.cpp) and the kernel files.
// Every launcher enqueues on `stream` and returns the hipError_t of the launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace llsa {

// Optional per-kernel timing (profile.cpp): events around each launch while enabled.
bool profiling_enabled();
void* prof_begin(const char* name, hipStream_t stream);
void prof_end(void* handle, hipStream_t stream);

#define LLSA_LAUNCH(name, kernel, grid, block, lds, stream, ...)                      \
  do {                                                                                 \
    void* prof_h_ = ::llsa::profiling_enabled() ? ::llsa::prof_begin(name, stream)     \
                                                : nullptr;                             \
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);                 \
    if (prof_h_) ::llsa::prof_end(prof_h_, stream);                                    \
  } while (0)

struct Shape {
  int bh;        // batch * heads
  int n;         // tokens per head
  int d;         // head_dim: 64 or 128
  int hbits;     // log2(height)
  int wbits;     // log2(width)
  int levels;    // L
  int topk;      // K
  int enrich;    // 0/1
  int coarse_levels;    // enrichment levels 2 .. 1 + coarse_levels (0: none)
  float coarse_lbias;   // log2 of a level-1 coarse weight ratio: 4 (weight 16^l) or 0 (1)
  int raster;    // token tensors in raster order
  int bf16;      // 1: bf16 token tensors, 0: fp32
  float scale;   // softmax scale
  int bshift;    // log2(B): 4 (B = 16, 4x4 tiles) or 6 (B = 64, 8x8 tiles)
  int fine_k;    // picks per 16-token query block seen by the attention: K * B / 16
  int exclude_overlap;   // 1: coarse keys over a finer selected key are dropped per block
  int n_level(int l) const { return n >> (bshift * l); }
};

hipError_t launch_reorder(const Shape& s, const void* x, void* y, int inverse,
                          hipStream_t stream);

hipError_t launch_pool(const Shape& s, const void* const x[3], float* const* lv[3],
                       hipStream_t stream);

hipError_t launch_select(const Shape& s, const float* const* q_lv, const float* const* k_lv,
                         int32_t* const* sel, int level_hi, int level_lo, hipStream_t stream);
hipError_t launch_pool_select(const Shape& s, const void* const x[3], float* const* lv[3],
                              int32_t* const* sel, hipStream_t stream);

hipError_t launch_attn_fwd(const Shape& s, const void* q, const void* k, const void* v,
                           const float* const* k_lv, const float* const* v_lv,
                           const int32_t* const* sel, void* o, float* lse, hipStream_t stream);

size_t transpose_workspace_bytes(int nmat, int rows, int cols, int k);
// true if a matrix of rows x k entries takes the radix path (at most 64 tiles of 4096), which
// has no limit on (cols + 1) * 2^ceil(log2 rows)
bool transpose_uses_radix(int rows, int k);
// Up to 8 matrix sets (nmat[i] matrices of rows[i] x k[i] -> cols[i]) in order on one stream,
// sharing one workspace.
size_t transpose_sets_workspace_bytes(int nsets, const int* nmat, const int* rows,
                                      const int* cols, const int* k);
hipError_t launch_transpose_sets(int nsets, const int* nmat, const int* rows, const int* cols,
                                 const int* k, const int32_t* const* csr, int32_t* const* off,
                                 int32_t* const* rows_out, void* ws, hipStream_t stream);
hipError_t launch_index_transpose(int nmat, int rows, int cols, int k, const int32_t* csr,
                                  int32_t* off, int32_t* rows_out, void* ws,
                                  hipStream_t stream);

size_t bwd_workspace_bytes(const Shape& s);
// Device address of this device's allocation-free scratch array (LLSA_NOALLOC_SCRATCH_BYTES),
// looked up on the first call on each device.
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_attn_bwd(const Shape& s, const void* q, const void* k, const void* v,
                           const void* dout, const float* lse,
                           const float* const* k_lv, const float* const* v_lv,
                           const int32_t* const* sel, const int32_t* const* csc_off,
                           const int32_t* const* csc_rows, const uint8_t* mask, void* dq,
                           void* dk, void* dv, void* ws, hipStream_t stream);

// Level-1 picks as 16-token blocks: [bh, N/16, K B/16] from [bh, N/B, K].
hipError_t launch_expand_blocks(const Shape& s, const int32_t* sel1, int32_t* fine,
                                hipStream_t stream);

// Calibration: a plain copy of `bytes` (a multiple of 16) and an MFMA-only loop of `blocks`
// 4-wave workgroups, `iters` rounds of 8 chains of 16x16x32 bf16 each (out: blocks * 256).
hipError_t launch_calib_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);
hipError_t launch_calib_mfma(float* out, int blocks, int iters, hipStream_t stream);

// Dense block mask [bh, n_1, n_1] (1 where key block c is in Sel_1[a]) of the mask-based
// comparator.
hipError_t launch_block_mask(const Shape& s, const int32_t* sel1, uint8_t* mask,
                             hipStream_t stream);

// Dense softmax attention over [bh, n, 64] bf16 sequences (the full-attention baseline).
hipError_t launch_dense_fwd(int bh, int n, float scale, const void* q, const void* k,
                            const void* v, void* o, float* lse, hipStream_t stream);
hipError_t launch_dense_bwd(int bh, int n, float scale, const void* q, const void* k,
                            const void* v, const void* dout, const float* lse, void* dq,
                            void* dk, void* dv, float* dd, hipStream_t stream);

}  // namespace llsa
