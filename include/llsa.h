/*
 * llsa.h — C ABI of the MI355X (gfx950) Log-linear Sparse Attention library (libllsa.so).
 *
 * The method: "Trainable Log-linear Sparse Attention for Efficient Diffusion Transformers"
 * (paper summary page, sec. 三 Hierarchical Top-K, sec. 四 Hierarchical KV Enrichment,
 * sec. 4.1 sparse backward via a CSR->CSC sparse index transpose, sec. 4.2 / Figure 2 2D index
 * reordering), and the popular article on arXiv:2512.16615 (sec. 三 and 四).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Token tensors (q, k, v, o, dout, dq, dk, dv) are contiguous [batch, heads, N, head_dim]
 *    with N = height * width.  Their token order is `layout`:
 *      LLSA_LAYOUT_MORTON: already in Morton (Z-order) position order;
 *      LLSA_LAYOUT_RASTER: raster order y*width + x; the kernels apply the Morton map in
 *                          their load/store addressing (the reorder step folded into them).
 *  - Pooled levels, selections, CSC indices and the log-sum-exp are always indexed in
 *    Morton/block order: level l has n_l = N / block^l tokens.
 *      level arrays  float   [batch, heads, n_l, head_dim]
 *      sel[l-1]      int32   [batch, heads, n_l, topk]  (key ids at level l, ascending)
 *      lse           float   [batch, heads, N]          (natural log, coarse weights included)
 *  - All data pointers are DEVICE pointers, 16-byte aligned; the caller owns every buffer.
 *    Inputs must not alias outputs.  The library allocates no device memory and keeps no
 *    state between calls (only a thread-local error message).
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only enqueues work;
 *    none synchronises.  Device faults surface at the caller's next synchronisation.
 *  - Return value: llsa_status.  Validation errors return before anything is enqueued and
 *    leave outputs untouched; LLSA_ERR_HIP means a launch failed (outputs undefined).
 *    llsa_last_error() gives a message for the last failure on the calling thread.
 *  - Results are deterministic: every sum has a fixed order and no data is added atomically
 *    (the only atomics are integer completion counts that order work).
 *  - Supported: head_dim 64 or 128, block 16 (4x4 pixel tiles) or 64 (8x8 pixel tiles),
 *    height and width powers of two >= 4, 256 <= N <= 2^23, N % block^levels == 0,
 *    1 <= topk <= min(32, N / block^levels) and topk * block / 16 <= 32,
 *    1 <= levels <= 6, batch*heads*N < 2^31.  dtype bf16 for every call; f32 for
 *    reorder/pool/select, and for attn_fwd with head_dim 64.
 */
#ifndef LLSA_H
#define LLSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LLSA_ABI_VERSION 5
#define LLSA_MAX_LEVELS 6
#define LLSA_MAX_TOPK 32

typedef enum {
  LLSA_OK = 0,
  LLSA_ERR_NULL = 1,        /* a required pointer is NULL */
  LLSA_ERR_SHAPE = 2,       /* sizes violate the constraints above */
  LLSA_ERR_DTYPE = 3,       /* unknown dtype or layout code */
  LLSA_ERR_UNSUPPORTED = 4, /* valid but not implemented (e.g. head_dim 96) */
  LLSA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required */
  LLSA_ERR_ALIGN = 6,       /* a pointer is not 16-byte aligned */
  LLSA_ERR_HIP = 7          /* a HIP launch failed */
} llsa_status;

typedef enum { LLSA_F32 = 0, LLSA_BF16 = 1 } llsa_dtype;
typedef enum { LLSA_LAYOUT_MORTON = 0, LLSA_LAYOUT_RASTER = 1 } llsa_layout;

typedef struct {
  int32_t batch;
  int32_t heads;
  int32_t height;   /* pixel rows    (power of two) */
  int32_t width;    /* pixel columns (power of two) */
  int32_t head_dim; /* 64 or 128 */
  int32_t block;    /* B: tokens per pooled token; 16 = a 4x4 tile, 64 = an 8x8 tile */
  int32_t levels;   /* L: pooled levels 1..L; the coarsest has N / B^L tokens */
  int32_t topk;     /* K: keys kept per query at every level */
  int32_t enrich;   /* 0: fine keys only; 1: also the K selected keys of levels 2..L */
  float scale;      /* softmax scale; 0 => 1/sqrt(head_dim) */
  int32_t dtype;    /* llsa_dtype of the token tensors */
  int32_t layout;   /* llsa_layout of the token tensors */
  /* Enrichment variants (zero = the method as described): */
  int32_t enrich_levels;      /* with enrich: only the coarse levels 2 .. 1 + enrich_levels
                                 (the finest ones; clamped to L); 0 = all levels 2..L */
  int32_t coarse_unit_weight; /* 0: a coarse key of level l has weight B^l (logit bias
                                 l ln B); 1: weight 1 (no bias) */
  int32_t coarse_exclude_overlap; /* 1: drop, per query block, a coarse key of level l that
                                     is the parent of a key selected for it at level l-1
                                     (a fine block for l = 2): no region counted twice */
} llsa_problem;

/* ABI version (LLSA_ABI_VERSION of the built library). */
int32_t llsa_abi_version(void);

/* Static string for a status code. */
const char* llsa_status_str(int32_t status);

/* Message describing the last failure on the calling thread ("" if none). */
const char* llsa_last_error(void);

/* Host-only validation of a problem description; enqueues nothing. */
int32_t llsa_check(const llsa_problem* p);

/* Workspace bytes llsa_attn_bwd needs (fwd_bytes is 0: the forward needs none). */
int32_t llsa_workspace_bytes(const llsa_problem* p, size_t* fwd_bytes, size_t* bwd_bytes);

/*
 * llsa_reorder — 2D index reordering (paper summary sec. 4.2 / Figure 2; article sec. 四,
 * "like Z-order or Hilbert curves").  Morton order: bits 2i / 2i+1 of the curve position are
 * bit i of x / y; bits beyond the shorter side extend the longer one.  inverse = 0:
 * y[.., m, :] = x[.., raster(m), :]; inverse = 1: y[.., raster(m), :] = x[.., m, :].
 * x, y: [batch, heads, N, head_dim] of p->dtype; p->layout is ignored.  Bit-exact copy.
 */
int32_t llsa_reorder(const llsa_problem* p, const void* x, void* y, int32_t inverse,
                     void* stream);

/*
 * llsa_pool — hierarchical compression by recursive mean pooling (summary sec. 三):
 * X_l[j] = (1/B) * sum_{t<B} X_{l-1}[j*B + t], l = 1..L, X_0 = the Morton-ordered tokens.
 * q, k, v: token tensors (layout p->layout, dtype p->dtype); a NULL input skips that tensor.
 * q_lv/k_lv/v_lv: arrays of L float pointers (level l at index l-1), each
 * [batch, heads, n_l, head_dim]; a NULL entry skips storing that level.  fp32 arithmetic.
 */
int32_t llsa_pool(const llsa_problem* p, const void* q, const void* k, const void* v,
                  float* const* q_lv, float* const* k_lv, float* const* v_lv, void* stream);

/*
 * llsa_select — coarse-to-fine top-K selection (summary sec. 三; article sec. 三).
 * Level L: scores Q_L . K_L over all n_L keys, top-K per row.  Level l < L: query a scores
 * only the K*B children {c*B + t} of Sel_{l+1}[a / B] and keeps the top-K.  Scores are fp32
 * dot products of the pooled levels; ties go to the lower key id; rows are stored ascending.
 * Computes levels level_hi down to level_lo (1 <= level_lo <= level_hi <= L); when
 * level_hi < L, sel[level_hi] (level level_hi + 1) is read as the parent selection.
 * q_lv, k_lv: L level pointers (only the levels computed are read); sel: L pointers.
 */
int32_t llsa_select(const llsa_problem* p, const float* const* q_lv, const float* const* k_lv,
                    int32_t* const* sel, int32_t level_hi, int32_t level_lo, void* stream);

/*
 * llsa_pool_select — llsa_pool followed by llsa_select of levels L..1 (summary sec. 三: the
 * hierarchical compression and the coarse-to-fine search), as one call.  Same arguments and
 * results as the two calls: q, k (required) and v (NULL skips it) are the tokens; q_lv and
 * k_lv need all L levels (the selection reads them), v_lv the levels llsa_pool needs; sel:
 * L pointers as for llsa_select.  V's levels are first read by the attention, not by the
 * selection, so with block 16, bf16 tokens and L >= 2 its pooling runs inside the selection
 * launches (their workgroups after the selection's), where it fills the chip while the
 * selection's few waves run their dependent chains.  Errors as for the two calls.
 */
int32_t llsa_pool_select(const llsa_problem* p, const void* q, const void* k, const void* v,
                         float* const* q_lv, float* const* k_lv, float* const* v_lv,
                         int32_t* const* sel, void* stream);

/*
 * llsa_expand_blocks — level-1 picks as the 16-token blocks they cover, the form the
 * attention kernels read: fine[b][h][q][i * (B/16) + t] = sel1[b][h][q / (B/16)][i] * (B/16)
 * + t for t < B/16, i < topk (ascending rows stay ascending; negative ids stay -1).
 * sel1: [b, H, N/B, topk] (Sel_1 from llsa_select); fine: [b, H, N/16, topk * B / 16],
 * caller-owned, distinct from sel1.  With block 16 a copy.
 */
int32_t llsa_expand_blocks(const llsa_problem* p, const int32_t* sel1, int32_t* fine,
                           void* stream);

/*
 * llsa_attn_fwd — sparse attention with hierarchical KV enrichment (summary sec. 四;
 * article sec. 三/四: gather of the selected blocks, no dense mask).  Each level-1 query
 * block p (B queries) attends to the B tokens of each block in sel[0][p] and, if enrich,
 * for l = 2..L to the pooled keys/values k_lv/v_lv[l-1][sel[l-1][p / B^(l-1)]] with weight
 * B^l (their exp(score) is multiplied by B^l).  s = scale * q.k; o = sum w e^s v / sum w e^s;
 * lse = log sum w e^s.  bf16: MFMA with fp32 accumulation and softmax (the fp32 pooled keys and
 * values enter the MFMA as bf16 hi + lo parts, about 16 mantissa bits; P is rounded once to
 * bf16 for P V); f32 (head_dim 64 only, else LLSA_ERR_UNSUPPORTED): fp32 MFMA.  k_lv/v_lv: L
 * pointers, levels >= 2 read.
 * Out-of-range indices in sel are skipped.  o: token tensor (layout), lse: [b, H, N] Morton.
 * sel[0] lists level-1 picks as 16-token blocks: [b, H, N/16, topk * block / 16]; with block
 * 16 that is Sel_1 itself, with block 64 the output of llsa_expand_blocks.  sel[l-1], l >= 2:
 * Sel_l as from llsa_select.
 */
int32_t llsa_attn_fwd(const llsa_problem* p, const void* q, const void* k, const void* v,
                      const float* const* k_lv, const float* const* v_lv,
                      const int32_t* const* sel, void* o, float* lse, void* stream);

/*
 * llsa_index_transpose — sparse index transpose CSR -> CSC (summary sec. 4.1; article sec.
 * 四: per-key counts, offsets by prefix sum, a flat vector of query ids per key).
 * csr: [nmat, rows, k] int32 column ids of each row (the K keys a query selected);
 * csc_off: [nmat, cols + 1]; csc_rows: [nmat, rows * k]: the rows that selected column c are
 * csc_rows[off[c] .. off[c+1]) in ascending order.  Entries outside [0, cols) are dropped
 * (off[cols] counts the kept ones; later csc_rows entries are unspecified).
 * Atomic-free (a stable sort by column), so the output is deterministic.
 * ws: device workspace of llsa_index_transpose_workspace() bytes (may be 0 for a matrix of at
 * most 4096 entries: ws may then be NULL).  Matrices of more than 64 tiles of 4096 entries
 * require (cols + 1) * 2^ceil(log2 rows) <= 2^32.
 */
int32_t llsa_index_transpose_workspace(int32_t nmat, int32_t rows, int32_t cols, int32_t k,
                                       size_t* bytes);
int32_t llsa_index_transpose(int32_t nmat, int32_t rows, int32_t cols, int32_t k,
                             const int32_t* csr, int32_t* csc_off, int32_t* csc_rows,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * llsa_index_transpose_levels — llsa_index_transpose of every level the backward reads, as one
 * call (summary sec. 4.1; article sec. 四): level 1 as 16-token blocks (sel[0] as for
 * llsa_attn_fwd; rows = cols = N/16, k = topk * block / 16) and, with enrichment, levels
 * 2 .. 1 + coarse levels (rows = cols = n_l, k = topk).  csc_off[l-1]: [batch, heads, rows + 1],
 * csc_rows[l-1]: [batch, heads, rows * k], exactly as llsa_index_transpose of that level writes
 * them.  Levels of at most 64 tiles of 4096 entries run together in two launches.  ws: device
 * workspace of llsa_index_transpose_levels_workspace() bytes (may be 0: ws may then be NULL).
 * Atomic-free, deterministic.  Errors as for llsa_index_transpose.
 */
int32_t llsa_index_transpose_levels_workspace(const llsa_problem* p, size_t* bytes);
int32_t llsa_index_transpose_levels(const llsa_problem* p, const int32_t* const* sel,
                                    int32_t* const* csc_off, int32_t* const* csc_rows, void* ws,
                                    size_t ws_bytes, void* stream);

/*
 * llsa_attn_bwd — sparse backward (summary sec. 4.1 and Figure 4: query-major dQ, key-major
 * dK/dV over the CSC index, no T x T mask).  Per query: P = w e^{s - lse}, dP = dO.v,
 * D = sum_e P_e dP_e, dS = P (dP - D); dq = scale sum dS k; fine keys get dk += scale dS q,
 * dv += P dO; a coarse key (l, j) collects the same into dK_l[j], dV_l[j], which are then
 * spread over its B^l fine tokens with factor 1/B^l (chain rule of the mean pooling).
 * D is recomputed from the scores (the forward output O is not needed).
 * No gradient through the selection or the pooled Q.  Outputs: complete dq, dk, dv
 * (layout p->layout).  csc_off/csc_rows: L pointers, level l from llsa_index_transpose of
 * sel[l-1] (rows = cols = n_l); levels >= 2 are read only if enrich.  bf16 only.
 * sel[0], csc_off[0], csc_rows[0]: level 1 as 16-token blocks (sel[0] as for llsa_attn_fwd;
 * its transpose has rows = cols = N/16 and k = topk * block / 16).  N <= 2^19 per head (the
 * level-1 transpose's 32-bit codes); LLSA_ERR_UNSUPPORTED above.
 * Deterministic: the query blocks of a key block picked by more than 128 of them are cut
 * into chunks of 128 whose partial dK/dV sums are added in chunk order (with head_dim 64 the
 * chunks run in the key-major launch, and an integer count per key block, one increment per
 * written chunk, tells the key block when they are all written; no data is summed
 * atomically).
 * ws: llsa_workspace_bytes(bwd) bytes of device memory (D, coarse partials, chunk partials).
 */
int32_t llsa_attn_bwd(const llsa_problem* p, const void* q, const void* k, const void* v,
                      const void* dout, const float* lse,
                      const float* const* k_lv, const float* const* v_lv,
                      const int32_t* const* sel, const int32_t* const* csc_off,
                      const int32_t* const* csc_rows, void* dq, void* dk, void* dv, void* ws,
                      size_t ws_bytes, void* stream);

/*
 * llsa_attn_bwd_noalloc — llsa_attn_bwd without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments (minus ws, ws_bytes), kernels and results as
 * llsa_attn_bwd: bit-identical outputs.  The workspace is a file-scope device array of
 * LLSA_NOALLOC_SCRATCH_BYTES that every device the library runs on holds until the process
 * ends; its address is looked up on the first call on each device (the current device, which
 * must be the stream's).  Allocates nothing, ever.  Problems whose llsa_workspace_bytes (bwd)
 * exceeds LLSA_NOALLOC_SCRATCH_BYTES fail with LLSA_ERR_WORKSPACE before anything is enqueued
 * (at 256x256 pixels: batch * heads <= 14 with the default L = 3, K = 8).  All calls on one
 * device share that device's array and nothing in it persists between calls that the next
 * call reads: calls that overlap on one device (concurrent streams or threads) race, and the
 * caller must serialise them.  Errors otherwise as for llsa_attn_bwd.
 */
#define LLSA_NOALLOC_SCRATCH_BYTES (96u << 20)
int32_t llsa_attn_bwd_noalloc(const llsa_problem* p, const void* q, const void* k,
                              const void* v, const void* dout, const float* lse,
                              const float* const* k_lv, const float* const* v_lv,
                              const int32_t* const* sel, const int32_t* const* csc_off,
                              const int32_t* const* csc_rows, void* dq, void* dk, void* dv,
                              void* stream);

/*
 * llsa_dense_attn_fwd / llsa_dense_attn_bwd — dense softmax attention over all N keys, the
 * full-attention baseline the sparse method is measured against (paper summary sec. 5.4 and
 * Figure 3 compare against dense FlashAttention at the same sequence length).  Not part of
 * the sparse path.  Tokens are a plain sequence (the result does not depend on their order).
 * q, k, v, o, dout, dq, dk, dv: bf16 [batch_heads, n, head_dim], contiguous, 16-byte aligned;
 * lse: fp32 [batch_heads, n] (natural log), written by the forward, read by the backward;
 * d_rows: fp32 [batch_heads, n] caller-owned scratch, receives D = rowsum(dout * o), computed
 * as sum_j P_ij dP_ij from the recomputed scores (the backward does not read o).
 * o = softmax(scale q k^T) v, flash-style (fp32 accumulation and softmax; in the forward P
 * enters the bf16 MFMA rounded to bf16; in the backward P, P dP and dS enter as bf16 hi + lo
 * pairs, the same arithmetic as llsa_attn_bwd).  Requires head_dim 64 and n a multiple of 128 in [128, 2^23];
 * scale 0 => 1/sqrt(head_dim).  Deterministic (no atomics).  Errors as for the calls above.
 */
int32_t llsa_dense_attn_fwd(int32_t batch_heads, int32_t n, int32_t head_dim, float scale,
                            const void* q, const void* k, const void* v, void* o, float* lse,
                            void* stream);
int32_t llsa_dense_attn_bwd(int32_t batch_heads, int32_t n, int32_t head_dim, float scale,
                            const void* q, const void* k, const void* v, const void* dout,
                            const float* lse, void* dq, void* dk, void* dv, float* d_rows,
                            void* stream);

/*
 * llsa_block_mask / llsa_attn_bwd_masked — the mask-based comparator of the sparse backward
 * (article sec. 4.1: sparse attention kernels that gather blocks in the forward but build a
 * T x T binary mask in the backward pay O(T^2) again; its Figure 4 measures such a
 * dense-mask baseline of the KV backward).  Not part of the sparse path.
 * llsa_block_mask writes mask: uint8 [batch, heads, n_1, n_1], caller-owned, 16-byte
 * aligned, mask[b][h][a][c] = 1 iff key block c is in sel1[b][h][a] (sel1 = Sel_1 as from
 * llsa_select), 0 elsewhere; it clears all batch*heads*n_1^2 bytes.
 * llsa_attn_bwd_masked computes what llsa_attn_bwd computes for a problem without coarse
 * keys (levels 1, or enrich 0), with the key-major pass finding the query blocks of each key
 * block by scanning its column of the mask instead of reading CSC_1 (no chunking); the
 * results are bit-identical to llsa_attn_bwd's when no key block is picked by more than 128
 * query blocks, and otherwise differ only in the fp32 order of dK/dV sums.  Arguments as for llsa_attn_bwd; ws: llsa_workspace_bytes
 * (bwd) bytes.  Both: bf16 and head_dim 64 only; LLSA_ERR_UNSUPPORTED if levels > 1 and
 * enrich, LLSA_ERR_SHAPE if the mask would exceed 2^34 bytes.  Errors otherwise as for the calls above.
 */
int32_t llsa_block_mask(const llsa_problem* p, const int32_t* sel1, uint8_t* mask,
                        void* stream);
int32_t llsa_attn_bwd_masked(const llsa_problem* p, const void* q, const void* k, const void* v,
                             const void* dout, const float* lse, const int32_t* sel1,
                             const uint8_t* mask, void* dq, void* dk, void* dv, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * llsa_calib_copy / llsa_calib_mfma — calibration kernels for the achievable peaks (not part
 * of the method).  llsa_calib_copy copies `bytes` (a nonzero multiple of 16, at most 2^40)
 * from src to dst (device, 16-byte aligned, not overlapping) with 16-byte vector loads and
 * stores: (2 * bytes) / time is the reachable HBM bandwidth.  llsa_calib_mfma runs `blocks`
 * workgroups of 4 waves (1 <= blocks <= 2^20), each wave `iters` rounds (1..2^16) of 8
 * independent v_mfma_f32_16x16x32_bf16 on constant all-ones operands, and writes
 * out[blocks * 256] = 8 * 32 * iters per thread (a check that the work was done): the
 * dense bf16 MFMA rate is blocks * 4 * iters * 8 * 16384 flops / time.
 */
int32_t llsa_calib_copy(const void* src, void* dst, size_t bytes, void* stream);
int32_t llsa_calib_mfma(float* out, int32_t blocks, int32_t iters, void* stream);

/*
 * Per-kernel timing (profiling aid, not part of the method).  llsa_profile_enable(1) makes
 * every later kernel launch of the library record a pair of hipEvents on its stream;
 * llsa_profile_read() waits for the recorded events, writes one line per kernel name,
 * "<name> <launches> <total_ms>\n", into buf (NUL-terminated, truncated to len), and clears
 * the records.  Returns LLSA_ERR_HIP if an event could not be read.  Thread-safe.
 */
int32_t llsa_profile_enable(int32_t on);
int32_t llsa_profile_read(char* buf, size_t len);

#ifdef __cplusplus
}
#endif
#endif /* LLSA_H */
