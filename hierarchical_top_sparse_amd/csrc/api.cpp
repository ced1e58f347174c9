// C ABI of libllsa.so: host-side validation, workspace sizing and kernel launches.
// Every entry point is declared and documented in include/llsa.h.  No C++ exception crosses
// the boundary; validation failures return before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/llsa.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int32_t fail(int32_t status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int32_t hip_status(hipError_t err, const char* what) {
  if (err == hipSuccess) return LLSA_OK;
  return fail(LLSA_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

bool is_pow2(long v) { return v > 0 && (v & (v - 1)) == 0; }
int log2i(long v) {
  int b = 0;
  while ((1L << b) < v) ++b;
  return b;
}
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int32_t check_problem(const llsa_problem* p) {
  if (!p) return fail(LLSA_ERR_NULL, "problem is NULL");
  if (p->dtype != LLSA_F32 && p->dtype != LLSA_BF16)
    return fail(LLSA_ERR_DTYPE, "unknown dtype code %d", p->dtype);
  if (p->layout != LLSA_LAYOUT_MORTON && p->layout != LLSA_LAYOUT_RASTER)
    return fail(LLSA_ERR_DTYPE, "unknown layout code %d", p->layout);
  if (p->batch < 1 || p->heads < 1)
    return fail(LLSA_ERR_SHAPE, "batch (%d) and heads (%d) must be >= 1", p->batch, p->heads);
  if (!is_pow2(p->height) || !is_pow2(p->width) || p->height < 4 || p->width < 4)
    return fail(LLSA_ERR_SHAPE, "height (%d) and width (%d) must be powers of two >= 4",
                p->height, p->width);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(LLSA_ERR_UNSUPPORTED, "head_dim %d: 64 and 128 are implemented", p->head_dim);
  if (p->block != 16 && p->block != 64)
    return fail(p->block > 1 && is_pow2(p->block) && (log2i(p->block) % 2 == 0)
                    ? LLSA_ERR_UNSUPPORTED
                    : LLSA_ERR_SHAPE,
                "block %d: 16 (4x4 tiles) and 64 (8x8 tiles) are implemented", p->block);
  if (p->levels < 1 || p->levels > LLSA_MAX_LEVELS)
    return fail(LLSA_ERR_SHAPE, "levels %d out of [1, %d]", p->levels, LLSA_MAX_LEVELS);
  const long n = (long)p->height * p->width;
  if (n < 256) return fail(LLSA_ERR_SHAPE, "N = %ld tokens: at least 256 needed", n);
  if (n > (1L << 23)) return fail(LLSA_ERR_SHAPE, "N = %ld tokens: at most 2^23 supported", n);
  const long span = 1L << (log2i(p->block) * p->levels);
  if (log2i(p->block) * p->levels > 23)
    return fail(LLSA_ERR_SHAPE, "block^levels exceeds 2^23 tokens");
  if (n % span != 0)
    return fail(LLSA_ERR_SHAPE, "N = %ld is not divisible by block^levels = %ld", n, span);
  const long n_top = n / span;
  if (p->topk < 1 || p->topk > LLSA_MAX_TOPK || p->topk > n_top)
    return fail(LLSA_ERR_SHAPE, "topk %d out of [1, min(%d, N/B^L = %ld)]", p->topk,
                LLSA_MAX_TOPK, n_top);
  if (p->topk * (p->block / 16) > LLSA_MAX_TOPK)
    return fail(LLSA_ERR_UNSUPPORTED, "topk %d with block %d covers %d 16-token blocks per "
                "query block: at most %d are supported", p->topk, p->block,
                p->topk * (p->block / 16), LLSA_MAX_TOPK);
  if (p->enrich != 0 && p->enrich != 1)
    return fail(LLSA_ERR_SHAPE, "enrich must be 0 or 1 (got %d)", p->enrich);
  if (p->enrich_levels < 0)
    return fail(LLSA_ERR_SHAPE, "enrich_levels must be >= 0 (got %d)", p->enrich_levels);
  if (p->coarse_unit_weight != 0 && p->coarse_unit_weight != 1)
    return fail(LLSA_ERR_SHAPE, "coarse_unit_weight must be 0 or 1 (got %d)",
                p->coarse_unit_weight);
  if (p->coarse_exclude_overlap != 0 && p->coarse_exclude_overlap != 1)
    return fail(LLSA_ERR_SHAPE, "coarse_exclude_overlap must be 0 or 1 (got %d)",
                p->coarse_exclude_overlap);
  if (!(p->scale >= 0.f) || std::isinf(p->scale))
    return fail(LLSA_ERR_SHAPE, "scale must be finite and >= 0");
  if ((long)p->batch * p->heads * n >= (1L << 31))
    return fail(LLSA_ERR_SHAPE, "batch*heads*N must be < 2^31");
  return LLSA_OK;
}

// Coarse levels whose keys enrich the attention: 2 .. 1 + the returned count.
int coarse_levels(const llsa_problem* p) {
  if (!p->enrich || p->levels < 2) return 0;
  return p->enrich_levels == 0 ? p->levels - 1 : std::min(p->enrich_levels, p->levels - 1);
}

llsa::Shape make_shape(const llsa_problem* p) {
  llsa::Shape s{};
  s.bh = p->batch * p->heads;
  s.n = p->height * p->width;
  s.d = p->head_dim;
  s.hbits = log2i(p->height);
  s.wbits = log2i(p->width);
  s.levels = p->levels;
  s.topk = p->topk;
  s.enrich = p->enrich;
  s.coarse_levels = coarse_levels(p);
  s.coarse_lbias = p->coarse_unit_weight ? 0.f : (float)log2i(p->block);   // weight B^l
  s.raster = p->layout == LLSA_LAYOUT_RASTER;
  s.bf16 = p->dtype == LLSA_BF16;
  s.scale = p->scale > 0.f ? p->scale : 1.0f / std::sqrt((float)p->head_dim);
  s.bshift = log2i(p->block);
  s.exclude_overlap = p->coarse_exclude_overlap;
  s.fine_k = p->topk * (p->block / 16);
  return s;
}

#define CHECK_PTR(ptr, name)                                            \
  do {                                                                  \
    if (!(ptr)) return fail(LLSA_ERR_NULL, "%s is NULL", name);         \
    if (!aligned16(ptr)) return fail(LLSA_ERR_ALIGN, "%s is not 16-byte aligned", name); \
  } while (0)

}  // namespace

extern "C" {

int32_t llsa_abi_version(void) { return LLSA_ABI_VERSION; }

const char* llsa_status_str(int32_t status) {
  switch (status) {
    case LLSA_OK: return "ok";
    case LLSA_ERR_NULL: return "null pointer";
    case LLSA_ERR_SHAPE: return "invalid shape";
    case LLSA_ERR_DTYPE: return "invalid dtype or layout";
    case LLSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case LLSA_ERR_WORKSPACE: return "workspace missing or too small";
    case LLSA_ERR_ALIGN: return "misaligned pointer";
    case LLSA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

const char* llsa_last_error(void) { return g_last_error.c_str(); }

int32_t llsa_check(const llsa_problem* p) {
  g_last_error.clear();
  return check_problem(p);
}

int32_t llsa_workspace_bytes(const llsa_problem* p, size_t* fwd_bytes, size_t* bwd_bytes) {
  const int32_t st = check_problem(p);
  if (st != LLSA_OK) return st;
  if (!fwd_bytes || !bwd_bytes) return fail(LLSA_ERR_NULL, "output pointer is NULL");
  *fwd_bytes = 0;
  *bwd_bytes = llsa::bwd_workspace_bytes(make_shape(p));
  return LLSA_OK;
}

int32_t llsa_reorder(const llsa_problem* p, const void* x, void* y, int32_t inverse,
                     void* stream) {
  int32_t st = check_problem(p);
  if (st != LLSA_OK) return st;
  CHECK_PTR(x, "x");
  CHECK_PTR(y, "y");
  if (x == y) return fail(LLSA_ERR_SHAPE, "reorder cannot run in place");
  if (inverse != 0 && inverse != 1) return fail(LLSA_ERR_SHAPE, "inverse must be 0 or 1");
  return hip_status(llsa::launch_reorder(make_shape(p), x, y, inverse, (hipStream_t)stream),
                    "llsa_reorder");
}

int32_t llsa_pool(const llsa_problem* p, const void* q, const void* k, const void* v,
                  float* const* q_lv, float* const* k_lv, float* const* v_lv, void* stream) {
  int32_t st = check_problem(p);
  if (st != LLSA_OK) return st;
  const void* x[3] = {q, k, v};
  float* const* lv[3] = {q_lv, k_lv, v_lv};
  const char* names[3] = {"q", "k", "v"};
  bool any = false;
  for (int t = 0; t < 3; ++t) {
    if (!x[t]) continue;
    any = true;
    if (!aligned16(x[t])) return fail(LLSA_ERR_ALIGN, "%s is not 16-byte aligned", names[t]);
    if (!lv[t]) return fail(LLSA_ERR_NULL, "level array of %s is NULL", names[t]);
    for (int l = 1; l <= p->levels; ++l) {
      float* ptr = lv[t][l - 1];
      // levels below L feed the next level and must be stored: 2..L-1 for block 16 (its
      // levels 1 and 2 come from the tokens), 1..L-1 for block 64
      if (!ptr && l < p->levels && (l >= 2 || p->block != 16))
        return fail(LLSA_ERR_NULL, "%s level %d is needed for level %d", names[t], l, l + 1);
      if (ptr && !aligned16(ptr))
        return fail(LLSA_ERR_ALIGN, "%s level %d is not 16-byte aligned", names[t], l);
    }
  }
  if (!any) return fail(LLSA_ERR_NULL, "q, k and v are all NULL");
  return hip_status(llsa::launch_pool(make_shape(p), x, lv, (hipStream_t)stream), "llsa_pool");
}

int32_t llsa_pool_select(const llsa_problem* p, const void* q, const void* k, const void* v,
                         float* const* q_lv, float* const* k_lv, float* const* v_lv,
                         int32_t* const* sel, void* stream) {
  int32_t st = check_problem(p);
  if (st != LLSA_OK) return st;
  CHECK_PTR(q, "q");
  CHECK_PTR(k, "k");
  if (!q_lv || !k_lv || !sel) return fail(LLSA_ERR_NULL, "level or selection array is NULL");
  const void* x[3] = {q, k, v};
  float* const* lv[3] = {q_lv, k_lv, v_lv};
  const char* names[3] = {"q", "k", "v"};
  for (int t = 0; t < 3; ++t) {
    if (!x[t]) continue;
    if (!aligned16(x[t])) return fail(LLSA_ERR_ALIGN, "%s is not 16-byte aligned", names[t]);
    if (!lv[t]) return fail(LLSA_ERR_NULL, "level array of %s is NULL", names[t]);
    for (int l = 1; l <= p->levels; ++l) {
      float* ptr = lv[t][l - 1];
      // the selection reads every level of Q and K; V's levels below L feed the next one
      if (!ptr && (t < 2 || (l < p->levels && (l >= 2 || p->block != 16))))
        return fail(LLSA_ERR_NULL, "%s level %d is needed", names[t], l);
      if (ptr && !aligned16(ptr))
        return fail(LLSA_ERR_ALIGN, "%s level %d is not 16-byte aligned", names[t], l);
    }
  }
  for (int l = 1; l <= p->levels; ++l) CHECK_PTR(sel[l - 1], "selection");
  return hip_status(llsa::launch_pool_select(make_shape(p), x, lv, sel, (hipStream_t)stream),
                    "llsa_pool_select");
}

int32_t llsa_select(const llsa_problem* p, const float* const* q_lv, const float* const* k_lv,
                    int32_t* const* sel, int32_t level_hi, int32_t level_lo, void* stream) {
  int32_t st = check_problem(p);
  if (st != LLSA_OK) return st;
  if (!q_lv || !k_lv || !sel) return fail(LLSA_ERR_NULL, "level or selection array is NULL");
  if (level_lo < 1 || level_hi > p->levels || level_lo > level_hi)
    return fail(LLSA_ERR_SHAPE, "levels %d..%d outside 1..%d", level_hi, level_lo, p->levels);
  for (int l = level_lo; l <= level_hi; ++l) {
    CHECK_PTR(q_lv[l - 1], "q level");
    CHECK_PTR(k_lv[l - 1], "k level");
    CHECK_PTR(sel[l - 1], "selection");
  }
  if (level_hi < p->levels) CHECK_PTR(sel[level_hi], "parent selection");
  return hip_status(llsa::launch_select(make_shape(p), q_lv, k_lv, sel, level_hi, level_lo,
                                        (hipStream_t)stream),
                    "llsa_select");
}

int32_t llsa_expand_blocks(const llsa_problem* p, const int32_t* sel1, int32_t* fine,
                           void* stream) {
  int32_t st = check_problem(p);
  if (st != LLSA_OK) return st;
  CHECK_PTR(sel1, "sel1");
  CHECK_PTR(fine, "fine");
  if ((const void*)sel1 == (const void*)fine)
    return fail(LLSA_ERR_SHAPE, "llsa_expand_blocks cannot run in place");
  return hip_status(llsa::launch_expand_blocks(make_shape(p), sel1, fine, (hipStream_t)stream),
                    "llsa_expand_blocks");
}

int32_t llsa_attn_fwd(const llsa_problem* p, const void* q, const void* k, const void* v,
                      const float* const* k_lv, const float* const* v_lv,
                      const int32_t* const* sel, void* o, float* lse, void* stream) {
  int32_t st = check_problem(p);
  if (st != LLSA_OK) return st;
  if (p->head_dim == 128 && p->dtype != LLSA_BF16)
    return fail(LLSA_ERR_UNSUPPORTED, "the 128-channel attention is implemented for bf16");
  CHECK_PTR(q, "q");
  CHECK_PTR(k, "k");
  CHECK_PTR(v, "v");
  CHECK_PTR(o, "o");
  CHECK_PTR(lse, "lse");
  if (!sel) return fail(LLSA_ERR_NULL, "sel is NULL");
  for (int l = 1; l <= p->levels; ++l) {
    if (l > 1 + coarse_levels(p)) break;
    CHECK_PTR(sel[l - 1], "selection");
    if (l >= 2) {
      if (!k_lv || !v_lv) return fail(LLSA_ERR_NULL, "pooled levels are NULL");
      CHECK_PTR(k_lv[l - 1], "pooled k");
      CHECK_PTR(v_lv[l - 1], "pooled v");
    }
  }
  return hip_status(llsa::launch_attn_fwd(make_shape(p), q, k, v, k_lv, v_lv, sel, o, lse,
                                          (hipStream_t)stream),
                    "llsa_attn_fwd");
}

int32_t llsa_index_transpose_workspace(int32_t nmat, int32_t rows, int32_t cols, int32_t k,
                                       size_t* bytes) {
  if (!bytes) return fail(LLSA_ERR_NULL, "bytes is NULL");
  if (nmat < 1 || rows < 1 || cols < 1 || k < 1)
    return fail(LLSA_ERR_SHAPE, "nmat, rows, cols and k must be >= 1");
  if ((long)nmat * rows * k >= (1L << 31))
    return fail(LLSA_ERR_SHAPE, "nmat*rows*k must be < 2^31");
  const int rbits = log2i(rows);
  if (!llsa::transpose_uses_radix(rows, k) && (((unsigned long)cols + 1) << rbits > (1UL << 32)))
    return fail(LLSA_ERR_SHAPE, "(cols+1) * 2^ceil(log2 rows) exceeds 2^32");
  *bytes = llsa::transpose_workspace_bytes(nmat, rows, cols, k);
  return LLSA_OK;
}

int32_t llsa_index_transpose(int32_t nmat, int32_t rows, int32_t cols, int32_t k,
                             const int32_t* csr, int32_t* csc_off, int32_t* csc_rows,
                             void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  int32_t st = llsa_index_transpose_workspace(nmat, rows, cols, k, &need);
  if (st != LLSA_OK) return st;
  CHECK_PTR(csr, "csr");
  CHECK_PTR(csc_off, "csc_off");
  CHECK_PTR(csc_rows, "csc_rows");
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(LLSA_ERR_WORKSPACE, "workspace of %zu bytes needed (%zu given)", need, ws_bytes);
  if (ws) CHECK_PTR(ws, "ws");
  return hip_status(llsa::launch_index_transpose(nmat, rows, cols, k, csr, csc_off, csc_rows, ws,
                                                 (hipStream_t)stream),
                    "llsa_index_transpose");
}

}  // extern "C"

namespace {

// The transposes the backward reads: level 1 as 16-token blocks (rows = cols = N/16, k = K B /
// 16), levels 2 .. 1 + coarse levels as selected (rows = cols = n_l, k = K).
int transpose_levels(const llsa_problem* p, int* nmat, int* rows, int* cols, int* k) {
  const int nlev = 1 + coarse_levels(p);
  const int n = p->height * p->width;
  for (int l = 1; l <= nlev; ++l) {
    nmat[l - 1] = p->batch * p->heads;
    rows[l - 1] = cols[l - 1] = l == 1 ? n / 16 : n >> (log2i(p->block) * l);
    k[l - 1] = l == 1 ? p->topk * (p->block / 16) : p->topk;
  }
  return nlev;
}

}  // namespace

extern "C" {

int32_t llsa_index_transpose_levels_workspace(const llsa_problem* p, size_t* bytes) {
  int32_t st = check_problem(p);
  if (st != LLSA_OK) return st;
  if (!bytes) return fail(LLSA_ERR_NULL, "bytes is NULL");
  int nmat[LLSA_MAX_LEVELS], rows[LLSA_MAX_LEVELS], cols[LLSA_MAX_LEVELS], k[LLSA_MAX_LEVELS];
  const int nlev = transpose_levels(p, nmat, rows, cols, k);
  for (int l = 0; l < nlev; ++l) {
    size_t b = 0;
    st = llsa_index_transpose_workspace(nmat[l], rows[l], cols[l], k[l], &b);
    if (st != LLSA_OK) return st;
  }
  *bytes = llsa::transpose_sets_workspace_bytes(nlev, nmat, rows, cols, k);
  return LLSA_OK;
}

int32_t llsa_index_transpose_levels(const llsa_problem* p, const int32_t* const* sel,
                                    int32_t* const* csc_off, int32_t* const* csc_rows, void* ws,
                                    size_t ws_bytes, void* stream) {
  size_t need = 0;
  int32_t st = llsa_index_transpose_levels_workspace(p, &need);
  if (st != LLSA_OK) return st;
  if (!sel || !csc_off || !csc_rows) return fail(LLSA_ERR_NULL, "index arrays are NULL");
  int nmat[LLSA_MAX_LEVELS], rows[LLSA_MAX_LEVELS], cols[LLSA_MAX_LEVELS], k[LLSA_MAX_LEVELS];
  const int nlev = transpose_levels(p, nmat, rows, cols, k);
  for (int l = 0; l < nlev; ++l) {
    CHECK_PTR(sel[l], "selection");
    CHECK_PTR(csc_off[l], "csc_off");
    CHECK_PTR(csc_rows[l], "csc_rows");
  }
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(LLSA_ERR_WORKSPACE, "workspace of %zu bytes needed (%zu given)", need, ws_bytes);
  if (ws) CHECK_PTR(ws, "ws");
  return hip_status(llsa::launch_transpose_sets(nlev, nmat, rows, cols, k, sel, csc_off, csc_rows,
                                                ws, (hipStream_t)stream),
                    "llsa_index_transpose_levels");
}

}  // extern "C"

namespace {

// Validation shared by llsa_attn_bwd and llsa_attn_bwd_noalloc (everything but the workspace).
int32_t check_bwd(const llsa_problem* p, const void* q, const void* k, const void* v,
                  const void* dout, const float* lse, const float* const* k_lv,
                  const float* const* v_lv, const int32_t* const* sel,
                  const int32_t* const* csc_off, const int32_t* const* csc_rows, void* dq,
                  void* dk, void* dv) {
  int32_t st = check_problem(p);
  if (st != LLSA_OK) return st;
  if (p->dtype != LLSA_BF16)
    return fail(LLSA_ERR_UNSUPPORTED, "the backward is implemented for bf16 only");
  if (coarse_levels(p) * p->topk > 32)
    return fail(LLSA_ERR_UNSUPPORTED, "backward supports at most 32 coarse keys per query "
                "(coarse levels * topk = %d)", coarse_levels(p) * p->topk);
  {
    // its level-1 index transpose packs (key block, query block) into 32-bit codes
    const unsigned long n1 = (unsigned long)p->height * p->width / 16;
    int rb = 0;
    while ((1UL << rb) < n1) ++rb;
    if (((n1 + 1) << rb) > (1UL << 32))
      return fail(LLSA_ERR_UNSUPPORTED, "the backward supports N <= 2^19 tokens per head "
                  "(N = %lu)", n1 * 16);
  }
  CHECK_PTR(q, "q");
  CHECK_PTR(k, "k");
  CHECK_PTR(v, "v");
  CHECK_PTR(dout, "dout");
  CHECK_PTR(lse, "lse");
  CHECK_PTR(dq, "dq");
  CHECK_PTR(dk, "dk");
  CHECK_PTR(dv, "dv");
  if (!sel || !csc_off || !csc_rows) return fail(LLSA_ERR_NULL, "index arrays are NULL");
  for (int l = 1; l <= p->levels; ++l) {
    if (l > 1 + coarse_levels(p)) break;
    CHECK_PTR(sel[l - 1], "selection");
    CHECK_PTR(csc_off[l - 1], "csc_off");
    CHECK_PTR(csc_rows[l - 1], "csc_rows");
    if (l >= 2) {
      if (!k_lv || !v_lv) return fail(LLSA_ERR_NULL, "pooled levels are NULL");
      CHECK_PTR(k_lv[l - 1], "pooled k");
      CHECK_PTR(v_lv[l - 1], "pooled v");
    }
  }
  return LLSA_OK;
}

}  // namespace

extern "C" {

int32_t llsa_attn_bwd(const llsa_problem* p, const void* q, const void* k, const void* v,
                      const void* dout, const float* lse,
                      const float* const* k_lv, const float* const* v_lv,
                      const int32_t* const* sel, const int32_t* const* csc_off,
                      const int32_t* const* csc_rows, void* dq, void* dk, void* dv, void* ws,
                      size_t ws_bytes, void* stream) {
  int32_t st = check_bwd(p, q, k, v, dout, lse, k_lv, v_lv, sel, csc_off, csc_rows, dq, dk, dv);
  if (st != LLSA_OK) return st;
  const llsa::Shape s = make_shape(p);
  const size_t need = llsa::bwd_workspace_bytes(s);
  if (!ws || ws_bytes < need)
    return fail(LLSA_ERR_WORKSPACE, "workspace of %zu bytes needed (%zu given)", need, ws_bytes);
  CHECK_PTR(ws, "ws");
  return hip_status(llsa::launch_attn_bwd(s, q, k, v, dout, lse, k_lv, v_lv, sel, csc_off,
                                          csc_rows, nullptr, dq, dk, dv, ws,
                                          (hipStream_t)stream),
                    "llsa_attn_bwd");
}

int32_t llsa_attn_bwd_noalloc(const llsa_problem* p, const void* q, const void* k,
                              const void* v, const void* dout, const float* lse,
                              const float* const* k_lv, const float* const* v_lv,
                              const int32_t* const* sel, const int32_t* const* csc_off,
                              const int32_t* const* csc_rows, void* dq, void* dk, void* dv,
                              void* stream) {
  int32_t st = check_bwd(p, q, k, v, dout, lse, k_lv, v_lv, sel, csc_off, csc_rows, dq, dk, dv);
  if (st != LLSA_OK) return st;
  const llsa::Shape s = make_shape(p);
  const size_t need = llsa::bwd_workspace_bytes(s);
  if (need > (size_t)LLSA_NOALLOC_SCRATCH_BYTES)
    return fail(LLSA_ERR_WORKSPACE, "this problem needs %zu bytes of backward workspace; the "
                "allocation-free entry holds at most %zu: use llsa_attn_bwd with a workspace",
                need, (size_t)LLSA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  st = hip_status(llsa::noalloc_scratch(&ws), "llsa_attn_bwd_noalloc: scratch address");
  if (st != LLSA_OK) return st;
  return hip_status(llsa::launch_attn_bwd(s, q, k, v, dout, lse, k_lv, v_lv, sel, csc_off,
                                          csc_rows, nullptr, dq, dk, dv, ws,
                                          (hipStream_t)stream),
                    "llsa_attn_bwd_noalloc");
}

}  // extern "C"

namespace {

// The mask-based comparator: bf16, no coarse keys, and a mask of at most 2^34 bytes.
int32_t check_masked(const llsa_problem* p) {
  int32_t st = check_problem(p);
  if (st != LLSA_OK) return st;
  if (p->dtype != LLSA_BF16)
    return fail(LLSA_ERR_UNSUPPORTED, "the mask-based backward is implemented for bf16 only");
  if (coarse_levels(p) > 0)
    return fail(LLSA_ERR_UNSUPPORTED, "the mask-based backward has no coarse keys: levels must "
                "be 1 or enrich 0");
  if (p->block != 16)
    return fail(LLSA_ERR_UNSUPPORTED, "the mask-based backward is implemented for block 16");
  if (p->head_dim != 64)
    return fail(LLSA_ERR_UNSUPPORTED, "the mask-based backward is implemented for head_dim 64");
  const long n1 = (long)p->height * p->width / 16;
  if ((long)p->batch * p->heads * n1 * n1 > (1L << 34))
    return fail(LLSA_ERR_SHAPE, "block mask of %ld bytes exceeds 2^34",
                (long)p->batch * p->heads * n1 * n1);
  return LLSA_OK;
}

}  // namespace

extern "C" {

int32_t llsa_calib_copy(const void* src, void* dst, size_t bytes, void* stream) {
  CHECK_PTR(src, "src");
  CHECK_PTR(dst, "dst");
  if (bytes == 0 || bytes % 16 != 0 || bytes > ((size_t)1 << 40))
    return fail(LLSA_ERR_SHAPE, "bytes = %zu: a nonzero multiple of 16 up to 2^40 is needed",
                bytes);
  if (src == dst) return fail(LLSA_ERR_SHAPE, "the copy cannot run in place");
  return hip_status(llsa::launch_calib_copy(src, dst, bytes, (hipStream_t)stream),
                    "llsa_calib_copy");
}

int32_t llsa_calib_mfma(float* out, int32_t blocks, int32_t iters, void* stream) {
  CHECK_PTR(out, "out");
  if (blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 16))
    return fail(LLSA_ERR_SHAPE, "blocks in [1, 2^20] and iters in [1, 2^16] are needed");
  return hip_status(llsa::launch_calib_mfma(out, blocks, iters, (hipStream_t)stream),
                    "llsa_calib_mfma");
}

int32_t llsa_block_mask(const llsa_problem* p, const int32_t* sel1, uint8_t* mask,
                        void* stream) {
  int32_t st = check_masked(p);
  if (st != LLSA_OK) return st;
  CHECK_PTR(sel1, "sel1");
  CHECK_PTR(mask, "mask");
  return hip_status(llsa::launch_block_mask(make_shape(p), sel1, mask, (hipStream_t)stream),
                    "llsa_block_mask");
}

int32_t llsa_attn_bwd_masked(const llsa_problem* p, const void* q, const void* k, const void* v,
                             const void* dout, const float* lse, const int32_t* sel1,
                             const uint8_t* mask, void* dq, void* dk, void* dv, void* ws,
                             size_t ws_bytes, void* stream) {
  int32_t st = check_masked(p);
  if (st != LLSA_OK) return st;
  CHECK_PTR(q, "q");
  CHECK_PTR(k, "k");
  CHECK_PTR(v, "v");
  CHECK_PTR(dout, "dout");
  CHECK_PTR(lse, "lse");
  CHECK_PTR(sel1, "sel1");
  CHECK_PTR(mask, "mask");
  CHECK_PTR(dq, "dq");
  CHECK_PTR(dk, "dk");
  CHECK_PTR(dv, "dv");
  const llsa::Shape s = make_shape(p);
  const size_t need = llsa::bwd_workspace_bytes(s);
  if (!ws || ws_bytes < need)
    return fail(LLSA_ERR_WORKSPACE, "workspace of %zu bytes needed (%zu given)", need, ws_bytes);
  CHECK_PTR(ws, "ws");
  const int32_t* sel[LLSA_MAX_LEVELS] = {sel1};
  const int32_t* none[LLSA_MAX_LEVELS] = {};
  return hip_status(llsa::launch_attn_bwd(s, q, k, v, dout, lse, nullptr, nullptr, sel, none,
                                          none, mask, dq, dk, dv, ws, (hipStream_t)stream),
                    "llsa_attn_bwd_masked");
}

}  // extern "C"

namespace {

int32_t check_dense(int32_t batch_heads, int32_t n, int32_t head_dim, float scale) {
  if (batch_heads < 1) return fail(LLSA_ERR_SHAPE, "batch_heads %d must be >= 1", batch_heads);
  if (head_dim != 64)
    return fail(LLSA_ERR_UNSUPPORTED, "head_dim %d: only 64 is implemented", head_dim);
  if (n < 128 || n % 128 != 0 || n > (1 << 23))
    return fail(LLSA_ERR_SHAPE, "N = %d: a multiple of 128 in [128, 2^23] is needed", n);
  if ((long)batch_heads * n >= (1L << 31))
    return fail(LLSA_ERR_SHAPE, "batch_heads*N must be < 2^31");
  if (!(scale >= 0.f) || std::isinf(scale))
    return fail(LLSA_ERR_SHAPE, "scale must be finite and >= 0");
  return LLSA_OK;
}

}  // namespace

extern "C" {

int32_t llsa_dense_attn_fwd(int32_t batch_heads, int32_t n, int32_t head_dim, float scale,
                            const void* q, const void* k, const void* v, void* o, float* lse,
                            void* stream) {
  int32_t st = check_dense(batch_heads, n, head_dim, scale);
  if (st != LLSA_OK) return st;
  CHECK_PTR(q, "q");
  CHECK_PTR(k, "k");
  CHECK_PTR(v, "v");
  CHECK_PTR(o, "o");
  CHECK_PTR(lse, "lse");
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)head_dim);
  return hip_status(llsa::launch_dense_fwd(batch_heads, n, sc, q, k, v, o, lse,
                                           (hipStream_t)stream),
                    "llsa_dense_attn_fwd");
}

int32_t llsa_dense_attn_bwd(int32_t batch_heads, int32_t n, int32_t head_dim, float scale,
                            const void* q, const void* k, const void* v, const void* dout,
                            const float* lse, void* dq, void* dk, void* dv, float* d_rows,
                            void* stream) {
  int32_t st = check_dense(batch_heads, n, head_dim, scale);
  if (st != LLSA_OK) return st;
  CHECK_PTR(q, "q");
  CHECK_PTR(k, "k");
  CHECK_PTR(v, "v");
  CHECK_PTR(dout, "dout");
  CHECK_PTR(lse, "lse");
  CHECK_PTR(dq, "dq");
  CHECK_PTR(dk, "dk");
  CHECK_PTR(dv, "dv");
  CHECK_PTR(d_rows, "d_rows");
  const float sc = scale > 0.f ? scale : 1.0f / std::sqrt((float)head_dim);
  return hip_status(llsa::launch_dense_bwd(batch_heads, n, sc, q, k, v, dout, lse, dq, dk, dv,
                                           d_rows, (hipStream_t)stream),
                    "llsa_dense_attn_bwd");
}

}  // extern "C"
