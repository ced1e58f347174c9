"""Plain, slow, fp64 CPU oracle for Log-linear Sparse Attention (LLSA).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the package entry point
and the benchmark's CPU-baseline leg may import this module.  The HIP library never calls it,
and it shares no code with the HIP library (it imports numpy only).

Sources (pages on the method; cited by title and section):
  [SUM] "Trainable Log-linear Sparse Attention for Efficient Diffusion Transformers",
        structured paper summary (mhpq.cn news 1142837):
        sec. 三 Hierarchical Top-K (recursive mean pooling, coarsest full QK^T + top-K,
        coarse-to-fine re-ranking over the K*B children), sec. 四 Hierarchical KV Enrichment
        (fine top-K KV plus coarse KV of several levels, KV reweighting W^(l) = B^l),
        sec. 4.1 (sparse backward through a CSR->CSC sparse index transpose),
        sec. 4.2 / Figure 2 (2D index reordering before pooling).
  [ART] Popular article on arXiv:2512.16615 (m.admirer.cn): sec. 三 (hierarchical top-K,
        KV enrichment, reweighting by the level's block size), sec. 四 (gather of selected
        blocks in the forward; key-major index via per-key counts and offsets; reordering
        "like Z-order or Hilbert curves").

Readings where the pages are silent or garbled (each is listed in the design notes):
  * tokens are reordered along the Morton (Z-order) curve, x (column) bits in even
    positions, so every aligned run of 4^m tokens is a 2^m x 2^m tile;
  * softmax scale 1/sqrt(d); a coarse key of level l gets weight B^l, i.e. its exp(score)
    is multiplied by B^l (logit bias l*ln B);
  * top-K ties go to the lower key id; selected ids are stored ascending;
  * ranking scores are plain dot products of pooled Q_l and pooled K_l;
  * enrichment adds, for every level l = 2..L, the K keys selected at level l for the query
    block's level-l ancestor; no de-duplication against the fine keys;
  * variants (switches, not the method's default): enrich_levels = m keeps only the coarse
    levels 2..1+m (the finest m; 0 = all), coarse_weight False gives every coarse key weight 1
    instead of B^l, exclude_overlap drops a coarse key whose span holds a key the query block
    already attends one level finer (a fine block for level 2, a level-(l-1) coarse key
    otherwise), so that no region is covered twice;
  * gradients flow to Q, K, V and through the pooled K/V of the coarse keys (chain rule of
    the mean), not through the top-K selection or the pooled Q.

Arrays are float64; tokens are [..., N, d].  Per-head functions take a single head [N, d].
"""
from __future__ import annotations

import math
from typing import Sequence

import numpy as np

# --------------------------------------------------------------------------------------
# 2D index reordering  ([SUM] sec. 4.2 / Figure 2; [ART] sec. 四)
# --------------------------------------------------------------------------------------


def _log2_exact(n: int) -> int:
    p = int(n).bit_length() - 1
    if n <= 0 or (1 << p) != n:
        raise ValueError(f"{n} is not a power of two")
    return p


def morton_perm(height: int, width: int) -> np.ndarray:
    """perm[m] = raster index (y*width + x) of the token at Morton position m.

    Position m's low 2r bits (r = min(log2 H, log2 W)) are de-interleaved: bit 2i is bit i
    of x, bit 2i+1 is bit i of y.  The remaining high bits of m extend the longer side.
    """
    p, q = _log2_exact(height), _log2_exact(width)
    r = min(p, q)
    m = np.arange(height * width, dtype=np.int64)
    x = np.zeros_like(m)
    y = np.zeros_like(m)
    for i in range(r):
        x |= ((m >> (2 * i)) & 1) << i
        y |= ((m >> (2 * i + 1)) & 1) << i
    high = m >> (2 * r)
    if q > p:
        x |= high << r
    elif p > q:
        y |= high << r
    return y * width + x


def reorder(x: np.ndarray, height: int, width: int, inverse: bool = False) -> np.ndarray:
    """Raster -> Morton (y[..., m, :] = x[..., perm[m], :]) or its inverse."""
    perm = morton_perm(height, width)
    if not inverse:
        return x[..., perm, :].copy()
    out = np.empty_like(x)
    out[..., perm, :] = x
    return out


# --------------------------------------------------------------------------------------
# Hierarchical compression: recursive mean pooling  ([SUM] sec. 三)
# --------------------------------------------------------------------------------------


def pool_levels(x: np.ndarray, block: int, levels: int) -> list:
    """[X_1, ..., X_L]: X_l[j] = mean of the `block` level-(l-1) tokens jB..jB+B-1."""
    out = []
    cur = x
    for _ in range(levels):
        n = cur.shape[-2]
        if n % block:
            raise ValueError("sequence length is not divisible by the block size")
        cur = cur.reshape(*cur.shape[:-2], n // block, block, cur.shape[-1]).mean(axis=-2)
        out.append(cur)
    return out


# --------------------------------------------------------------------------------------
# Coarse-to-fine top-K selection  ([SUM] sec. 三; [ART] sec. 三)
# --------------------------------------------------------------------------------------


def topk_ids(scores: np.ndarray, cand: np.ndarray, k: int) -> np.ndarray:
    """The k candidate ids with the largest scores (ties: lower id first), ascending.

    scores: [rows, C]; cand: [C] or [rows, C] candidate key ids.
    """
    cand = np.broadcast_to(cand, scores.shape)
    # order candidates by id first so that the stable sort on -score breaks ties by id
    by_id = np.argsort(cand, axis=-1, kind="stable")
    cand_s = np.take_along_axis(cand, by_id, axis=-1)
    score_s = np.take_along_axis(scores, by_id, axis=-1)
    best = np.argsort(-score_s, axis=-1, kind="stable")[:, :k]
    return np.sort(np.take_along_axis(cand_s, best, axis=-1), axis=-1)


def select_coarsest(q_top: np.ndarray, k_top: np.ndarray, k: int) -> np.ndarray:
    """Coarsest level: full Q_L K_L^T, then top-k per row.  [n_L, k] int64."""
    scores = q_top @ k_top.T
    return topk_ids(scores, np.arange(k_top.shape[0]), k)


def select_level(q_l: np.ndarray, k_l: np.ndarray, parent_sel: np.ndarray, block: int,
                 k: int) -> np.ndarray:
    """Level l < L: query a re-ranks the children {c*B + t} of its parent's picks.

    parent_sel: [n_l / B, K_{l+1}] ids at level l+1.  Returns [n_l, k] int64.
    All B sibling queries of a parent share one candidate list.
    """
    n_l = q_l.shape[0]
    out = np.empty((n_l, k), dtype=np.int64)
    t = np.arange(block)
    for parent in range(n_l // block):
        cand = (parent_sel[parent][:, None] * block + t[None, :]).reshape(-1)
        rows = slice(parent * block, (parent + 1) * block)
        scores = q_l[rows] @ k_l[cand].T
        out[rows] = topk_ids(scores, cand, k)
    return out


def select(q_lv: Sequence[np.ndarray], k_lv: Sequence[np.ndarray], block: int,
           topk) -> list:
    """Per-head selection for levels 1..L: returns [Sel_1, ..., Sel_L].

    topk: an int, or per-level ints [K_1, ..., K_L] (to let K cover every candidate).
    """
    levels = len(q_lv)
    ks = [topk] * levels if np.isscalar(topk) else list(topk)
    sel = [None] * levels
    sel[levels - 1] = select_coarsest(q_lv[-1], k_lv[-1], ks[-1])
    for l in range(levels - 1, 0, -1):          # level index l (1-based) = l
        sel[l - 1] = select_level(q_lv[l - 1], k_lv[l - 1], sel[l], block, ks[l - 1])
    return sel


# --------------------------------------------------------------------------------------
# Sparse attention with hierarchical KV enrichment  ([SUM] sec. 四; [ART] sec. 三/四)
# --------------------------------------------------------------------------------------


def key_list(p: int, k: np.ndarray, v: np.ndarray, k_lv, v_lv, sel, block: int,
             enrich: bool, enrich_levels: int = 0, coarse_weight: bool = True,
             exclude_overlap: bool = False):
    """Keys, values and log-weights attended by level-1 query block p.

    Fine: every token of the K blocks in Sel_1[p] (log-weight 0).
    Coarse (enrich): for l = 2..L, the keys Sel_l[a] of block p's level-l ancestor
    a = p // B^(l-1), each with weight B^l (log-weight l*ln B).  Variants: enrich_levels m > 0
    stops at level min(L, 1 + m); coarse_weight False uses weight 1 (log-weight 0);
    exclude_overlap drops a level-l key that is the parent of one of the keys selected one
    level finer for p (Sel_1[p] for l = 2, Sel_(l-1) of p's level-(l-1) ancestor above).
    Also returns the identity of every key: (level, index), level 0 = fine token.
    """
    keys, vals, logw, ident = [], [], [], []
    for j in sel[0][p]:
        toks = np.arange(j * block, (j + 1) * block)
        keys.append(k[toks])
        vals.append(v[toks])
        logw.append(np.zeros(block))
        ident += [(0, int(t)) for t in toks]
    if enrich:
        top = len(sel) if not enrich_levels else min(len(sel), 1 + enrich_levels)
        for l in range(2, top + 1):
            a = p // block ** (l - 1)
            ids = sel[l - 1][a]
            if exclude_overlap:
                finer = sel[l - 2][p // block ** (l - 2)]
                covered = {int(x) // block for x in finer}
                ids = np.array([j for j in ids if int(j) not in covered], dtype=np.int64)
            keys.append(k_lv[l - 1][ids])
            vals.append(v_lv[l - 1][ids])
            logw.append(np.full(len(ids), l * math.log(block) if coarse_weight else 0.0))
            ident += [(l, int(j)) for j in ids]
    return np.concatenate(keys), np.concatenate(vals), np.concatenate(logw), ident


def attention_forward(q, k, v, k_lv, v_lv, sel, block: int, enrich: bool = True,
                      scale: float | None = None, blocks=None, enrich_levels: int = 0,
                      coarse_weight: bool = True, exclude_overlap: bool = False):
    """Per-head forward in Morton order.  Returns (o [N, d], lse [N]) (rows of `blocks` only
    are filled when `blocks` is given; the rest stay NaN).

    o_i = sum_e w_e exp(s_e) v_e / sum_e w_e exp(s_e), s_e = scale * q_i.k_e,
    lse_i = log sum_e w_e exp(s_e)  (natural log, weights included).
    """
    n, d = q.shape
    scale = 1.0 / math.sqrt(d) if not scale else scale
    o = np.full((n, d), np.nan)
    lse = np.full(n, np.nan)
    nblk = n // block
    for p in (range(nblk) if blocks is None else blocks):
        kk, vv, logw, _ = key_list(p, k, v, k_lv, v_lv, sel, block, enrich, enrich_levels,
                                   coarse_weight, exclude_overlap)
        rows = slice(p * block, (p + 1) * block)
        s = scale * (q[rows] @ kk.T) + logw[None, :]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        o[rows] = (e @ vv) / z
        lse[rows] = (m + np.log(z))[:, 0]
    return o, lse


def attention_backward(q, k, v, k_lv, v_lv, sel, do, block: int, enrich: bool = True,
                       scale: float | None = None, enrich_levels: int = 0,
                       coarse_weight: bool = True, exclude_overlap: bool = False,
                       blocks=None):
    """Per-head gradients (dq, dk, dv) in Morton order, given upstream dO.  With `blocks`,
    only those level-1 query blocks contribute: their dq rows are exact, and dk/dv hold the
    sum of their contributions (exact for a key all of whose queries are in `blocks`).

    Softmax Jacobian per query: P_e = w_e exp(s_e) / Z, dP_e = dO.v_e,
    dS_e = P_e (dP_e - sum_f P_f dP_f); dq = scale * sum_e dS_e k_e;
    fine key e: dk_e += scale * dS_e q, dv_e += P_e dO;
    coarse key (l, j): the same into dK_l[j], dV_l[j], then each of the B^l fine tokens it
    averages receives dK_l[j] / B^l (chain rule of the mean).  No gradient through the
    selection or the pooled Q.
    """
    n, d = q.shape
    scale = 1.0 / math.sqrt(d) if not scale else scale
    levels = len(sel)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dk_lv = [np.zeros_like(x) for x in k_lv]
    dv_lv = [np.zeros_like(x) for x in v_lv]
    for p in (range(n // block) if blocks is None else blocks):
        kk, vv, logw, ident = key_list(p, k, v, k_lv, v_lv, sel, block, enrich, enrich_levels,
                                       coarse_weight, exclude_overlap)
        rows = slice(p * block, (p + 1) * block)
        s = scale * (q[rows] @ kk.T) + logw[None, :]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        prob = e / e.sum(axis=1, keepdims=True)
        dprob = do[rows] @ vv.T
        ds = prob * (dprob - (prob * dprob).sum(axis=1, keepdims=True))
        dq[rows] = scale * (ds @ kk)
        gk = scale * (ds.T @ q[rows])
        gv = prob.T @ do[rows]
        for col, (lvl, idx) in enumerate(ident):
            if lvl == 0:
                dk[idx] += gk[col]
                dv[idx] += gv[col]
            else:
                dk_lv[lvl - 1][idx] += gk[col]
                dv_lv[lvl - 1][idx] += gv[col]
    for l in range(2, levels + 1 if enrich else 2):   # coarse keys only with enrichment
        span = block ** l
        dk += np.repeat(dk_lv[l - 1], span, axis=0) / span
        dv += np.repeat(dv_lv[l - 1], span, axis=0) / span
    return dq, dk, dv


# --------------------------------------------------------------------------------------
# Dense softmax attention: the full-attention baseline the pages compare against
# ([SUM] sec. 5.4 / Figure 3: speed-up over dense FlashAttention at the same length)
# --------------------------------------------------------------------------------------


def dense_attention_forward(q, k, v, scale: float | None = None):
    """Per-head dense attention over all keys: (o [N, d], lse [N]).

    o = softmax(scale q k^T) v row by row; lse = log sum_j exp(scale q_i.k_j).
    """
    d = q.shape[1]
    scale = 1.0 / math.sqrt(d) if not scale else scale
    s = scale * (q @ k.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    return (e @ v) / z, (m + np.log(z))[:, 0]


def dense_attention_backward(q, k, v, do, scale: float | None = None):
    """Per-head gradients (dq, dk, dv) of dense attention given upstream dO.

    P = softmax(scale q k^T), dP = dO v^T, dS = P (dP - rowsum(P dP)),
    dq = scale dS k, dk = scale dS^T q, dv = P^T dO.
    """
    d = q.shape[1]
    scale = 1.0 / math.sqrt(d) if not scale else scale
    s = scale * (q @ k.T)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    prob = e / e.sum(axis=1, keepdims=True)
    dprob = do @ v.T
    ds = prob * (dprob - (prob * dprob).sum(axis=1, keepdims=True))
    return scale * (ds @ k), scale * (ds.T @ q), prob.T @ do


# --------------------------------------------------------------------------------------
# Sparse index transpose: CSR -> CSC  ([SUM] sec. 4.1; [ART] sec. 四)
# --------------------------------------------------------------------------------------


def csr_to_csc(sel: np.ndarray, n_cols: int):
    """Key-major inverse of a fixed-K row index.

    Per-key counts, exclusive prefix sum into offsets, then a stable scatter of the row
    ids by key (rows ascending within a key).  Returns (off [n_cols+1], rows [nnz]).
    """
    n_rows, kk = sel.shape
    keys = sel.reshape(-1)
    counts = np.bincount(keys, minlength=n_cols)
    off = np.zeros(n_cols + 1, dtype=np.int64)
    off[1:] = np.cumsum(counts)
    fill = off[:-1].copy()
    rows = np.empty(keys.size, dtype=np.int64)
    for e in range(keys.size):            # entries in row-major order => stable
        c = keys[e]
        rows[fill[c]] = e // kk
        fill[c] += 1
    return off, rows


# --------------------------------------------------------------------------------------
# Whole path over [batch, heads, N, d] raster-order tensors
# --------------------------------------------------------------------------------------


def llsa_forward(q, k, v, height: int, width: int, block: int, levels: int, topk,
                 enrich: bool = True, scale: float | None = None, sel_override=None,
                 enrich_levels: int = 0, coarse_weight: bool = True,
                 exclude_overlap: bool = False):
    """Full forward: reorder -> pool -> select -> attention -> inverse reorder.

    Returns a dict with o (raster), lse (Morton order, [b, H, N]), and the Morton-order
    intermediates: qm, km, vm, q_lv, k_lv, v_lv (lists over levels), sel ([b][H] lists).
    sel_override[b][h], when given, replaces the selection (attention on given indices).
    """
    b, hh, n, d = q.shape
    qm, km, vm = (reorder(t, height, width) for t in (q, k, v))
    q_lv, k_lv, v_lv = (pool_levels(t, block, levels) for t in (qm, km, vm))
    om = np.empty_like(qm)
    lse = np.empty((b, hh, n))
    sels = []
    for bi in range(b):
        row = []
        for hi in range(hh):
            ql = [x[bi, hi] for x in q_lv]
            kl = [x[bi, hi] for x in k_lv]
            vl = [x[bi, hi] for x in v_lv]
            sel = (select(ql, kl, block, topk) if sel_override is None
                   else sel_override[bi][hi])
            om[bi, hi], lse[bi, hi] = attention_forward(
                qm[bi, hi], km[bi, hi], vm[bi, hi], kl, vl, sel, block, enrich, scale,
                enrich_levels=enrich_levels, coarse_weight=coarse_weight,
                exclude_overlap=exclude_overlap)
            row.append(sel)
        sels.append(row)
    return dict(o=reorder(om, height, width, inverse=True), om=om, lse=lse, qm=qm, km=km,
                vm=vm, q_lv=q_lv, k_lv=k_lv, v_lv=v_lv, sel=sels)


def llsa_backward(q, k, v, do, height: int, width: int, block: int, levels: int, sels,
                  enrich: bool = True, scale: float | None = None, enrich_levels: int = 0,
                  coarse_weight: bool = True, exclude_overlap: bool = False):
    """Full backward on the forward's selection: returns raster-order (dq, dk, dv)."""
    qm, km, vm, dom = (reorder(t, height, width) for t in (q, k, v, do))
    k_lv, v_lv = (pool_levels(t, block, levels) for t in (km, vm))
    dq, dk, dv = (np.empty_like(qm) for _ in range(3))
    for bi in range(q.shape[0]):
        for hi in range(q.shape[1]):
            kl = [x[bi, hi] for x in k_lv]
            vl = [x[bi, hi] for x in v_lv]
            dq[bi, hi], dk[bi, hi], dv[bi, hi] = attention_backward(
                qm[bi, hi], km[bi, hi], vm[bi, hi], kl, vl, sels[bi][hi], dom[bi, hi], block,
                enrich, scale, enrich_levels, coarse_weight, exclude_overlap)
    return tuple(reorder(t, height, width, inverse=True) for t in (dq, dk, dv))


def selection_candidates(n: int, block: int, levels: int, k: int) -> int:
    """Number of (query, key) scores the coarse-to-fine selection evaluates.

    Coarsest level: n_L^2; every finer level l < L: n_l * K * B  ([SUM] sec. 三).
    """
    n_top = n // block ** levels
    return n_top * n_top + sum((n // block ** l) * k * block for l in range(1, levels))
