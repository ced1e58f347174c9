"""Pins for the CPU oracle: each check ties it to something other than itself.

Sources: [SUM] "Trainable Log-linear Sparse Attention for Efficient Diffusion Transformers"
(paper summary: sec. 三 hierarchical top-K, sec. 四 KV enrichment and reweighting, sec. 4.1
sparse index transpose, sec. 4.2 2D reordering); [ART] popular article on arXiv:2512.16615
(sec. 三, 四).  The pages print no worked numerical example, so the pins are closed forms,
invariants, library routines (scipy sparse transpose, torch's scaled_dot_product_attention
and autograd in float64, Python's sort) and brute force on tiny inputs.
"""
import math
import os

import numpy as np
import pytest
import scipy.sparse
import torch

from oracle import llsa_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_ints(name):
    with open(os.path.join(GOLDEN, name)) as f:
        rows = [ln for ln in f if ln.strip() and not ln.startswith("#")]
    return np.array([int(t) for ln in rows for t in ln.split()], dtype=np.int64)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ----------------------------------------------------------------------------- reorder


def test_morton_golden_4x4():
    assert np.array_equal(orc.morton_perm(4, 4), _golden_ints("zorder_4x4.txt"))


def test_morton_golden_2x4():
    assert np.array_equal(orc.morton_perm(2, 4), _golden_ints("zorder_2x4.txt"))


@pytest.mark.parametrize("h,w", [(16, 16), (64, 64), (32, 64), (64, 16), (128, 128)])
def test_morton_is_bijection(h, w):
    perm = orc.morton_perm(h, w)
    assert np.array_equal(np.sort(perm), np.arange(h * w))


@pytest.mark.parametrize("h,w,side", [(16, 16, 4), (64, 64, 4), (64, 64, 16), (128, 128, 16),
                                      (32, 64, 4), (64, 32, 16)])
def test_morton_runs_are_square_tiles(h, w, side):
    """Every aligned run of side^2 curve positions covers one aligned side x side tile."""
    perm = orc.morton_perm(h, w)
    run = side * side
    for start in range(0, h * w, run):
        ys, xs = np.divmod(perm[start:start + run], w)
        assert ys.max() - ys.min() == side - 1 and xs.max() - xs.min() == side - 1
        assert ys.min() % side == 0 and xs.min() % side == 0
        assert len(set(zip(ys.tolist(), xs.tolist()))) == run


def test_reorder_inverse_roundtrip():
    x = _rand((2, 3, 256, 5), 1)
    y = orc.reorder(x, 16, 16)
    assert np.array_equal(orc.reorder(y, 16, 16, inverse=True), x)
    assert np.array_equal(y[0, 0, 2], x[0, 0, 16])     # position 2 is (x=0, y=1)


# ----------------------------------------------------------------------------- pooling


def test_pool_closed_form():
    x = np.arange(16, dtype=np.float64)[:, None]          # tokens 0..15, d = 1
    l1, l2 = orc.pool_levels(x, 4, 2)
    assert np.allclose(l1[:, 0], [1.5, 5.5, 9.5, 13.5])
    assert np.allclose(l2[:, 0], [7.5])


def test_pool_direct_mean_and_global_mean():
    x = _rand((2, 2, 4096, 8), 2)
    lv = orc.pool_levels(x, 16, 3)
    for l, xl in enumerate(lv, start=1):
        span = 16 ** l
        direct = x.reshape(2, 2, 4096 // span, span, 8).mean(axis=3)   # non-recursive
        assert np.allclose(xl, direct, rtol=0, atol=1e-12)
        assert np.allclose(xl.mean(axis=2), x.mean(axis=2), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- selection


def _python_topk(scores_row, allowed, k):
    """Brute force with Python's sort: largest score first, ties to the lower id."""
    ids = sorted((j for j in range(len(scores_row)) if allowed[j]),
                 key=lambda j: (-scores_row[j], j))[:k]
    return sorted(ids)


def test_single_level_is_plain_block_topk():
    """L = 1 is the single-level top-K baseline: exhaustive top-K over all blocks."""
    q = _rand((256, 8), 3)
    k = _rand((256, 8), 4)
    ql, kl = orc.pool_levels(q, 16, 1), orc.pool_levels(k, 16, 1)
    sel = orc.select(ql, kl, 16, 5)
    s = ql[0] @ kl[0].T
    for a in range(16):
        assert list(sel[0][a]) == _python_topk(s[a], [True] * 16, 5)


def test_hierarchical_selection_equals_masked_dense_topk():
    """Each level equals a top-K over ALL keys of that level, masked to the children of the
    parent's picks (a dense-mask formulation of the same rule)."""
    q = _rand((65536, 6), 5)
    k = _rand((65536, 6), 6)
    B, L, K = 16, 3, 3
    ql, kl = orc.pool_levels(q, B, L), orc.pool_levels(k, B, L)
    sel = orc.select(ql, kl, B, K)
    top = ql[-1] @ kl[-1].T
    for a in range(top.shape[0]):
        assert list(sel[-1][a]) == _python_topk(top[a], [True] * top.shape[1], K)
    for l in range(L - 1, 0, -1):
        s = ql[l - 1] @ kl[l - 1].T
        for a in range(0, s.shape[0], 37):
            parents = set(sel[l][a // B].tolist())
            allowed = [(c // B) in parents for c in range(s.shape[1])]
            assert list(sel[l - 1][a]) == _python_topk(s[a], allowed, K)


def test_selection_closed_form_monotone_keys():
    """Keys whose projection on u grows with position: queries along +u (first half of the
    sequence) pick the last K ids at every level, queries along -u the first K."""
    n, B, L, K = 65536, 16, 3, 4
    u = np.array([1.0, 0.0, 0.0, 0.0])
    k = np.outer(np.arange(n, dtype=np.float64) + 1.0, u)
    q = np.outer(np.where(np.arange(n) < n // 2, 1.0, -1.0), u)
    ql, kl = orc.pool_levels(q, B, L), orc.pool_levels(k, B, L)
    sel = orc.select(ql, kl, B, K)
    for l in range(1, L + 1):
        nl = n // B ** l
        for a in range(nl):
            want = list(range(nl - K, nl)) if a < nl // 2 else list(range(K))
            assert list(sel[l - 1][a]) == want, (l, a)


def test_selection_ties_go_to_lower_id():
    q = np.ones((256, 2))
    k = np.ones((256, 2))
    ql, kl = orc.pool_levels(q, 16, 1), orc.pool_levels(k, 16, 1)
    sel = orc.select(ql, kl, 16, 3)
    assert all(list(r) == [0, 1, 2] for r in sel[0])


def test_selection_subset_sorted_distinct():
    q = _rand((1024, 8), 7)
    k = _rand((1024, 8), 8)
    B, L, K = 4, 3, 5
    ql, kl = orc.pool_levels(q, B, L), orc.pool_levels(k, B, L)
    sel = orc.select(ql, kl, B, K)
    for l in range(1, L):
        child, parent = sel[l - 1], sel[l]
        for a in range(child.shape[0]):
            row = child[a]
            assert len(row) == K and np.all(np.diff(row) > 0)
            assert set((row // B).tolist()) <= set(parent[a // B].tolist())


def test_selection_full_k_selects_everything():
    q = _rand((4096, 8), 9)
    k = _rand((4096, 8), 10)
    B, L = 16, 2
    ks = [16 * B, 16]                      # K_L = n_L, K_1 = K_2 * B
    ql, kl = orc.pool_levels(q, B, L), orc.pool_levels(k, B, L)
    sel = orc.select(ql, kl, B, ks)
    assert all(np.array_equal(r, np.arange(16)) for r in sel[1])
    assert all(np.array_equal(r, np.arange(256)) for r in sel[0])


def test_selection_cost_geometric_bound():
    """Selection work: n_L^2 + sum_{l<L} n_l K B  <=  n_L^2 + B/(B-1) * N K ([SUM] sec. 三)."""
    for n, L in [(4096, 2), (65536, 3), (262144, 3), (65536, 4)]:
        c = orc.selection_candidates(n, 16, L, 8)
        nl = n // 16 ** L
        assert c <= nl * nl + 16 / 15 * n * 8
        assert c == nl * nl + sum((n // 16 ** l) * 8 * 16 for l in range(1, L))


# ----------------------------------------------------------------------------- attention


def _sdpa(q, k, v, mask=None, scale=None):
    qt, kt, vt = (torch.as_tensor(x) for x in (q, k, v))
    m = None if mask is None else torch.as_tensor(mask)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m,
                                                            scale=scale)


def _dense_mask_formulation(qm, km, vm, sel, B, enrich, scale, top=None, weighted=True,
                            exclude=False):
    """torch float64: one query row per token against [fine tokens ; pooled keys of levels
    2..top (default L)], with an additive mask holding 0 (selected fine), l*ln B (selected
    coarse; 0 when not weighted) or -inf.  Token i's level-l ancestor is i // B^l.  Pooling is
    done with torch so autograd carries gradients through it."""
    n, d = qm.shape
    L = len(sel)
    top = L if top is None else top
    kl, vl = [km], [vm]
    for _ in range(L):
        kl.append(kl[-1].reshape(-1, B, d).mean(dim=1))
        vl.append(vl[-1].reshape(-1, B, d).mean(dim=1))
    extra_k = [kl[l] for l in range(2, top + 1)] if enrich else []
    extra_v = [vl[l] for l in range(2, top + 1)] if enrich else []
    keys = torch.cat([km] + extra_k)
    vals = torch.cat([vm] + extra_v)
    mask = np.full((n, keys.shape[0]), -np.inf)
    i = np.arange(n)
    for slot in range(sel[0].shape[1]):
        blk = sel[0][i // B, slot]
        for t in range(B):
            mask[i, blk * B + t] = 0.0
    if enrich:
        base = n
        for l in range(2, top + 1):
            finer = sel[l - 2][i // B ** (l - 1)]   # [n, K]: keys one level finer, per token
            for slot in range(sel[l - 1].shape[1]):
                j = sel[l - 1][i // B ** l, slot]
                value = np.full(n, l * math.log(B) if weighted else 0.0)
                if exclude:   # the key's token span meets a finer selected key's span
                    lo, hi = j * B ** l, (j + 1) * B ** l
                    flo, fhi = finer * B ** (l - 1), (finer + 1) * B ** (l - 1)
                    meets = ((np.maximum(lo[:, None], flo) < np.minimum(hi[:, None], fhi))
                             .any(axis=1))
                    value[meets] = -np.inf
                mask[i, base + j] = value
            base += n // B ** l
    return _sdpa(qm[None], keys[None], vals[None], mask[None], scale)[0]


def _attn_case(seed, n=1024, d=16, B=4, L=3, K=3):
    q, k, v = (_rand((n, d), seed + i) for i in range(3))
    ql, kl, vl = (orc.pool_levels(x, B, L) for x in (q, k, v))
    sel = orc.select(ql, kl, B, K)
    return q, k, v, kl, vl, sel


@pytest.mark.parametrize("n,B,L,K,enrich", [(4096, 16, 2, 3, True), (1024, 4, 3, 3, True),
                                             (1024, 4, 3, 2, False), (256, 16, 1, 3, False),
                                             (4096, 4, 4, 2, True), (4096, 64, 1, 3, False),
                                             (4096, 64, 2, 1, True)])
def test_attention_matches_dense_mask_formulation(n, B, L, K, enrich):
    q, k, v, kl, vl, sel = _attn_case(11, n=n, B=B, L=L, K=K)
    o, lse = orc.attention_forward(q, k, v, kl, vl, sel, B, enrich)
    ref = _dense_mask_formulation(torch.tensor(q), torch.tensor(k), torch.tensor(v), sel, B,
                                  enrich, 1 / math.sqrt(q.shape[1]))
    assert np.allclose(o, ref.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("B,L,levels_kept,weighted", [(4, 3, 1, True), (4, 4, 2, False),
                                                      (4, 3, 0, False), (16, 2, 1, False)])
def test_enrichment_variants_match_dense_mask_formulation(B, L, levels_kept, weighted):
    """The variants: only the finest `levels_kept` coarse levels (0 = all), and weight 1
    instead of B^l; forward against the masked formulation, backward against its autograd."""
    n = 4096 if B == 16 else 1024
    q, k, v, kl, vl, sel = _attn_case(13, n=n, d=8, B=B, L=L, K=2)
    do = _rand(q.shape, 14)
    kw = dict(enrich_levels=levels_kept, coarse_weight=weighted)
    o, _ = orc.attention_forward(q, k, v, kl, vl, sel, B, True, **kw)
    top = L if levels_kept == 0 else min(L, 1 + levels_kept)
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    ref = _dense_mask_formulation(qt, kt, vt, sel, B, True, 1 / math.sqrt(q.shape[1]), top,
                                  weighted)
    assert np.allclose(o, ref.detach().numpy(), rtol=0, atol=1e-12)
    ref.backward(torch.tensor(do))
    grads = orc.attention_backward(q, k, v, kl, vl, sel, do, B, True, **kw)
    for g, t in zip(grads, (qt, kt, vt)):
        assert np.allclose(g, t.grad.numpy(), rtol=0, atol=1e-10)
    # the default is the full enrichment with weights B^l: a variant must differ from it
    o_full, _ = orc.attention_forward(q, k, v, kl, vl, sel, B, True)
    assert not np.allclose(o, o_full, rtol=0, atol=1e-6) or (levels_kept == 0 and weighted)


@pytest.mark.parametrize("B,L,K,levels_kept", [(4, 3, 2, 0), (4, 4, 2, 0), (16, 2, 3, 0),
                                               (4, 4, 2, 2)])
def test_overlap_excluded_coarse_keys_match_dense_mask_formulation(B, L, K, levels_kept):
    """The variant that drops coarse keys whose span meets a finer selected key: forward and
    backward against the masked formulation built from token spans."""
    n = 4096 if B == 16 else 1024
    q, k, v, kl, vl, sel = _attn_case(15, n=n, d=8, B=B, L=L, K=K)
    do = _rand(q.shape, 16)
    kw = dict(enrich_levels=levels_kept, exclude_overlap=True)
    o, _ = orc.attention_forward(q, k, v, kl, vl, sel, B, True, **kw)
    top = L if levels_kept == 0 else min(L, 1 + levels_kept)
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    ref = _dense_mask_formulation(qt, kt, vt, sel, B, True, 1 / math.sqrt(q.shape[1]), top,
                                  True, exclude=True)
    assert np.allclose(o, ref.detach().numpy(), rtol=0, atol=1e-12)
    ref.backward(torch.tensor(do))
    for g, t in zip(orc.attention_backward(q, k, v, kl, vl, sel, do, B, True, **kw),
                    (qt, kt, vt)):
        assert np.allclose(g, t.grad.numpy(), rtol=0, atol=1e-10)
    # some coarse keys are dropped and some kept, so the case exercises both branches
    kept = [len(orc.key_list(p, k, v, kl, vl, sel, B, True, exclude_overlap=True)[3])
            for p in range(n // B)]
    full = [len(orc.key_list(p, k, v, kl, vl, sel, B, True)[3]) for p in range(n // B)]
    assert min(f - c for f, c in zip(full, kept)) >= 0 and sum(full) > sum(kept)
    assert any(c > K * B for c in kept)


def test_attention_full_k_no_enrich_is_dense_attention():
    """K covering every candidate and no enrichment = plain softmax attention."""
    n, d, B, L = 4096, 16, 16, 2
    q, k, v = (_rand((n, d), 20 + i) for i in range(3))
    ql, kl, vl = (orc.pool_levels(x, B, L) for x in (q, k, v))
    sel = orc.select(ql, kl, B, [16 * B, 16])
    o, _ = orc.attention_forward(q, k, v, kl, vl, sel, B, enrich=False)
    ref = _sdpa(q[None], k[None], v[None])[0].numpy()
    assert np.allclose(o, ref, rtol=0, atol=1e-12)


def test_coarse_weight_equals_duplication():
    """A coarse key with weight B^l equals B^l unweighted copies of it ([SUM] sec. 四)."""
    q, k, v, kl, vl, sel = _attn_case(30, n=1024, B=4, L=3, K=2)
    B = 4
    o, _ = orc.attention_forward(q, k, v, kl, vl, sel, B, True)
    for p in (0, 37, 255):  # level-1 blocks of 4 tokens
        kk, vv, _, ident = orc.key_list(p, k, v, kl, vl, sel, B, True)
        reps = np.array([1 if lvl == 0 else B ** lvl for lvl, _ in ident])
        kd, vd = np.repeat(kk, reps, axis=0), np.repeat(vv, reps, axis=0)
        ref = _sdpa(q[p * B:(p + 1) * B][None], kd[None], vd[None])[0].numpy()
        assert np.allclose(o[p * B:(p + 1) * B], ref, rtol=0, atol=1e-12)


def test_constant_values_and_normalisation():
    q, k, v, kl, vl, sel = _attn_case(40, n=4096, B=16, L=2, K=3)
    v = np.tile(np.linspace(-1, 1, q.shape[1]), (q.shape[0], 1))
    vl = orc.pool_levels(v, 16, 2)
    o, lse = orc.attention_forward(q, k, v, kl, vl, sel, 16, True)
    assert np.allclose(o, v, rtol=0, atol=1e-12)
    # sum_e w_e exp(s_e - lse) = 1 for every query
    scale = 1 / math.sqrt(q.shape[1])
    for p in (0, 100):
        kk, _, logw, _ = orc.key_list(p, k, v, kl, vl, sel, 16, True)
        s = scale * q[p * 16:(p + 1) * 16] @ kk.T + logw
        assert np.allclose(np.exp(s - lse[p * 16:(p + 1) * 16, None]).sum(1), 1.0, atol=1e-12)


@pytest.mark.parametrize("enrich", [False, True])
def test_attention_forward_restricted_blocks(enrich):
    """attention_forward(blocks=...) fills exactly the rows of the given query blocks, equal to
    the dense-mask formulation's rows (torch SDPA), and leaves the others NaN; all blocks give
    the unrestricted result."""
    B = 4
    q, k, v, kl, vl, sel = _attn_case(13, n=1024, d=8, B=B, L=3, K=3)
    blocks = [0, 5, 17, 255]
    o, lse = orc.attention_forward(q, k, v, kl, vl, sel, B, enrich, blocks=blocks)
    ref = _dense_mask_formulation(torch.tensor(q), torch.tensor(k), torch.tensor(v), sel, B,
                                  enrich, 1 / math.sqrt(q.shape[1])).numpy()
    rows = np.concatenate([np.arange(b * B, b * B + B) for b in blocks])
    others = np.setdiff1d(np.arange(q.shape[0]), rows)
    assert np.allclose(o[rows], ref[rows], rtol=0, atol=1e-12)
    assert np.isnan(o[others]).all() and np.isnan(lse[others]).all()
    assert np.isfinite(lse[rows]).all()
    o_all, lse_all = orc.attention_forward(q, k, v, kl, vl, sel, B, enrich,
                                           blocks=range(q.shape[0] // B))
    o_ref, lse_ref = orc.attention_forward(q, k, v, kl, vl, sel, B, enrich)
    assert np.array_equal(o_all, o_ref) and np.array_equal(lse_all, lse_ref)


def test_attention_backward_restricted_blocks():
    """attention_backward(blocks=users of some key blocks), no enrichment: the users' dq rows
    and the key blocks' dk, dv rows equal torch float64 autograd of the dense-mask
    formulation (a key block's gradient comes only from the query blocks that picked it);
    with enrichment the given blocks' dq rows still do; all blocks give the full result."""
    B = 4
    for enrich in (False, True):
        q, k, v, kl, vl, sel = _attn_case(17, n=1024, d=8, B=B, L=3, K=3)
        do = _rand(q.shape, 18)
        kb = [0, 7, 63, 255]
        users = sorted({int(a) for j in kb for a in np.nonzero((sel[0] == j).any(axis=1))[0]})
        assert 0 < len(users) < q.shape[0] // B
        gq, gk, gv = orc.attention_backward(q, k, v, kl, vl, sel, do, B, enrich, blocks=users)
        qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        _dense_mask_formulation(qt, kt, vt, sel, B, enrich,
                                1 / math.sqrt(q.shape[1])).backward(torch.tensor(do))
        qrows = np.concatenate([np.arange(b * B, b * B + B) for b in users])
        krows = np.concatenate([np.arange(j * B, j * B + B) for j in kb])
        assert np.allclose(gq[qrows], qt.grad.numpy()[qrows], rtol=0, atol=1e-10)
        if not enrich:
            assert np.allclose(gk[krows], kt.grad.numpy()[krows], rtol=0, atol=1e-10)
            assert np.allclose(gv[krows], vt.grad.numpy()[krows], rtol=0, atol=1e-10)
        full = orc.attention_backward(q, k, v, kl, vl, sel, do, B, enrich)
        every = orc.attention_backward(q, k, v, kl, vl, sel, do, B, enrich,
                                       blocks=range(q.shape[0] // B))
        for a, b in zip(full, every):
            assert np.array_equal(a, b)


# ----------------------------------------------------------------------------- backward


@pytest.mark.parametrize("n,B,L,enrich", [(1024, 4, 3, True), (4096, 16, 2, True),
                                          (1024, 4, 2, False)])
def test_backward_matches_autograd_of_dense_mask_formulation(n, B, L, enrich):
    q, k, v, kl, vl, sel = _attn_case(50, n=n, d=8, B=B, L=L, K=2)
    do = _rand(q.shape, 59)
    dq, dk, dv = orc.attention_backward(q, k, v, kl, vl, sel, do, B, enrich)
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = _dense_mask_formulation(qt, kt, vt, sel, B, enrich, 1 / math.sqrt(q.shape[1]))
    o.backward(torch.tensor(do))
    assert np.allclose(dq, qt.grad.numpy(), rtol=0, atol=1e-10)
    assert np.allclose(dk, kt.grad.numpy(), rtol=0, atol=1e-10)
    assert np.allclose(dv, vt.grad.numpy(), rtol=0, atol=1e-10)


def test_backward_block64_matches_autograd_of_dense_mask_formulation():
    """B = 64 (8x8 tiles): two levels, one coarse key per query block."""
    q, k, v, kl, vl, sel = _attn_case(52, n=4096, d=8, B=64, L=2, K=1)
    do = _rand(q.shape, 53)
    dq, dk, dv = orc.attention_backward(q, k, v, kl, vl, sel, do, 64, True)
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = _dense_mask_formulation(qt, kt, vt, sel, 64, True, 1 / math.sqrt(q.shape[1]))
    o.backward(torch.tensor(do))
    for g, t in zip((dq, dk, dv), (qt, kt, vt)):
        assert np.allclose(g, t.grad.numpy(), rtol=0, atol=1e-10)


def test_backward_finite_differences():
    """Central differences of sum(o * dO) with the selection frozen."""
    q, k, v, kl, vl, sel = _attn_case(60, n=256, d=4, B=16, L=2, K=2)
    do = _rand(q.shape, 69)
    B = 16

    def loss(q_, k_, v_):
        kl_ = orc.pool_levels(k_, B, 2)
        vl_ = orc.pool_levels(v_, B, 2)
        o, _ = orc.attention_forward(q_, k_, v_, kl_, vl_, sel, B, True)
        return float((o * do).sum())

    dq, dk, dv = orc.attention_backward(q, k, v, kl, vl, sel, do, B, True)
    rng = np.random.default_rng(61)
    h = 1e-6
    for grad, which in ((dq, 0), (dk, 1), (dv, 2)):
        for _ in range(6):
            i, c = int(rng.integers(256)), int(rng.integers(4))
            args = [q.copy(), k.copy(), v.copy()]
            args[which][i, c] += h
            up = loss(*args)
            args[which][i, c] -= 2 * h
            dn = loss(*args)
            assert abs((up - dn) / (2 * h) - grad[i, c]) < 1e-6 * max(1.0, abs(grad[i, c]))


def test_backward_invariants():
    """sum over tokens of dK is 0 and of dV is sum of dO (softmax rows sum to one, and the
    push-down of a coarse gradient spreads it over its B^l tokens with weight 1/B^l)."""
    q, k, v, kl, vl, sel = _attn_case(70, n=1024, d=8, B=4, L=3, K=3)
    do = _rand(q.shape, 79)
    dq, dk, dv = orc.attention_backward(q, k, v, kl, vl, sel, do, 4, True)
    assert np.allclose(dk.sum(0), 0.0, atol=1e-10)
    assert np.allclose(dv.sum(0), do.sum(0), atol=1e-10)


def test_backward_full_k_no_enrich_is_dense_gradient():
    n, d, B = 256, 8, 16
    q, k, v = (_rand((n, d), 80 + i) for i in range(3))
    ql, kl, vl = (orc.pool_levels(x, B, 1) for x in (q, k, v))
    sel = orc.select(ql, kl, B, [16])
    do = _rand((n, d), 89)
    dq, dk, dv = orc.attention_backward(q, k, v, kl, vl, sel, do, B, False)
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    _sdpa(qt[None], kt[None], vt[None])[0].backward(torch.tensor(do))
    for a, b in ((dq, qt), (dk, kt), (dv, vt)):
        assert np.allclose(a, b.grad.numpy(), rtol=0, atol=1e-10)


def test_dense_baseline_matches_sdpa_and_autograd():
    """The dense baseline's oracle equals torch float64 SDPA and its autograd gradients."""
    n, d = 384, 64
    q, k, v, do = (_rand((n, d), 90 + i) for i in range(4))
    o, lse = orc.dense_attention_forward(q, k, v)
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    ref = _sdpa(qt[None], kt[None], vt[None])[0]
    assert np.allclose(o, ref.detach().numpy(), rtol=0, atol=1e-12)
    s = (q @ k.T) / math.sqrt(d)
    assert np.allclose(lse, np.log(np.exp(s).sum(axis=1)), rtol=0, atol=1e-10)
    ref.backward(torch.tensor(do))
    for a, b in zip(orc.dense_attention_backward(q, k, v, do), (qt, kt, vt)):
        assert np.allclose(a, b.grad.numpy(), rtol=0, atol=1e-10)


def test_dense_baseline_is_the_full_k_sparse_case():
    """With K covering every candidate and no enrichment the sparse oracle is the dense one."""
    n, d, B = 256, 8, 16
    q, k, v, do = (_rand((n, d), 95 + i) for i in range(4))
    ql, kl, vl = (orc.pool_levels(x, B, 1) for x in (q, k, v))
    sel = orc.select(ql, kl, B, [16])
    o, lse = orc.attention_forward(q, k, v, kl, vl, sel, B, False)
    od, lsed = orc.dense_attention_forward(q, k, v)
    assert np.allclose(o, od, rtol=0, atol=1e-12) and np.allclose(lse, lsed, rtol=0, atol=1e-12)
    for a, b in zip(orc.attention_backward(q, k, v, kl, vl, sel, do, B, False),
                    orc.dense_attention_backward(q, k, v, do)):
        assert np.allclose(a, b, rtol=0, atol=1e-10)


# ----------------------------------------------------------------------------- CSC


@pytest.mark.parametrize("rows,cols,k,seed", [(256, 256, 8, 1), (4096, 4096, 8, 2),
                                              (16, 16, 8, 3), (100, 37, 5, 4)])
def test_csc_matches_scipy_transpose(rows, cols, k, seed):
    rng = np.random.default_rng(seed)
    sel = np.sort(np.stack([rng.choice(cols, k, replace=False) for _ in range(rows)]), axis=1)
    off, r = orc.csr_to_csc(sel, cols)
    csr = scipy.sparse.csr_matrix((np.ones(rows * k), sel.reshape(-1),
                                   np.arange(0, rows * k + 1, k)), shape=(rows, cols))
    csc = csr.tocsc()
    csc.sort_indices()
    assert np.array_equal(off, csc.indptr)
    assert np.array_equal(r, csc.indices)
    assert off[0] == 0 and off[-1] == rows * k and np.all(np.diff(off) >= 0)


def test_csc_of_selection_is_inverse():
    q, k, v, kl, vl, sel = _attn_case(90, n=1024, B=4, L=3, K=4)
    for lvl in sel:
        off, rows = orc.csr_to_csc(lvl, lvl.shape[0])
        pairs = {(int(rows[e]), c) for c in range(lvl.shape[0]) for e in range(off[c], off[c + 1])}
        assert pairs == {(a, int(c)) for a in range(lvl.shape[0]) for c in lvl[a]}


# ----------------------------------------------------------------------------- whole path


def test_full_path_raster_roundtrip_dense_case():
    """Whole raster-order path with full K and no enrichment equals dense attention on the
    raster tokens (the reorder is invisible in the result)."""
    b, hh, H, W, d = 1, 2, 16, 16, 8
    q, k, v = (_rand((b, hh, H * W, d), 100 + i) for i in range(3))
    res = orc.llsa_forward(q, k, v, H, W, 16, 1, [16], enrich=False)
    ref = _sdpa(q, k, v).numpy()
    assert np.allclose(res["o"], ref, rtol=0, atol=1e-12)
    do = _rand(q.shape, 109)
    dq, dk, dv = orc.llsa_backward(q, k, v, do, H, W, 16, 1, res["sel"], enrich=False)
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    _sdpa(qt, kt, vt).backward(torch.tensor(do))
    for a, t in ((dq, qt), (dk, kt), (dv, vt)):
        assert np.allclose(a, t.grad.numpy(), rtol=0, atol=1e-10)
