"""GPU parity of every hot-path step against the CPU oracle, through the C ABI.

Inputs come from the seeded generator (smooth 2D fields + noise for Q/K, N(0,1) for V/dO);
shapes follow the workloads: 64x64 fp32 (L=2), 128x128 (L=2), 256x256 (L=3), 512x512 (L=3),
plus small and ragged cases.  Full-size configurations compare whole heads chosen by index
(heads are independent), the rest compare every output.
"""
import numpy as np
import pytest
import torch

from hierarchical_top_sparse_amd import _abi, gen, ops
from oracle import llsa_oracle as orc
from tests.parity_util import (assert_close, check_selection, gpu_sel_lists,
                                lse_tolerance, to64)

pytestmark = pytest.mark.gpu

DEV = "cuda"
RASTER, MORTON = _abi.LLSA_LAYOUT_RASTER, _abi.LLSA_LAYOUT_MORTON


def _inputs(batch, heads, height, width, dtype, seed, grad=False):
    x = gen.make_inputs(batch, heads, height, width, 64, dtype, seed, with_grad=grad)
    return {k: v.to(DEV) for k, v in x.items()}, {k: to64(v) for k, v in x.items()}


def _problem(x, height, width, levels, topk=8, enrich=True, layout=RASTER):
    return ops.make_problem(x, height, width, levels, topk, enrich, 0.0, layout)


def _bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32).cpu()


# ----------------------------------------------------------------------------- reorder


@pytest.mark.parametrize("h,w,dtype", [(64, 64, torch.float32), (128, 128, torch.bfloat16),
                                       (64, 256, torch.bfloat16), (256, 64, torch.float32),
                                       (512, 512, torch.bfloat16)])
def test_reorder_bit_exact(h, w, dtype):
    x = torch.randn(1, 3, h * w, 64, dtype=torch.float32).to(dtype).to(DEV)
    p = _problem(x, h, w, 1, topk=1)
    y = ops.reorder(p, x)
    perm = torch.from_numpy(orc.morton_perm(h, w))
    assert torch.equal(_bits(y), _bits(x.cpu()[:, :, perm, :]))
    back = ops.reorder(p, y, inverse=True)
    assert torch.equal(_bits(back), _bits(x))


# ----------------------------------------------------------------------------- pooling


@pytest.mark.parametrize("h,w,levels,dtype,layout", [
    (64, 64, 2, torch.float32, RASTER), (128, 128, 2, torch.bfloat16, MORTON),
    (256, 256, 3, torch.bfloat16, RASTER), (128, 256, 3, torch.bfloat16, RASTER)])
def test_pool_matches_oracle(h, w, levels, dtype, layout):
    d, ref = _inputs(1, 2, h, w, dtype, 11)
    q, k, v = d["q"], d["k"], d["v"]
    p = _problem(q, h, w, levels, layout=layout)
    if layout == MORTON:
        q, k, v = (ops.reorder(p, t) for t in (q, k, v))
    lv = {t: [torch.empty((1, 2, p.n_level(l), 64), device=DEV) for l in range(1, levels + 1)]
          for t in "qkv"}
    _abi.llsa_pool(p, q, k, v, lv["q"], lv["k"], lv["v"])
    for t in "qkv":
        want = orc.pool_levels(orc.reorder(ref[t], h, w), 16, levels)
        for l in range(levels):
            got = to64(lv[t][l])
            assert np.abs(got - want[l]).max() <= 1e-5 * max(1.0, np.abs(want[l]).max()), (t, l)


# ----------------------------------------------------------------------------- selection


@pytest.mark.parametrize("h,w,levels,topk", [(64, 64, 2, 8), (128, 128, 2, 8), (256, 256, 3, 8),
                                             (128, 256, 3, 5), (64, 64, 1, 16), (64, 64, 2, 3),
                                             (128, 128, 1, 32), (128, 128, 2, 32),
                                             (256, 256, 1, 32), (64, 128, 1, 20)])
def test_select_matches_oracle_within_tie_window(h, w, levels, topk):
    d, ref = _inputs(1, 3, h, w, torch.bfloat16, 21)
    p = _problem(d["q"], h, w, levels, topk)
    fwd = ops.llsa_forward(p, d["q"], d["k"], d["v"])
    q_lv = orc.pool_levels(orc.reorder(ref["q"], h, w), 16, levels)
    k_lv = orc.pool_levels(orc.reorder(ref["k"], h, w), 16, levels)
    sel = [s.cpu().numpy().astype(np.int64) for s in fwd["sel"]]
    flips = check_selection(sel, q_lv, k_lv, topk, f"{h}x{w} L{levels}")
    total = sum(s.shape[0] * s.shape[1] * s.shape[2] for s in sel)
    assert flips <= max(2, total // 1000), f"{flips} near-tie flips out of {total} rows"


def test_select_single_level_from_given_parent():
    """llsa_select on one level with an oracle-supplied parent selection."""
    h = w = 128
    d, ref = _inputs(1, 2, h, w, torch.bfloat16, 23)
    p = _problem(d["q"], h, w, 2)
    fwd = ops.llsa_forward(p, d["q"], d["k"], d["v"])
    q_lv = orc.pool_levels(orc.reorder(ref["q"], h, w), 16, 2)
    k_lv = orc.pool_levels(orc.reorder(ref["k"], h, w), 16, 2)
    parent = np.stack([orc.select_coarsest(q_lv[1][0, i], k_lv[1][0, i], 8) for i in range(2)])
    sel = [torch.empty_like(fwd["sel"][0]),
           torch.from_numpy(parent[None].astype(np.int32)).to(DEV)]
    _abi.llsa_select(p, fwd["q_lv"], fwd["k_lv"], sel, level_hi=1, level_lo=1)
    got = sel[0].cpu().numpy().astype(np.int64)
    for i in range(2):
        from tests.parity_util import check_level
        check_level(got[0, i], q_lv[0][0, i], k_lv[0][0, i], parent[i], 8, f"head {i}")


@pytest.mark.parametrize("h,w,L,K,level_hi,level_lo", [
    (256, 256, 3, 6, 2, 1), (256, 256, 3, 6, 3, 2), (256, 256, 3, 6, 2, 2),
    (256, 256, 3, 6, 3, 3), (512, 512, 4, 4, 3, 1), (512, 512, 4, 4, 4, 1)])
def test_select_level_range_from_given_parent(h, w, L, K, level_hi, level_lo):
    """llsa_select over a sub-range of levels: levels above level_hi come from the oracle;
    every computed level is checked teacher-forced on the GPU's parents (a chain of several
    single-query ancestors when level_hi - level_lo >= 2)."""
    from tests.parity_util import check_level
    d, ref = _inputs(1, 2, h, w, torch.bfloat16, 29)
    p = _problem(d["q"], h, w, L, K)
    fwd = ops.llsa_forward(p, d["q"], d["k"], d["v"])
    q_lv = orc.pool_levels(orc.reorder(ref["q"], h, w), 16, L)
    k_lv = orc.pool_levels(orc.reorder(ref["k"], h, w), 16, L)
    want = [orc.select(q_lv_h, k_lv_h, 16, K) for q_lv_h, k_lv_h in
            zip(zip(*[x[0] for x in q_lv]), zip(*[x[0] for x in k_lv]))]
    sel = [torch.full_like(s, -7) for s in fwd["sel"]]
    for l in range(level_hi + 1, L + 1):
        sel[l - 1] = torch.from_numpy(np.stack([want[i][l - 1] for i in range(2)])[None]
                                      .astype(np.int32)).to(DEV)
    _abi.llsa_select(p, fwd["q_lv"], fwd["k_lv"], sel, level_hi=level_hi, level_lo=level_lo)
    got = [s.cpu().numpy().astype(np.int64) for s in sel]
    for l in range(L, 0, -1):
        for i in range(2):
            if l > level_hi:
                continue
            if l < level_lo:   # untouched
                assert (got[l - 1][0, i] == -7).all()
                continue
            parent = None if l == L else got[l][0, i]
            check_level(got[l - 1][0, i], q_lv[l - 1][0, i], k_lv[l - 1][0, i], parent, K,
                        f"levels {level_hi}..{level_lo} head {i} level {l}")


# ----------------------------------------------------------------------------- transpose


@pytest.mark.parametrize("nmat,rows,cols,k,seed", [(1, 16, 16, 8, 0), (3, 256, 256, 8, 1),
                                                   (2, 4096, 4096, 8, 2), (1, 16384, 16384, 8, 3),
                                                   (2, 1000, 333, 5, 4), (1, 300, 7, 3, 5),
                                                   (1, 32768, 32768, 8, 6),
                                                   (1, 40000, 500, 7, 7)])
def test_index_transpose_bit_exact(nmat, rows, cols, k, seed):
    rng = np.random.default_rng(seed)
    csr = np.stack([np.sort(np.stack([rng.choice(cols, k, replace=False) for _ in range(rows)]),
                            axis=1) for _ in range(nmat)]).astype(np.int32)
    if seed == 4:   # unsorted rows and a few out-of-range ids (dropped)
        csr = csr[:, :, ::-1].copy()
        csr[0, 3, 1] = cols + 5
        csr[1, 7, 0] = -2
    t = torch.from_numpy(csr).to(DEV)
    off = torch.empty((nmat, cols + 1), dtype=torch.int32, device=DEV)
    rws = torch.empty((nmat, rows * k), dtype=torch.int32, device=DEV)
    ws = torch.empty(_abi.llsa_index_transpose_workspace(nmat, rows, cols, k), dtype=torch.uint8,
                     device=DEV)
    _abi.llsa_index_transpose(nmat, rows, cols, k, t, off, rws, ws)
    off, rws = off.cpu().numpy(), rws.cpu().numpy()
    for m in range(nmat):
        keep = (csr[m] >= 0) & (csr[m] < cols)
        want_off, want_rows = orc.csr_to_csc(np.where(keep, csr[m], 0), cols)
        if not keep.all():   # oracle on the kept entries only
            flat_rows = np.repeat(np.arange(rows), k)[keep.reshape(-1)]
            flat_keys = csr[m].reshape(-1)[keep.reshape(-1)]
            order = np.argsort(flat_keys, kind="stable")
            want_rows = flat_rows[order]
            want_off = np.concatenate([[0], np.cumsum(np.bincount(flat_keys, minlength=cols))])
        assert np.array_equal(off[m], want_off)
        assert np.array_equal(rws[m][:want_off[-1]], want_rows)


def _random_transpose_cases(n_cases=10, seed=2024):
    """Seeded shapes: rows up to 50,000 (beyond 32 sort tiles: the merge path), columns from
    1, k up to 32; uniform or skewed (a few popular columns take most entries) column draws."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n_cases):
        cases.append((int(rng.integers(1, 4)), int(rng.integers(1, 50001)),
                      int(rng.integers(1, 20001)), int(rng.integers(1, 33)), bool(i % 2), i))
    return cases


@pytest.mark.parametrize("nmat,rows,cols,k,skewed,seed", _random_transpose_cases())
def test_index_transpose_random_shapes(nmat, rows, cols, k, skewed, seed):
    """Bit-exact against a stable sort by column, rows ascending within a column, on seeded
    random shapes (duplicate ids within a row allowed: each entry is kept)."""
    rng = np.random.default_rng(100 + seed)
    if skewed:   # Zipf-like column popularity
        w = 1.0 / np.arange(1, cols + 1) ** 1.2
        csr = rng.choice(cols, size=(nmat, rows, k), p=w / w.sum())
    else:
        csr = rng.integers(0, cols, size=(nmat, rows, k))
    csr = csr.astype(np.int32)
    t = torch.from_numpy(csr).to(DEV)
    off = torch.empty((nmat, cols + 1), dtype=torch.int32, device=DEV)
    rws = torch.empty((nmat, rows * k), dtype=torch.int32, device=DEV)
    ws = torch.empty(_abi.llsa_index_transpose_workspace(nmat, rows, cols, k), dtype=torch.uint8,
                     device=DEV)
    _abi.llsa_index_transpose(nmat, rows, cols, k, t, off, rws, ws)
    off, rws = off.cpu().numpy(), rws.cpu().numpy()
    for m in range(nmat):
        flat_keys = csr[m].reshape(-1)
        flat_rows = np.repeat(np.arange(rows), k)
        order = np.argsort(flat_keys, kind="stable")
        want_off = np.concatenate([[0], np.cumsum(np.bincount(flat_keys, minlength=cols))])
        assert np.array_equal(off[m], want_off), (m, rows, cols, k)
        assert np.array_equal(rws[m], flat_rows[order]), (m, rows, cols, k)


# ----------------------------------------------------------------------------- attention


def _oracle_sel(ref, h, w, levels, topk, b=0, hh=0):
    q_lv = orc.pool_levels(orc.reorder(ref["q"][b, hh], h, w), 16, levels)
    k_lv = orc.pool_levels(orc.reorder(ref["k"][b, hh], h, w), 16, levels)
    return orc.select(q_lv, k_lv, 16, topk)


@pytest.mark.parametrize("h,w,levels,topk,enrich,dtype,layout", [
    (64, 64, 2, 8, True, torch.float32, RASTER),
    (64, 64, 2, 8, True, torch.bfloat16, RASTER),
    (64, 64, 2, 5, True, torch.bfloat16, MORTON),
    (128, 256, 3, 8, True, torch.bfloat16, RASTER),
    (128, 128, 2, 7, False, torch.bfloat16, RASTER),
    (64, 64, 1, 16, False, torch.float32, MORTON),
    (128, 128, 1, 32, False, torch.bfloat16, RASTER),
    (128, 128, 2, 32, True, torch.bfloat16, MORTON),
    (64, 128, 1, 24, False, torch.float32, RASTER),
    (128, 128, 2, 17, True, torch.float32, RASTER),
])
def test_attn_fwd_on_oracle_indices(h, w, levels, topk, enrich, dtype, layout):
    """Forward attention in isolation: GPU attention on the oracle's own selection."""
    d, ref = _inputs(1, 2, h, w, dtype, 31)
    p = _problem(d["q"], h, w, levels, topk, enrich, layout)
    sels = [_oracle_sel(ref, h, w, levels, topk, 0, i) for i in range(2)]
    sel_t = [torch.from_numpy(np.stack([sels[i][l] for i in range(2)])[None].astype(np.int32))
             .to(DEV) for l in range(levels)]
    q, k, v = d["q"], d["k"], d["v"]
    if layout == MORTON:
        q, k, v = (ops.reorder(p, t) for t in (q, k, v))
    kl = [torch.empty((1, 2, p.n_level(l), 64), device=DEV) for l in range(1, levels + 1)]
    vl = [torch.empty((1, 2, p.n_level(l), 64), device=DEV) for l in range(1, levels + 1)]
    _abi.llsa_pool(p, None, k, v, None, kl, vl)
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, p.n), device=DEV)
    _abi.llsa_attn_fwd(p, q, k, v, kl, vl, sel_t, o, lse)
    if layout == MORTON:
        o = ops.reorder(p, o, inverse=True)
    res = orc.llsa_forward(ref["q"], ref["k"], ref["v"], h, w, 16, levels, topk, enrich,
                           sel_override=[sels])
    assert_close(to64(o), res["o"], dtype, "o")
    assert_close(lse, res["lse"], dtype, "lse",
                 tol_abs=lse_tolerance(ref["q"], ref["k"], dtype, levels if enrich else 0))


@pytest.mark.parametrize("h,w,levels,topk,enrich,layout", [
    (64, 64, 2, 8, True, RASTER),
    (64, 64, 2, 5, True, MORTON),
    (128, 256, 3, 8, True, RASTER),
    (128, 128, 2, 8, False, RASTER),
    (64, 64, 1, 16, False, RASTER),
    (128, 128, 1, 32, False, RASTER),
    (128, 128, 2, 32, True, MORTON),
    (64, 128, 1, 21, False, RASTER),
])
def test_attn_bwd_on_oracle_indices(h, w, levels, topk, enrich, layout):
    """Backward in isolation: GPU gradients on the oracle's selection (and GPU forward)."""
    d, ref = _inputs(1, 2, h, w, torch.bfloat16, 41, grad=True)
    p = _problem(d["q"], h, w, levels, topk, enrich, layout)
    sels = [_oracle_sel(ref, h, w, levels, topk, 0, i) for i in range(2)]
    sel_t = [torch.from_numpy(np.stack([sels[i][l] for i in range(2)])[None].astype(np.int32))
             .to(DEV) for l in range(levels)]
    q, k, v, do = d["q"], d["k"], d["v"], d["do"]
    if layout == MORTON:
        q, k, v, do = (ops.reorder(p, t) for t in (q, k, v, do))
    kl = [torch.empty((1, 2, p.n_level(l), 64), device=DEV) for l in range(1, levels + 1)]
    vl = [torch.empty((1, 2, p.n_level(l), 64), device=DEV) for l in range(1, levels + 1)]
    _abi.llsa_pool(p, None, k, v, None, kl, vl)
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, p.n), device=DEV)
    _abi.llsa_attn_fwd(p, q, k, v, kl, vl, sel_t, o, lse)
    fwd = dict(o=o, lse=lse, k_lv=kl, v_lv=vl, sel=sel_t)
    dq, dk, dv = ops.llsa_backward(p, q, k, v, fwd, do)
    if layout == MORTON:
        dq, dk, dv = (ops.reorder(p, t, inverse=True) for t in (dq, dk, dv))
    want = orc.llsa_backward(ref["q"], ref["k"], ref["v"], ref["do"], h, w, 16, levels, [sels],
                             enrich)
    for name, got, ref_g in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        assert_close(to64(got), ref_g, torch.bfloat16, name)



@pytest.mark.parametrize("h,w,levels,topk,enrich,popular", [
    (128, 128, 1, 8, False, 1.0),    # every query block picks blocks 0..7: 1024 picks each
    (128, 128, 2, 8, True, 0.5),     # half the query blocks do, the rest pick their own
    (64, 128, 1, 16, False, 0.9),
    (256, 256, 3, 8, True, 1.0),     # full size: 8 blocks of 4096 picks, 248 overflow chunks
    (256, 256, 3, 8, True, 0.3),     # (the most a head's chunk slots can hold is 256)
    (256, 256, 2, 16, True, 0.7),    # 16 picks: 16 blocks of ~2900 picks
])
def test_attn_bwd_popular_key_blocks(h, w, levels, topk, enrich, popular):
    """Backward on selections where a few key blocks are picked by (nearly) every query block,
    the skew of attention to a few large-norm keys: the key-major pass cuts those blocks into
    chunks of 128 picks run by separate waves and adds their partial sums in chunk order."""
    d, ref = _inputs(1, 2, h, w, torch.bfloat16, 47, grad=True)
    p = _problem(d["q"], h, w, levels, topk, enrich)
    sels = [_oracle_sel(ref, h, w, levels, topk, 0, i) for i in range(2)]
    rng = np.random.default_rng(3)
    for i in range(2):
        s1 = sels[i][0].copy()
        hot = rng.random(s1.shape[0]) < popular
        s1[hot] = np.arange(topk)          # the same key blocks for the popular rows
        sels[i][0] = s1
    sel_t = [torch.from_numpy(np.stack([sels[i][l] for i in range(2)])[None].astype(np.int32))
             .to(DEV) for l in range(levels)]
    q, k, v, do = d["q"], d["k"], d["v"], d["do"]
    kl = [torch.empty((1, 2, p.n_level(l), 64), device=DEV) for l in range(1, levels + 1)]
    vl = [torch.empty((1, 2, p.n_level(l), 64), device=DEV) for l in range(1, levels + 1)]
    _abi.llsa_pool(p, None, k, v, None, kl, vl)
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, p.n), device=DEV)
    _abi.llsa_attn_fwd(p, q, k, v, kl, vl, sel_t, o, lse)
    dq, dk, dv = ops.llsa_backward(p, q, k, v, dict(o=o, lse=lse, k_lv=kl, v_lv=vl, sel=sel_t),
                                   do)
    want = orc.llsa_backward(ref["q"], ref["k"], ref["v"], ref["do"], h, w, 16, levels, [sels],
                             enrich)
    for name, got, ref_g in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        assert_close(to64(got), ref_g, torch.bfloat16, name)


@pytest.mark.parametrize("h,w,levels,topk,enrich_levels,unit_weight,exclude", [
    (128, 256, 3, 8, 1, False, False),    # only level 2's coarse keys
    (128, 256, 3, 8, 0, True, False),     # all coarse levels, weight 1
    (512, 512, 4, 4, 2, True, False),     # levels 2..3 of 4, weight 1
    (128, 128, 2, 8, 3, False, False),    # enrich_levels beyond L - 1 is clamped
    (128, 256, 3, 8, 0, False, True),     # overlap-excluded coarse keys
    (256, 256, 3, 8, 0, False, True),
    (128, 128, 2, 16, 0, True, True),     # exclusion with 16 picks and unit weights
    (512, 512, 4, 4, 2, False, True),     # exclusion with levels 2..3 of 4
])
def test_enrichment_variants_on_oracle_indices(h, w, levels, topk, enrich_levels, unit_weight,
                                               exclude):
    """Forward and backward of the enrichment variants against the oracle's variants, on the
    oracle's selection."""
    d, ref = _inputs(1, 2, h, w, torch.bfloat16, 43, grad=True)
    p = ops.make_problem(d["q"], h, w, levels, topk, True, 0.0, RASTER, enrich_levels,
                         unit_weight, coarse_exclude_overlap=exclude)
    sels = [_oracle_sel(ref, h, w, levels, topk, 0, i) for i in range(2)]
    sel_t = [torch.from_numpy(np.stack([sels[i][l] for i in range(2)])[None].astype(np.int32))
             .to(DEV) for l in range(levels)]
    q, k, v, do = d["q"], d["k"], d["v"], d["do"]
    kl = [torch.empty((1, 2, p.n_level(l), 64), device=DEV) for l in range(1, levels + 1)]
    vl = [torch.empty((1, 2, p.n_level(l), 64), device=DEV) for l in range(1, levels + 1)]
    _abi.llsa_pool(p, None, k, v, None, kl, vl)
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, p.n), device=DEV)
    _abi.llsa_attn_fwd(p, q, k, v, kl, vl, sel_t, o, lse)
    dq, dk, dv = ops.llsa_backward(p, q, k, v, dict(o=o, lse=lse, k_lv=kl, v_lv=vl, sel=sel_t),
                                   do)
    kw = dict(enrich_levels=enrich_levels, coarse_weight=not unit_weight,
              exclude_overlap=exclude)
    res = orc.llsa_forward(ref["q"], ref["k"], ref["v"], h, w, 16, levels, topk, True,
                           sel_override=[sels], **kw)
    assert_close(to64(o), res["o"], torch.bfloat16, "o")
    assert_close(lse, res["lse"], torch.bfloat16, "lse",
                 tol_abs=lse_tolerance(ref["q"], ref["k"], torch.bfloat16, levels))
    want = orc.llsa_backward(ref["q"], ref["k"], ref["v"], ref["do"], h, w, 16, levels, [sels],
                             True, **kw)
    for name, got, ref_g in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        assert_close(to64(got), ref_g, torch.bfloat16, name)

# ----------------------------------------------------------------------------- whole path


def _end_to_end(cfg_name, heads_checked, backward, levels=None, topk=8):
    """The whole path on a workload's full shape; levels/topk override the workload's (the
    single-level comparator: levels 1, topk 32)."""
    cfg = gen.CONFIGS[cfg_name]
    h, w = cfg["height"], cfg["width"]
    L = levels or cfg["levels"]
    d, ref = _inputs(cfg["batch"], cfg["heads"], h, w, cfg["dtype"], cfg["seed_base"],
                     grad=backward)
    p = _problem(d["q"], h, w, L, topk)
    fwd = ops.llsa_forward(p, d["q"], d["k"], d["v"])
    grads = ops.llsa_backward(p, d["q"], d["k"], d["v"], fwd, d["do"]) if backward else None
    torch.cuda.synchronize()
    sel_np = [s.cpu().numpy().astype(np.int64) for s in fwd["sel"]]
    for (bi, hi) in heads_checked:
        sl = (slice(bi, bi + 1), slice(hi, hi + 1))
        q64, k64, v64 = (ref[t][sl] for t in "qkv")
        q_lv = orc.pool_levels(orc.reorder(q64, h, w), 16, L)
        k_lv = orc.pool_levels(orc.reorder(k64, h, w), 16, L)
        check_selection([s[sl] for s in sel_np], q_lv, k_lv, topk, f"{cfg_name} b{bi} h{hi}")
        sels = [[[s[bi, hi] for s in sel_np]]]
        res = orc.llsa_forward(q64, k64, v64, h, w, 16, L, topk, True, sel_override=sels)
        assert_close(to64(fwd["o"][sl]), res["o"], cfg["dtype"], f"{cfg_name} o b{bi} h{hi}")
        assert_close(fwd["lse"][sl], res["lse"], cfg["dtype"], f"{cfg_name} lse",
                     tol_abs=lse_tolerance(q64, k64, cfg["dtype"], L))
        if backward:
            want = orc.llsa_backward(q64, k64, v64, ref["do"][sl], h, w, 16, L, sels, True)
            for name, got, ref_g in zip(("dq", "dk", "dv"), grads, want):
                assert_close(to64(got[sl]), ref_g, cfg["dtype"], f"{cfg_name} {name} b{bi} h{hi}")


def test_e2e_tiny64_fp32():
    _end_to_end("tiny64", [(0, 0), (0, 1)], backward=False)


def test_e2e_ffhq128():
    _end_to_end("ffhq128", [(0, 0), (3, 5), (1, 2)], backward=False)


def test_e2e_px256():
    _end_to_end("px256", [(0, 0), (0, 5)], backward=False)


def test_e2e_px256_train():
    _end_to_end("px256_train", [(0, 0), (1, 4)], backward=True)


def test_e2e_px512_train():
    _end_to_end("px512_train", [(0, 3)], backward=True)


def test_e2e_px256_train_single_level_top32():
    """The single-level comparator (one level, K = 32 blocks per query, selection over all
    4096 blocks) on the 256x256 training shape."""
    _end_to_end("px256_train", [(0, 2), (1, 5)], backward=True, levels=1, topk=32)


@pytest.mark.parametrize("h,w,levels,topk", [
    (16, 16, 1, 1),     # the smallest problem: 256 tokens, one pick
    (16, 16, 2, 1),     # a coarsest level of a single key
    (4, 64, 2, 1),      # a side of one 4x4 tile
    (64, 4, 1, 8),
    (32, 32, 2, 4),     # K = n_L: every coarsest key is picked
    (16, 16, 1, 16),    # K = n_1: every block is picked (dense attention, checked below)
])
def test_whole_path_small_and_degenerate(h, w, levels, topk):
    """The whole path (selection, forward, transposes, backward) on the smallest and most
    degenerate problems the contract allows, against the oracle on the GPU's selection."""
    d, ref = _inputs(1, 2, h, w, torch.bfloat16, 61, grad=True)
    p = _problem(d["q"], h, w, levels, topk)
    fwd = ops.llsa_forward(p, d["q"], d["k"], d["v"])
    grads = ops.llsa_backward(p, d["q"], d["k"], d["v"], fwd, d["do"])
    torch.cuda.synchronize()
    sel_np = [s.cpu().numpy().astype(np.int64) for s in fwd["sel"]]
    q_lv = orc.pool_levels(orc.reorder(ref["q"], h, w), 16, levels)
    k_lv = orc.pool_levels(orc.reorder(ref["k"], h, w), 16, levels)
    check_selection(sel_np, q_lv, k_lv, topk, f"{h}x{w} L{levels} K{topk}")
    sels = [[[s[0, i] for s in sel_np] for i in range(2)]]
    res = orc.llsa_forward(ref["q"], ref["k"], ref["v"], h, w, 16, levels, topk, True,
                           sel_override=sels)
    assert_close(to64(fwd["o"]), res["o"], torch.bfloat16, "o")
    assert_close(fwd["lse"], res["lse"], torch.bfloat16, "lse",
                 tol_abs=lse_tolerance(ref["q"], ref["k"], torch.bfloat16, levels))
    want = orc.llsa_backward(ref["q"], ref["k"], ref["v"], ref["do"], h, w, 16, levels, sels,
                             True)
    for name, got, ref_g in zip(("dq", "dk", "dv"), grads, want):
        assert_close(to64(got), ref_g, torch.bfloat16, name)
    if levels == 1 and topk * 16 == h * w:
        for i in range(2):   # every key of the head attended: plain softmax attention
            qm, km, vm, dom = (orc.reorder(ref[t], h, w)[0, i] for t in ("q", "k", "v", "do"))
            o_d, _ = orc.dense_attention_forward(qm, km, vm)
            got = orc.reorder(to64(fwd["o"]), h, w)[0, i]
            assert_close(got, o_d, torch.bfloat16, f"dense-equivalent o head {i}")
            for name, g, want_d in zip(("dq", "dk", "dv"), grads,
                                       orc.dense_attention_backward(qm, km, vm, dom)):
                assert_close(orc.reorder(to64(g), h, w)[0, i], want_d, torch.bfloat16,
                             f"dense-equivalent {name} head {i}")


def test_deterministic_and_autograd():
    h = w = 128
    d, _ = _inputs(1, 2, h, w, torch.bfloat16, 51, grad=True)
    outs = []
    for _ in range(2):
        q, k, v = (d[t].clone().requires_grad_(True) for t in "qkv")
        o = ops.llsa_attention(q, k, v, h, w, levels=2)
        o.backward(d["do"])
        outs.append([o.detach(), q.grad, k.grad, v.grad])
    for a, b in zip(*outs):
        assert torch.equal(_bits(a), _bits(b))
    p = _problem(d["q"], h, w, 2)
    fwd = ops.llsa_forward(p, d["q"], d["k"], d["v"])
    grads = ops.llsa_backward(p, d["q"], d["k"], d["v"], fwd, d["do"])
    assert torch.equal(_bits(fwd["o"]), _bits(outs[0][0]))
    for g, g2 in zip(grads, outs[0][1:]):
        assert torch.equal(_bits(g), _bits(g2))


def _max_inputs(n, seed):
    return {t: gen.to_dtype(gen.gaussian(seed + i, 1, 1, n, 64), torch.bfloat16)
            for i, t in enumerate(("q", "k", "v", "do"))}


def test_maximum_size_forward_sampled():
    """The largest problem the contract allows per head: N = 2^23 tokens (2048 x 4096 pixels,
    Morton layout, L = 4, K = 8, no enrichment).  Checked where the oracle can be computed
    piecewise: the selection of sampled sibling groups at every level (teacher-forced, tie
    window) and O and LSE of sampled query blocks, first and last included."""
    h, w, L, K = 2048, 4096, 4, 8
    n = h * w
    x = _max_inputs(n, 9100)
    d = {t: v.to(DEV) for t, v in x.items() if t != "do"}
    p = _problem(d["q"], h, w, L, K, enrich=False, layout=MORTON)
    fwd = ops.llsa_forward(p, d["q"], d["k"], d["v"])
    torch.cuda.synchronize()
    print("maximum size forward: GPU done", flush=True)
    sel = [s[0, 0].cpu().numpy().astype(np.int64) for s in fwd["sel"]]
    q, k, v = (x[t][0, 0].double().numpy() for t in ("q", "k", "v"))
    q_lv, k_lv = orc.pool_levels(q, 16, L), orc.pool_levels(k, 16, L)
    from tests.parity_util import check_level
    rng = np.random.default_rng(5)
    check_level(sel[L - 1], q_lv[L - 1], k_lv[L - 1], None, K, "level 4")
    for l in range(L - 1, 0, -1):   # a few whole sibling groups per level
        n_par = q_lv[l].shape[0]
        for par in sorted({0, n_par - 1, *rng.integers(0, n_par, 3).tolist()}):
            rows = slice(par * 16, par * 16 + 16)
            check_level(sel[l - 1][rows], q_lv[l - 1][rows], k_lv[l - 1], sel[l][par:par + 1],
                        K, f"level {l} parent {par}")
    n1 = n // 16
    qb = sorted({0, n1 - 1, *rng.integers(0, n1, 30).tolist()})
    o_want, lse_want = orc.attention_forward(q, k, v, [], [], sel, 16, False, blocks=qb)
    rows = np.concatenate([np.arange(b * 16, b * 16 + 16) for b in qb])
    assert_close(fwd["o"][0, 0].double().cpu().numpy()[rows], o_want[rows], torch.bfloat16,
                 "o (sampled blocks)")
    assert_close(fwd["lse"][0, 0].double().cpu().numpy()[rows], lse_want[rows],
                 torch.bfloat16, "lse (sampled blocks)", stored_bf16=False,
                 tol_abs=lse_tolerance(q, k, torch.bfloat16, 0))


def test_maximum_size_backward_sampled():
    """The largest backward: N = 2^19 tokens (512 x 1024 pixels; the level-1 transpose packs
    (key block, query block) codes in 32 bits), L = 3, K = 8, no enrichment, Morton layout:
    dQ of every query block that picked a sampled key block, and dK, dV of those key blocks
    (exact: without enrichment a key block's gradient comes only from the query blocks that
    picked it)."""
    h, w, L, K = 512, 1024, 3, 8
    n = h * w
    x = _max_inputs(n, 9200)
    d = {t: v.to(DEV) for t, v in x.items()}
    p = _problem(d["q"], h, w, L, K, enrich=False, layout=MORTON)
    fwd = ops.llsa_forward(p, d["q"], d["k"], d["v"])
    dq, dk, dv = ops.llsa_backward(p, d["q"], d["k"], d["v"], fwd, d["do"])
    torch.cuda.synchronize()
    print("maximum size backward: GPU done", flush=True)
    sel = [s[0, 0].cpu().numpy().astype(np.int64) for s in fwd["sel"]]
    q, k, v, do = (x[t][0, 0].double().numpy() for t in ("q", "k", "v", "do"))
    rng = np.random.default_rng(6)
    n1 = n // 16
    kb = sorted({0, n1 - 1, *rng.integers(0, n1, 14).tolist()})
    users = sorted({int(a) for j in kb for a in np.nonzero((sel[0] == j).any(axis=1))[0]})
    gq, gk, gv = orc.attention_backward(q, k, v, [], [], sel, do, 16, False, blocks=users)
    qrows = np.concatenate([np.arange(b * 16, b * 16 + 16) for b in users])
    krows = np.concatenate([np.arange(j * 16, j * 16 + 16) for j in kb])
    for name, got, want, r in (("dq", dq, gq, qrows), ("dk", dk, gk, krows),
                               ("dv", dv, gv, krows)):
        assert_close(got[0, 0].double().cpu().numpy()[r], want[r], torch.bfloat16,
                     f"{name} (sampled)")


@pytest.mark.parametrize("h,w,levels,topk,block,enrich", [
    (256, 256, 3, 8, 16, True),     # level 1: 8 tiles per head; levels 2, 3: one tile each
    (512, 512, 3, 8, 16, True),     # level 1: 32 tiles per head; level 2: 2 tiles
    (256, 256, 2, 8, 64, True),     # 16-token blocks from 64-token picks (32 picks per row)
    (128, 128, 1, 32, 16, False),   # the single-level comparator's index
    (1024, 512, 3, 8, 16, False),   # level 1: 256 tiles per head (the bitonic path)
])
def test_index_transpose_levels_bit_exact(h, w, levels, topk, block, enrich):
    """Every level's CSC in one call equals the oracle's CSC of that level's selection
    (counts, offsets, rows ascending per key), as the per-level call computes it."""
    d, _ = _inputs(1, 3, h, w, torch.bfloat16, 81)
    p = ops.make_problem(d["q"], h, w, levels, topk, enrich, 0.0, RASTER, block=block)
    fwd = ops.llsa_forward(p, d["q"], d["k"], d["v"])
    sel = [fwd["fine"]] + list(fwd["sel"][1:])
    offs, rows = ops.build_csc(p, sel)
    torch.cuda.synchronize()
    for l in range(1, 2 + p.coarse_levels):
        nl, kk = p.csc_dims(l)
        s_np = sel[l - 1].cpu().numpy()
        o_np, r_np = offs[l - 1].cpu().numpy(), rows[l - 1].cpu().numpy()
        for hi in range(3):
            want_off, want_rows = orc.csr_to_csc(s_np[0, hi].astype(np.int64), nl)
            assert np.array_equal(o_np[0, hi], want_off), (l, hi)
            assert np.array_equal(r_np[0, hi], want_rows), (l, hi)
        one_off = torch.empty_like(offs[l - 1])
        one_rows = torch.empty_like(rows[l - 1])
        ws = torch.empty(_abi.llsa_index_transpose_workspace(3, nl, nl, kk), device=DEV,
                         dtype=torch.uint8)
        _abi.llsa_index_transpose(3, nl, nl, kk, sel[l - 1], one_off, one_rows, ws)
        assert torch.equal(one_off, offs[l - 1]) and torch.equal(one_rows, rows[l - 1])
