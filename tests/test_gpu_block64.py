"""GPU parity of the B = 64 variant (8x8-pixel blocks; the pages' Figure 3 compares B = 16 and
64) against the fp64 oracle run with block 64, through the C ABI: pooling, selection within
the tie window, the 16-token expansion of the level-1 picks, attention forward and backward on
the oracle's selection, and the whole path at the 256x256 training shape."""
import numpy as np
import pytest
import torch

from hierarchical_top_sparse_amd import _abi, gen, ops
from oracle import llsa_oracle as orc
from tests.parity_util import assert_close, check_selection, lse_tolerance, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"
B = 64
RASTER, MORTON = _abi.LLSA_LAYOUT_RASTER, _abi.LLSA_LAYOUT_MORTON


def _inputs(batch, heads, h, w, dtype, seed, grad=False):
    x = gen.make_inputs(batch, heads, h, w, 64, dtype, seed, with_grad=grad)
    return {k: v.to(DEV) for k, v in x.items()}, {k: to64(v) for k, v in x.items()}


def _problem(x, h, w, levels, topk, enrich=True, layout=RASTER):
    return ops.make_problem(x, h, w, levels, topk, enrich, 0.0, layout, block=B)


def _levels(ref, t, h, w, levels, bi=0, hi=0):
    return orc.pool_levels(orc.reorder(ref[t][bi, hi], h, w), B, levels)


@pytest.mark.parametrize("h,w,levels,dtype,layout", [
    (256, 256, 2, torch.bfloat16, RASTER), (64, 128, 1, torch.float32, MORTON),
    (512, 512, 3, torch.bfloat16, RASTER)])
def test_pool_block64_matches_oracle(h, w, levels, dtype, layout):
    d, ref = _inputs(1, 2, h, w, dtype, 71)
    p = _problem(d["q"], h, w, levels, 1, layout=layout)
    x = ops.reorder(p, d["k"]) if layout == MORTON else d["k"]
    kl = [torch.empty((1, 2, p.n_level(l), 64), device=DEV) for l in range(1, levels + 1)]
    _abi.llsa_pool(p, None, x, None, None, kl, [None] * levels)
    for hi in range(2):
        want = _levels(ref, "k", h, w, levels, 0, hi)
        for l in range(levels):
            got = kl[l][0, hi].double().cpu().numpy()
            assert np.abs(got - want[l]).max() <= 1e-5 * max(1.0, np.abs(want[l]).max()), l


@pytest.mark.parametrize("h,w,levels,topk", [(256, 256, 2, 8), (128, 128, 1, 8),
                                             (512, 512, 2, 6), (128, 256, 2, 5)])
def test_select_block64_within_tie_window(h, w, levels, topk):
    d, ref = _inputs(1, 2, h, w, torch.bfloat16, 72)
    p = _problem(d["q"], h, w, levels, topk)
    fwd = ops.llsa_forward(p, d["q"], d["k"], d["v"])
    sel = [s.cpu().numpy().astype(np.int64) for s in fwd["sel"]]
    q_lv = orc.pool_levels(orc.reorder(ref["q"], h, w), B, levels)
    k_lv = orc.pool_levels(orc.reorder(ref["k"], h, w), B, levels)
    flips = check_selection(sel, q_lv, k_lv, topk, f"B64 {h}x{w} L{levels}", block=B)
    total = sum(s.shape[0] * s.shape[1] * s.shape[2] for s in sel)
    assert flips <= max(2, total // 1000)
    # the expansion to 16-token blocks, by its definition
    fine = fwd["fine"].cpu().numpy()
    s1 = sel[0]
    want = (s1[:, :, np.arange(s1.shape[2] * 4) // 4, :, None] * 4 + np.arange(4)).reshape(
        fine.shape)
    assert np.array_equal(fine, want)


def _oracle_sel(ref, h, w, levels, topk, hi):
    q_lv = _levels(ref, "q", h, w, levels, 0, hi)
    k_lv = _levels(ref, "k", h, w, levels, 0, hi)
    return orc.select(q_lv, k_lv, B, topk)


def _gpu_sel(p, sels, levels):
    sel_t = [torch.from_numpy(np.stack([sels[i][l] for i in range(2)])[None].astype(np.int32))
             .to(DEV) for l in range(levels)]
    fine = torch.empty((1, 2, p.n // 16, p.fine_k), device=DEV, dtype=torch.int32)
    _abi.llsa_expand_blocks(p, sel_t[0], fine)
    return [fine] + sel_t[1:]


@pytest.mark.parametrize("h,w,levels,topk,enrich,dtype,layout", [
    (128, 128, 2, 4, True, torch.bfloat16, RASTER),
    (256, 256, 2, 8, True, torch.bfloat16, MORTON),
    (64, 64, 1, 8, False, torch.float32, RASTER),
    (512, 512, 3, 1, True, torch.bfloat16, RASTER),
])
def test_attn_fwd_block64_on_oracle_indices(h, w, levels, topk, enrich, dtype, layout):
    d, ref = _inputs(1, 2, h, w, dtype, 73)
    p = _problem(d["q"], h, w, levels, topk, enrich, layout)
    sels = [_oracle_sel(ref, h, w, levels, topk, i) for i in range(2)]
    att = _gpu_sel(p, sels, levels)
    q, k, v = d["q"], d["k"], d["v"]
    if layout == MORTON:
        q, k, v = (ops.reorder(p, t) for t in (q, k, v))
    kl = [torch.empty((1, 2, p.n_level(l), 64), device=DEV) for l in range(1, levels + 1)]
    vl = [torch.empty((1, 2, p.n_level(l), 64), device=DEV) for l in range(1, levels + 1)]
    _abi.llsa_pool(p, None, k, v, None, kl, vl)
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, p.n), device=DEV)
    _abi.llsa_attn_fwd(p, q, k, v, kl, vl, att, o, lse)
    if layout == MORTON:
        o = ops.reorder(p, o, inverse=True)
    res = orc.llsa_forward(ref["q"], ref["k"], ref["v"], h, w, B, levels, topk, enrich,
                           sel_override=[sels])
    assert_close(to64(o), res["o"], dtype, "o")
    assert_close(lse, res["lse"], dtype, "lse",
                 tol_abs=lse_tolerance(ref["q"], ref["k"], dtype, levels if enrich else 0,
                                       block=B))


@pytest.mark.parametrize("h,w,levels,topk,enrich", [
    (128, 128, 2, 4, True), (256, 256, 2, 8, True), (64, 128, 1, 6, False),
    (512, 512, 3, 1, True)])
def test_attn_bwd_block64_on_oracle_indices(h, w, levels, topk, enrich):
    d, ref = _inputs(1, 2, h, w, torch.bfloat16, 74, grad=True)
    p = _problem(d["q"], h, w, levels, topk, enrich)
    sels = [_oracle_sel(ref, h, w, levels, topk, i) for i in range(2)]
    att = _gpu_sel(p, sels, levels)
    q, k, v, do = d["q"], d["k"], d["v"], d["do"]
    kl = [torch.empty((1, 2, p.n_level(l), 64), device=DEV) for l in range(1, levels + 1)]
    vl = [torch.empty((1, 2, p.n_level(l), 64), device=DEV) for l in range(1, levels + 1)]
    _abi.llsa_pool(p, None, k, v, None, kl, vl)
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, p.n), device=DEV)
    _abi.llsa_attn_fwd(p, q, k, v, kl, vl, att, o, lse)
    fwd = dict(o=o, lse=lse, k_lv=kl, v_lv=vl, sel=att)
    dq, dk, dv = ops.llsa_backward(p, q, k, v, fwd, do)
    want = orc.llsa_backward(ref["q"], ref["k"], ref["v"], ref["do"], h, w, B, levels, [sels],
                             enrich)
    for name, got, ref_g in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        assert_close(to64(got), ref_g, torch.bfloat16, name)


def test_block64_overlap_exclusion_on_oracle_indices():
    """B = 64 with overlap-excluded coarse keys (256x256, L = 2, K = 8)."""
    h = w = 256
    levels, topk = 2, 8
    d, ref = _inputs(1, 2, h, w, torch.bfloat16, 75, grad=True)
    p = ops.make_problem(d["q"], h, w, levels, topk, True, 0.0, RASTER, block=B,
                         coarse_exclude_overlap=True)
    sels = [_oracle_sel(ref, h, w, levels, topk, i) for i in range(2)]
    att = _gpu_sel(p, sels, levels)
    q, k, v, do = d["q"], d["k"], d["v"], d["do"]
    kl = [torch.empty((1, 2, p.n_level(l), 64), device=DEV) for l in range(1, levels + 1)]
    vl = [torch.empty((1, 2, p.n_level(l), 64), device=DEV) for l in range(1, levels + 1)]
    _abi.llsa_pool(p, None, k, v, None, kl, vl)
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, p.n), device=DEV)
    _abi.llsa_attn_fwd(p, q, k, v, kl, vl, att, o, lse)
    dq, dk, dv = ops.llsa_backward(p, q, k, v, dict(o=o, lse=lse, k_lv=kl, v_lv=vl, sel=att),
                                   do)
    res = orc.llsa_forward(ref["q"], ref["k"], ref["v"], h, w, B, levels, topk, True,
                           sel_override=[sels], exclude_overlap=True)
    assert_close(to64(o), res["o"], torch.bfloat16, "o")
    want = orc.llsa_backward(ref["q"], ref["k"], ref["v"], ref["do"], h, w, B, levels, [sels],
                             True, exclude_overlap=True)
    for name, got, ref_g in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        assert_close(to64(got), ref_g, torch.bfloat16, name)


@pytest.mark.parametrize("enrich_levels,unit_weight,exclude", [
    (1, False, False),    # only level 2's coarse keys (64^2-token blocks)
    (0, True, False),     # both coarse levels, weight 1
    (0, True, True),      # weight 1 and overlap exclusion
    (1, False, True)])
def test_block64_enrichment_variants_on_oracle_indices(enrich_levels, unit_weight, exclude):
    """B = 64 at L = 3 (512x512, K = 1: level 3 is one block per head) crossed with the
    enrichment switches, forward and backward against the oracle on the oracle's selection."""
    h = w = 512
    levels, topk = 3, 1
    d, ref = _inputs(1, 2, h, w, torch.bfloat16, 76, grad=True)
    p = ops.make_problem(d["q"], h, w, levels, topk, True, 0.0, RASTER, enrich_levels,
                         unit_weight, block=B, coarse_exclude_overlap=exclude)
    sels = [_oracle_sel(ref, h, w, levels, topk, i) for i in range(2)]
    att = _gpu_sel(p, sels, levels)
    q, k, v, do = d["q"], d["k"], d["v"], d["do"]
    kl = [torch.empty((1, 2, p.n_level(l), 64), device=DEV) for l in range(1, levels + 1)]
    vl = [torch.empty((1, 2, p.n_level(l), 64), device=DEV) for l in range(1, levels + 1)]
    _abi.llsa_pool(p, None, k, v, None, kl, vl)
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, p.n), device=DEV)
    _abi.llsa_attn_fwd(p, q, k, v, kl, vl, att, o, lse)
    dq, dk, dv = ops.llsa_backward(p, q, k, v, dict(o=o, lse=lse, k_lv=kl, v_lv=vl, sel=att),
                                   do)
    kw = dict(enrich_levels=enrich_levels, coarse_weight=not unit_weight,
              exclude_overlap=exclude)
    res = orc.llsa_forward(ref["q"], ref["k"], ref["v"], h, w, B, levels, topk, True,
                           sel_override=[sels], **kw)
    assert_close(to64(o), res["o"], torch.bfloat16, "o")
    assert_close(lse, res["lse"], torch.bfloat16, "lse",
                 tol_abs=lse_tolerance(ref["q"], ref["k"], torch.bfloat16, levels, block=B))
    want = orc.llsa_backward(ref["q"], ref["k"], ref["v"], ref["do"], h, w, B, levels, [sels],
                             True, **kw)
    for name, got, ref_g in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        assert_close(to64(got), ref_g, torch.bfloat16, name)


def test_e2e_block64_px256_train():
    """The whole B = 64 path (L = 2, K = 8) at the 256x256 batch-2 training shape; two heads
    checked against the oracle on the GPU's selection."""
    cfg = gen.CONFIGS["px256_train"]
    h, w = cfg["height"], cfg["width"]
    d, ref = _inputs(cfg["batch"], cfg["heads"], h, w, cfg["dtype"], cfg["seed_base"], True)
    p = _problem(d["q"], h, w, 2, 8)
    fwd = ops.llsa_forward(p, d["q"], d["k"], d["v"])
    grads = ops.llsa_backward(p, d["q"], d["k"], d["v"], fwd, d["do"])
    torch.cuda.synchronize()
    sel_np = [s.cpu().numpy().astype(np.int64) for s in fwd["sel"]]
    for bi, hi in ((0, 1), (1, 4)):
        sl = (slice(bi, bi + 1), slice(hi, hi + 1))
        sels = [[[s[bi, hi] for s in sel_np]]]
        q64, k64, v64 = (ref[t][sl] for t in "qkv")
        res = orc.llsa_forward(q64, k64, v64, h, w, B, 2, 8, True, sel_override=sels)
        assert_close(to64(fwd["o"][sl]), res["o"], torch.bfloat16, f"o b{bi} h{hi}")
        want = orc.llsa_backward(q64, k64, v64, ref["do"][sl], h, w, B, 2, sels, True)
        for name, got, ref_g in zip(("dq", "dk", "dv"), grads, want):
            assert_close(to64(got[sl]), ref_g, torch.bfloat16, f"{name} b{bi} h{hi}")
