"""GPU parity of the hot path with 128-channel heads (head_dim 128) against the CPU oracle,
through the C ABI: pooling, the selection within the tie window, the forward and backward on
the oracle's selection (enrichment variants, popular key blocks, blocks of 64 tokens), the
whole path on the 128x128 and 256x256 workloads' shapes, and determinism.  Inputs are the
seeded generator's with 128 channels per head (smooth fields + noise for Q/K, N(0,1) for V,
dO); the enrichment-ablation setting these stand in for is the summary page's sec. 5.5 /
Table 5 (a variant of the method's switches, here crossed with the head width)."""
import numpy as np
import pytest
import torch

from hierarchical_top_sparse_amd import _abi, gen, ops
from oracle import llsa_oracle as orc
from tests.parity_util import assert_close, check_level, check_selection, lse_tolerance, to64

pytestmark = pytest.mark.gpu

DEV = "cuda"
D = 128
RASTER, MORTON = _abi.LLSA_LAYOUT_RASTER, _abi.LLSA_LAYOUT_MORTON


def _inputs(batch, heads, h, w, dtype, seed, grad=False):
    x = gen.make_inputs(batch, heads, h, w, D, dtype, seed, with_grad=grad)
    return {k: v.to(DEV) for k, v in x.items()}, {k: to64(v) for k, v in x.items()}


def _bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32).cpu()


def _levels(ref, t, h, w, levels, block=16, bi=0, hi=0):
    return orc.pool_levels(orc.reorder(ref[t][bi, hi], h, w), block, levels)


def _oracle_sel(ref, h, w, levels, topk, hi, block=16):
    return orc.select(_levels(ref, "q", h, w, levels, block, 0, hi),
                      _levels(ref, "k", h, w, levels, block, 0, hi), block, topk)


def _sel_tensors(p, sels, levels):
    sel_t = [torch.from_numpy(np.stack([sels[i][l] for i in range(2)])[None].astype(np.int32))
             .to(DEV) for l in range(levels)]
    if p.block == 16:
        return sel_t
    fine = torch.empty((1, 2, p.n // 16, p.fine_k), device=DEV, dtype=torch.int32)
    _abi.llsa_expand_blocks(p, sel_t[0], fine)
    return [fine] + sel_t[1:]


def _pooled_kv(p, k, v):
    kl = [torch.empty((1, 2, p.n_level(l), D), device=DEV) for l in range(1, p.levels + 1)]
    vl = [torch.empty((1, 2, p.n_level(l), D), device=DEV) for l in range(1, p.levels + 1)]
    _abi.llsa_pool(p, None, k, v, None, kl, vl)
    return kl, vl


@pytest.mark.parametrize("h,w,levels,dtype,layout,block", [
    (128, 128, 2, torch.bfloat16, RASTER, 16), (64, 64, 2, torch.float32, MORTON, 16),
    (256, 256, 3, torch.bfloat16, RASTER, 16), (256, 256, 2, torch.bfloat16, RASTER, 64)])
def test_pool_head128(h, w, levels, dtype, layout, block):
    d, ref = _inputs(1, 2, h, w, dtype, 101)
    p = ops.make_problem(d["q"], h, w, levels, 8, layout=layout, block=block)
    q, k, v = d["q"], d["k"], d["v"]
    if layout == MORTON:
        q, k, v = (ops.reorder(p, t) for t in (q, k, v))
        back = ops.reorder(p, q, inverse=True)
        assert torch.equal(_bits(back), _bits(d["q"]))
    lv = {t: [torch.empty((1, 2, p.n_level(l), D), device=DEV) for l in range(1, levels + 1)]
          for t in "qkv"}
    _abi.llsa_pool(p, q, k, v, lv["q"], lv["k"], lv["v"])
    for t in "qkv":
        want = orc.pool_levels(orc.reorder(ref[t], h, w), block, levels)
        for l in range(levels):
            got = to64(lv[t][l])
            assert np.abs(got - want[l]).max() <= 1e-5 * max(1.0, np.abs(want[l]).max()), (t, l)


@pytest.mark.parametrize("h,w,levels,topk", [(128, 128, 2, 8), (256, 256, 3, 8),
                                             (128, 128, 1, 32), (128, 256, 3, 5)])
def test_select_head128_within_tie_window(h, w, levels, topk):
    d, ref = _inputs(1, 2, h, w, torch.bfloat16, 102)
    p = ops.make_problem(d["q"], h, w, levels, topk)
    fwd = ops.llsa_forward(p, d["q"], d["k"], d["v"])
    q_lv = orc.pool_levels(orc.reorder(ref["q"], h, w), 16, levels)
    k_lv = orc.pool_levels(orc.reorder(ref["k"], h, w), 16, levels)
    sel = [s.cpu().numpy().astype(np.int64) for s in fwd["sel"]]
    flips = check_selection(sel, q_lv, k_lv, topk, f"D128 {h}x{w} L{levels}")
    total = sum(s.shape[0] * s.shape[1] * s.shape[2] for s in sel)
    assert flips <= max(2, total // 1000)


def test_select_head128_from_given_parent():
    h = w = 128
    d, ref = _inputs(1, 2, h, w, torch.bfloat16, 103)
    p = ops.make_problem(d["q"], h, w, 2)
    fwd = ops.llsa_forward(p, d["q"], d["k"], d["v"])
    parent = np.stack([orc.select_coarsest(_levels(ref, "q", h, w, 2, 16, 0, i)[1],
                                           _levels(ref, "k", h, w, 2, 16, 0, i)[1], 8)
                       for i in range(2)])
    sel = [torch.empty_like(fwd["sel"][0]),
           torch.from_numpy(parent[None].astype(np.int32)).to(DEV)]
    _abi.llsa_select(p, fwd["q_lv"], fwd["k_lv"], sel, level_hi=1, level_lo=1)
    got = sel[0].cpu().numpy().astype(np.int64)
    for i in range(2):
        check_level(got[0, i], _levels(ref, "q", h, w, 2, 16, 0, i)[0],
                    _levels(ref, "k", h, w, 2, 16, 0, i)[0], parent[i], 8, f"head {i}")


@pytest.mark.parametrize("h,w,levels,topk,enrich,layout,block,variant", [
    (64, 64, 2, 8, True, RASTER, 16, {}),
    (128, 256, 3, 8, True, RASTER, 16, {}),
    (128, 128, 2, 5, True, MORTON, 16, {}),
    (128, 128, 1, 32, False, RASTER, 16, {}),
    (128, 128, 2, 32, True, RASTER, 16, {}),
    (128, 256, 3, 8, True, RASTER, 16, dict(coarse_unit_weight=True,
                                             coarse_exclude_overlap=True)),
    (128, 256, 3, 8, True, RASTER, 16, dict(enrich_levels=1)),
    (256, 256, 2, 8, True, RASTER, 64, {}),
])
def test_attn_head128_on_oracle_indices(h, w, levels, topk, enrich, layout, block, variant):
    """Forward and backward in isolation on the oracle's selection, 128 channels per head."""
    d, ref = _inputs(1, 2, h, w, torch.bfloat16, 104, grad=True)
    p = ops.make_problem(d["q"], h, w, levels, topk, enrich, 0.0, layout,
                         variant.get("enrich_levels", 0), variant.get("coarse_unit_weight", False),
                         block, variant.get("coarse_exclude_overlap", False))
    sels = [_oracle_sel(ref, h, w, levels, topk, i, block) for i in range(2)]
    att = _sel_tensors(p, sels, levels)
    q, k, v, do = d["q"], d["k"], d["v"], d["do"]
    if layout == MORTON:
        q, k, v, do = (ops.reorder(p, t) for t in (q, k, v, do))
    kl, vl = _pooled_kv(p, k, v)
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, p.n), device=DEV)
    _abi.llsa_attn_fwd(p, q, k, v, kl, vl, att, o, lse)
    dq, dk, dv = ops.llsa_backward(p, q, k, v, dict(o=o, lse=lse, k_lv=kl, v_lv=vl, sel=att,
                                                    fine=att[0]), do)
    if layout == MORTON:
        o, dq, dk, dv = (ops.reorder(p, t, inverse=True) for t in (o, dq, dk, dv))
    kw = dict(enrich_levels=variant.get("enrich_levels", 0),
              coarse_weight=not variant.get("coarse_unit_weight", False),
              exclude_overlap=variant.get("coarse_exclude_overlap", False))
    res = orc.llsa_forward(ref["q"], ref["k"], ref["v"], h, w, block, levels, topk, enrich,
                           sel_override=[sels], **kw)
    assert_close(to64(o), res["o"], torch.bfloat16, "o")
    assert_close(lse, res["lse"], torch.bfloat16, "lse",
                 tol_abs=lse_tolerance(ref["q"], ref["k"], torch.bfloat16,
                                       levels if enrich else 0, D, block))
    want = orc.llsa_backward(ref["q"], ref["k"], ref["v"], ref["do"], h, w, block, levels,
                             [sels], enrich, **kw)
    for name, got, ref_g in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        assert_close(to64(got), ref_g, torch.bfloat16, name)


@pytest.mark.parametrize("h,w,levels,topk,enrich,popular", [
    (128, 128, 1, 8, False, 1.0),    # every query block picks blocks 0..7: 1024 picks each
    (256, 256, 3, 8, True, 0.5),     # overflow chunks of 128 picks, 128 channels
])
def test_attn_bwd_head128_popular_key_blocks(h, w, levels, topk, enrich, popular):
    d, ref = _inputs(1, 2, h, w, torch.bfloat16, 105, grad=True)
    p = ops.make_problem(d["q"], h, w, levels, topk, enrich)
    sels = [_oracle_sel(ref, h, w, levels, topk, i) for i in range(2)]
    rng = np.random.default_rng(4)
    for i in range(2):
        s1 = sels[i][0].copy()
        s1[rng.random(s1.shape[0]) < popular] = np.arange(topk)
        sels[i][0] = s1
    att = _sel_tensors(p, sels, levels)
    q, k, v, do = d["q"], d["k"], d["v"], d["do"]
    kl, vl = _pooled_kv(p, k, v)
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, p.n), device=DEV)
    _abi.llsa_attn_fwd(p, q, k, v, kl, vl, att, o, lse)
    dq, dk, dv = ops.llsa_backward(p, q, k, v, dict(o=o, lse=lse, k_lv=kl, v_lv=vl, sel=att),
                                   do)
    want = orc.llsa_backward(ref["q"], ref["k"], ref["v"], ref["do"], h, w, 16, levels, [sels],
                             enrich)
    for name, got, ref_g in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        assert_close(to64(got), ref_g, torch.bfloat16, name)


@pytest.mark.parametrize("cfg_name,heads_checked", [("ffhq128", [(0, 0), (3, 5)]),
                                                   ("px256_train", [(0, 1), (1, 4)])])
def test_e2e_head128(cfg_name, heads_checked):
    """The whole path (pool, select, forward, transposes, backward) on a workload's shape with
    128 channels per head, against the oracle on the GPU's selection."""
    cfg = gen.CONFIGS[cfg_name]
    h, w, L = cfg["height"], cfg["width"], cfg["levels"]
    d, ref = _inputs(cfg["batch"], cfg["heads"], h, w, torch.bfloat16, cfg["seed_base"] + 500,
                     grad=True)
    p = ops.make_problem(d["q"], h, w, L, 8)
    fwd = ops.llsa_forward(p, d["q"], d["k"], d["v"])
    grads = ops.llsa_backward(p, d["q"], d["k"], d["v"], fwd, d["do"])
    torch.cuda.synchronize()
    sel_np = [s.cpu().numpy().astype(np.int64) for s in fwd["sel"]]
    for bi, hi in heads_checked:
        sl = (slice(bi, bi + 1), slice(hi, hi + 1))
        q64, k64, v64 = (ref[t][sl] for t in "qkv")
        q_lv = orc.pool_levels(orc.reorder(q64, h, w), 16, L)
        k_lv = orc.pool_levels(orc.reorder(k64, h, w), 16, L)
        check_selection([s[sl] for s in sel_np], q_lv, k_lv, 8, f"{cfg_name} D128 b{bi} h{hi}")
        sels = [[[s[bi, hi] for s in sel_np]]]
        res = orc.llsa_forward(q64, k64, v64, h, w, 16, L, 8, True, sel_override=sels)
        assert_close(to64(fwd["o"][sl]), res["o"], torch.bfloat16, f"{cfg_name} D128 o")
        assert_close(fwd["lse"][sl], res["lse"], torch.bfloat16, f"{cfg_name} D128 lse",
                     tol_abs=lse_tolerance(q64, k64, torch.bfloat16, L, D))
        want = orc.llsa_backward(q64, k64, v64, ref["do"][sl], h, w, 16, L, sels, True)
        for name, got, ref_g in zip(("dq", "dk", "dv"), grads, want):
            assert_close(to64(got[sl]), ref_g, torch.bfloat16, f"{cfg_name} D128 {name}")


def test_head128_deterministic_and_autograd():
    h = w = 128
    d, _ = _inputs(1, 2, h, w, torch.bfloat16, 106, grad=True)
    outs = []
    for _ in range(2):
        q, k, v = (d[t].clone().requires_grad_(True) for t in "qkv")
        o = ops.llsa_attention(q, k, v, h, w, levels=2)
        o.backward(d["do"])
        outs.append([o.detach(), q.grad, k.grad, v.grad])
    for a, b in zip(*outs):
        assert torch.equal(_bits(a), _bits(b))


def test_head128_fp32_attention_is_refused():
    d, _ = _inputs(1, 1, 64, 64, torch.float32, 107)
    p = ops.make_problem(d["q"], 64, 64, 2)
    with pytest.raises(_abi.LlsaError) as e:
        ops.llsa_forward(p, d["q"], d["k"], d["v"])
    assert e.value.status == 4
