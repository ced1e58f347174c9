"""llsa_pool_select against llsa_pool followed by llsa_select (levels L..1), through the C ABI:
the combined call pools V inside the selection launches where it can (block 16, bf16 tokens,
L >= 2) and must give bit-identical pooled levels and selections in every case, including the
cases it runs as the two plain calls (no V, L = 1, block 64, fp32).  The two plain calls are
themselves checked against the oracle by the parity tests."""
import pytest
import torch

from hierarchical_top_sparse_amd import _abi, gen, ops

pytestmark = pytest.mark.gpu
DEV = "cuda"
RASTER, MORTON = _abi.LLSA_LAYOUT_RASTER, _abi.LLSA_LAYOUT_MORTON


def _buffers(p, with_v):
    lv = lambda l: torch.full((p.batch, p.heads, p.n_level(l), 64), float("nan"), device=DEV)
    q_lv = [lv(l) for l in range(1, p.levels + 1)]
    k_lv = [lv(l) for l in range(1, p.levels + 1)]
    v_lv = None
    if with_v:   # V's level 1 is stored only where level 2 is pooled from it (block 64)
        v_lv = [lv(1) if p.block != 16 else None] + [lv(l) for l in range(2, p.levels + 1)]
    sel = [torch.full((p.batch, p.heads, p.n_level(l), p.topk), -7, device=DEV,
                      dtype=torch.int32) for l in range(1, p.levels + 1)]
    return q_lv, k_lv, v_lv, sel


@pytest.mark.parametrize("batch,heads,h,w,levels,topk,block,dtype,layout,with_v", [
    (2, 6, 256, 256, 3, 8, 16, torch.bfloat16, RASTER, True),    # V in both selection launches
    (1, 2, 128, 128, 2, 8, 16, torch.bfloat16, RASTER, True),    # L = 2: one selection launch
    (1, 2, 512, 512, 4, 4, 16, torch.bfloat16, MORTON, True),    # V's level 4 after them
    (1, 3, 256, 256, 3, 16, 16, torch.bfloat16, RASTER, True),   # K = 16
    (1, 2, 128, 256, 3, 8, 16, torch.bfloat16, RASTER, True),    # non-square
    (1, 2, 256, 256, 3, 8, 16, torch.bfloat16, RASTER, False),   # no V: the plain calls
    (1, 2, 64, 64, 1, 4, 16, torch.bfloat16, RASTER, False),     # L = 1
    (1, 2, 256, 256, 2, 8, 64, torch.bfloat16, RASTER, True),    # block 64: the plain calls
    (1, 2, 128, 128, 2, 8, 16, torch.float32, RASTER, True),     # fp32: the plain calls
    (1, 1, 16, 16, 2, 1, 16, torch.bfloat16, RASTER, True),      # the smallest problem
])
def test_pool_select_matches_the_two_calls(batch, heads, h, w, levels, topk, block, dtype,
                                           layout, with_v):
    x = gen.make_inputs(batch, heads, h, w, 64, dtype, 91)
    q, k, v = (x[t].to(DEV) for t in ("q", "k", "v"))
    p = ops.make_problem(q, h, w, levels, topk, True, 0.0, layout, block=block)
    vv = v if with_v else None
    q1, k1, v1, s1 = _buffers(p, with_v)
    _abi.llsa_pool(p, q, k, vv, q1, k1, v1)
    _abi.llsa_select(p, q1, k1, s1, levels, 1)
    q2, k2, v2, s2 = _buffers(p, with_v)
    _abi.llsa_pool_select(p, q, k, vv, q2, k2, v2, s2)
    torch.cuda.synchronize()
    for name, a, b in (("q", q1, q2), ("k", k1, k2), ("v", v1 or [], v2 or [])):
        for l, (ta, tb) in enumerate(zip(a, b), start=1):
            if ta is None:
                assert tb is None
                continue
            assert torch.equal(ta, tb), f"{name} level {l}"
            assert not torch.isnan(ta).any(), f"{name} level {l} not written"
    for l, (ta, tb) in enumerate(zip(s1, s2), start=1):
        assert torch.equal(ta, tb), f"selection level {l}"
        assert (ta >= 0).all(), f"selection level {l} not written"


def test_pool_select_twice_in_a_row_same_result():
    """Two calls in a row (the second on the same buffers) give the same levels and picks."""
    x = gen.make_inputs(2, 6, 256, 256, 64, torch.bfloat16, 92)
    q, k, v = (x[t].to(DEV) for t in ("q", "k", "v"))
    p = ops.make_problem(q, 256, 256, 3, 8)
    q2, k2, v2, s2 = _buffers(p, True)
    _abi.llsa_pool_select(p, q, k, v, q2, k2, v2, s2)
    first = [t.clone() for t in s2] + [t.clone() for t in v2 if t is not None]
    _abi.llsa_pool_select(p, q, k, v, q2, k2, v2, s2)
    torch.cuda.synchronize()
    again = list(s2) + [t for t in v2 if t is not None]
    for a, b in zip(first, again):
        assert torch.equal(a, b)
