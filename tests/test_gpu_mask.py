"""GPU checks of the mask-based comparator (the dense-mask backward the article sets against
its index transpose, sec. 4.1 and Figure 4), through the C ABI:
  * the block mask is exactly the one-hot of Sel_1 (its definition, built here with numpy);
  * the backward whose key-major pass scans the mask gives dQ, dK, dV bit-identical to the
    CSC-based backward, and both match the oracle.
"""
import numpy as np
import pytest
import torch

from hierarchical_top_sparse_amd import gen, ops
from oracle import llsa_oracle as orc
from tests.parity_util import assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    return t.contiguous().view(torch.int16).cpu()


def _run(batch, heads, h, w, levels, topk, enrich, seed):
    x = gen.make_inputs(batch, heads, h, w, 64, torch.bfloat16, seed, with_grad=True)
    d = {t: v.to(DEV) for t, v in x.items()}
    p = ops.make_problem(d["q"], h, w, levels, topk, enrich)
    fwd = ops.llsa_forward(p, d["q"], d["k"], d["v"])
    csc = ops.llsa_backward(p, d["q"], d["k"], d["v"], fwd, d["do"])
    masked = ops.llsa_backward_masked(p, d["q"], d["k"], d["v"], fwd, d["do"])
    torch.cuda.synchronize()
    return x, p, fwd, csc, masked


@pytest.mark.parametrize("batch,heads,h,w,levels,topk,enrich,seed", [
    (1, 2, 64, 64, 1, 8, True, 61),        # n_1 = 256
    (1, 3, 128, 128, 1, 32, True, 62),     # the single-level top-32 shape
    (1, 2, 128, 256, 2, 8, False, 63),     # levels 2 without coarse keys; n_1 not a power of 4
    (2, 6, 256, 256, 1, 32, True, 64),     # the 256x256 training shape, single level
])
def test_masked_backward_matches_csc(batch, heads, h, w, levels, topk, enrich, seed):
    _, p, fwd, (dq, dk, dv), (mq, mk, mv, mask) = _run(batch, heads, h, w, levels, topk, enrich,
                                                       seed)
    sel = fwd["sel"][0].cpu().numpy()
    n1 = p.n_level(1)
    want = np.zeros((batch, heads, n1, n1), dtype=np.uint8)
    bi, hi, ai, _ = np.indices(sel.shape)
    want[bi, hi, ai, sel] = 1
    assert np.array_equal(mask.cpu().numpy(), want)
    assert torch.equal(_bits(dq), _bits(mq)), "dq"
    # the CSC pass cuts key blocks with more than 128 picks into chunks (partial sums added in
    # chunk order); the mask scan runs each block in one wave: bit-identical below that count
    counts = np.bincount(sel.reshape(-1) + n1 * np.repeat(np.arange(batch * heads),
                                                          sel.shape[2] * topk),
                         minlength=batch * heads * n1)
    for name, a, b in (("dk", dk, mk), ("dv", dv, mv)):
        if counts.max() <= 128:
            assert torch.equal(_bits(a), _bits(b)), name
        else:
            assert_close(to64(a), to64(b), torch.bfloat16, name)


def test_masked_backward_matches_oracle():
    h = w = 128
    x, p, fwd, _, (mq, mk, mv, _) = _run(1, 2, h, w, 1, 32, True, 65)
    ref = {t: to64(v) for t, v in x.items()}
    sels = [[[s[0, i].cpu().numpy().astype(np.int64) for s in fwd["sel"]] for i in range(2)]]
    want = orc.llsa_backward(ref["q"], ref["k"], ref["v"], ref["do"], h, w, 16, 1, sels, True)
    for name, got, ref_g in zip(("dq", "dk", "dv"), (mq, mk, mv), want):
        assert_close(to64(got), ref_g, torch.bfloat16, f"masked {name}")
