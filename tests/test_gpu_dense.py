"""GPU parity of the dense full-attention baseline (the comparator of the speed-up figures)
against the fp64 CPU oracle, through the C ABI: forward output and log-sum-exp, and the three
gradients, on seeded inputs of the same distributions as the sparse workloads."""
import numpy as np
import pytest
import torch

from hierarchical_top_sparse_amd import _abi, gen
from oracle import llsa_oracle as orc
from tests.parity_util import assert_close, lse_tolerance, to64

pytestmark = pytest.mark.gpu


def _inputs(bh, n, seed):
    side = int(np.sqrt(n))
    h, w = (side, n // side) if side * (n // side) == n else (1, n)
    x = gen.make_inputs(1, bh, h, w, 64, torch.bfloat16, seed, with_grad=True)
    return {t: x[t].reshape(bh, n, 64).contiguous() for t in ("q", "k", "v", "do")}


@pytest.mark.parametrize("bh,n,seed", [(2, 128, 3), (2, 1024, 5), (1, 4096, 7), (3, 384, 9)])
def test_dense_forward_backward_match_oracle(bh, n, seed):
    x = _inputs(bh, n, seed)
    d = {t: v.cuda() for t, v in x.items()}
    o = torch.empty_like(d["q"])
    lse = torch.empty((bh, n), device="cuda", dtype=torch.float32)
    _abi.llsa_dense_attn_fwd(d["q"], d["k"], d["v"], o, lse)
    dq, dk, dv = (torch.empty_like(d["q"]) for _ in range(3))
    drows = torch.empty_like(lse)
    _abi.llsa_dense_attn_bwd(d["q"], d["k"], d["v"], d["do"], lse, dq, dk, dv, drows)
    torch.cuda.synchronize()
    for h in range(bh):
        q, k, v, do = (to64(x[t][h]) for t in ("q", "k", "v", "do"))
        want_o, want_lse = orc.dense_attention_forward(q, k, v)
        assert_close(to64(o[h]), want_o, torch.bfloat16, f"dense o n{n} h{h}")
        assert_close(lse[h], want_lse, torch.bfloat16, f"dense lse n{n} h{h}",
                     tol_abs=lse_tolerance(q, k, torch.bfloat16))
        for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv),
                                   orc.dense_attention_backward(q, k, v, do)):
            assert_close(to64(got[h]), want, torch.bfloat16, f"dense {name} n{n} h{h}")


def test_dense_is_deterministic():
    x = _inputs(2, 512, 11)
    d = {t: v.cuda() for t, v in x.items()}
    outs = []
    for _ in range(2):
        o = torch.empty_like(d["q"])
        lse = torch.empty((2, 512), device="cuda", dtype=torch.float32)
        _abi.llsa_dense_attn_fwd(d["q"], d["k"], d["v"], o, lse)
        g = [torch.empty_like(d["q"]) for _ in range(3)]
        _abi.llsa_dense_attn_bwd(d["q"], d["k"], d["v"], d["do"], lse, *g,
                                 torch.empty_like(lse))
        outs.append([o, lse] + g)
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
