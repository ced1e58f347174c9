"""Host-side behaviour of the autograd op (no GPU): the forward state it keeps for the
backward is freed with the graph, without waiting for Python's cycle collector.

The library calls are replaced by stand-ins of the right shapes; what is checked is the
Function's bookkeeping, not the arithmetic (the GPU parity tests check that)."""
import gc
import weakref

import torch

from hierarchical_top_sparse_amd import ops


def _fake_forward(p, q, k, v):
    lv = lambda l: torch.zeros(p.batch, p.heads, p.n_level(l), p.head_dim)   # noqa: E731
    sel = [torch.zeros(p.batch, p.heads, p.n_level(l), p.topk, dtype=torch.int32)
           for l in range(1, p.levels + 1)]
    return dict(o=q * 2.0, lse=torch.zeros(p.batch, p.heads, p.n),
                q_lv=[lv(l) for l in range(1, p.levels + 1)],
                k_lv=[lv(l) for l in range(1, p.levels + 1)],
                v_lv=[None] + [lv(l) for l in range(2, p.levels + 1)], sel=sel, fine=sel[0])


def test_forward_state_is_freed_after_backward_without_gc(monkeypatch):
    seen = {}

    def fake_backward(p, q, k, v, fwd, dout):
        seen["fwd"] = {key: fwd[key] for key in ("lse", "fine", "k_lv", "v_lv", "sel")}
        assert "o" not in fwd
        return dout * 2.0, torch.zeros_like(k), torch.zeros_like(v)

    monkeypatch.setattr(ops, "llsa_forward", _fake_forward)
    monkeypatch.setattr(ops, "llsa_backward", fake_backward)
    gc.collect()
    gc.disable()
    try:
        q, k, v = (torch.randn(1, 2, 256, 64, requires_grad=True) for _ in range(3))
        o = ops.llsa_attention(q, k, v, 16, 16, levels=2)
        o_ref = weakref.ref(o)
        o.backward(torch.ones_like(o))
        assert torch.equal(q.grad, torch.full_like(q, 2.0))
        fwd = seen.pop("fwd")
        assert fwd["v_lv"][0] is None and len(fwd["k_lv"]) == 2 and len(fwd["sel"]) == 2
        lse_ref = weakref.ref(fwd["lse"])
        del fwd
        del o
        assert o_ref() is None, "the output is kept alive by a reference cycle"
        assert lse_ref() is None, "the saved forward state outlived the backward"
    finally:
        gc.enable()
