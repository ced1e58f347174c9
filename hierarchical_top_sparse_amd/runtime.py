"""A preallocated LLSA training step (forward + backward) with optional HIP-graph replay.

`Step` owns every intermediate of one fwd+bwd pass (pooled levels, selections, O, LSE, CSC
indices, workspaces, gradients) for fixed shapes, and issues the C-ABI calls of a step in
order.  `capture()` records the whole sequence into a HIP graph (torch.cuda.CUDAGraph on
ROCm) so that replays do not wait on the host between calls; the library allocates nothing
and never synchronises, and none of its calls records a memset, so the whole step can be
captured.

The CSR->CSC transposes (every level in one call) depend only on the selection, and the sparse
forward does not read them: `run(overlap=True)` (the default) issues them on a second stream,
forked after the selection and joined before the backward, so that these small, latency-bound
kernels run beside the HBM-bound forward instead of after it.  All streams have the default
priority.
"""
from __future__ import annotations

import torch

from . import _abi


class Step:
    """dout=None makes a forward-only step (pooling, selection, sparse attention)."""

    def __init__(self, p: _abi.Problem, q, k, v, dout=None, fuse_prologue: bool = True):
        self.p = p
        # one llsa_pool_select call (V pooled inside the selection launches) instead of
        # llsa_pool + llsa_select; the same pooled levels and picks either way
        self.fuse_prologue = fuse_prologue
        self.q, self.k, self.v, self.dout = q, k, v, dout
        self.backward = dout is not None
        dev, f32 = q.device, torch.float32
        L = p.levels
        lv = lambda l: torch.empty((p.batch, p.heads, p.n_level(l), p.head_dim), device=dev,
                                   dtype=f32)
        self.q_lv = [lv(l) for l in range(1, L + 1)]
        self.k_lv = [lv(l) for l in range(1, L + 1)]
        # V level 1 only where level 2 is pooled from it (block 64)
        self.v_lv = [lv(1) if p.block != 16 and L >= 2 else None] + [lv(l) for l in range(2, L + 1)]
        self.pool_v = bool(p.enrich) and L >= 2
        self.sel = [torch.empty((p.batch, p.heads, p.n_level(l), p.topk), device=dev,
                                dtype=torch.int32) for l in range(1, L + 1)]
        # level 1 as the attention reads it (16-token blocks): sel[0] itself for B = 16
        self.fine = (self.sel[0] if p.block == 16 else
                     torch.empty((p.batch, p.heads, p.n // 16, p.fine_k), device=dev,
                                 dtype=torch.int32))
        self.att_sel = [self.fine] + self.sel[1:]
        self.o = torch.empty_like(q)
        self.lse = torch.empty((p.batch, p.heads, p.n), device=dev, dtype=f32)
        self.csc_levels = 1 + p.coarse_levels if self.backward else 0
        dims = [p.csc_dims(l) for l in range(1, self.csc_levels + 1)]
        self.off = [torch.empty((p.batch, p.heads, nl + 1), device=dev, dtype=torch.int32)
                    for nl, _ in dims]
        self.rows = [torch.empty((p.batch, p.heads, nl * kk), device=dev, dtype=torch.int32)
                     for nl, kk in dims]
        self.nmat = p.batch * p.heads
        tws = _abi.llsa_index_transpose_levels_workspace(p) if self.backward else 0
        self.tws = torch.empty(max(tws, 16), device=dev, dtype=torch.uint8)
        _, bws = _abi.llsa_workspace_bytes(p) if self.backward else (0, 0)
        self.bws = torch.empty(max(bws, 16), device=dev, dtype=torch.uint8)
        self.dq, self.dk, self.dv = ((torch.empty_like(q) for _ in range(3)) if self.backward
                                     else (None, None, None))
        self.graph = None
        self.side = torch.cuda.Stream(device=dev)

    def _transpose_calls(self):
        if not self.csc_levels:
            return []
        return [("transpose", lambda: _abi.llsa_index_transpose_levels(
            self.p, self.att_sel, self.off, self.rows, self.tws))]

    def calls(self):
        """(name, thunk) for every C-ABI call of one step, in order (one stream)."""
        a, p = _abi, self.p
        vv = self.v if self.pool_v else None
        if self.fuse_prologue:
            head = [("pool_select", lambda: a.llsa_pool_select(p, self.q, self.k, vv, self.q_lv,
                                                               self.k_lv, self.v_lv, self.sel))]
        else:
            head = [("pool", lambda: a.llsa_pool(p, self.q, self.k, vv, self.q_lv, self.k_lv,
                                                 self.v_lv)),
                    ("select", lambda: a.llsa_select(p, self.q_lv, self.k_lv, self.sel))]
        if p.block != 16:
            head.append(("expand", lambda: a.llsa_expand_blocks(p, self.sel[0], self.fine)))
        fwd = [("attn_fwd", lambda: a.llsa_attn_fwd(p, self.q, self.k, self.v, self.k_lv,
                                                     self.v_lv, self.att_sel, self.o, self.lse))]
        bwd = [("attn_bwd", lambda: a.llsa_attn_bwd(
            p, self.q, self.k, self.v, self.dout, self.lse, self.k_lv, self.v_lv, self.att_sel,
            self.off, self.rows, self.dq, self.dk, self.dv, self.bws))] if self.backward else []
        self._parts = (head, fwd, self._transpose_calls(), bwd)
        return head + fwd + self._parts[2] + bwd

    def run(self, overlap: bool = True):
        """One step on the current stream; with overlap, the transposes run on a side stream
        between the selection and the backward."""
        self.calls()
        head, fwd, tr, bwd = self._parts
        for _, fn in head:
            fn()
        if not overlap or not tr:
            for _, fn in fwd + tr + bwd:
                fn()
            return
        main = torch.cuda.current_stream()
        self.side.wait_stream(main)
        # the forward is issued first, so that a captured graph keeps it on the selection's
        # queue and only the (shorter) transposes cross to another one
        for _, fn in fwd:
            fn()
        with torch.cuda.stream(self.side):
            for _, fn in tr:
                fn()
        main.wait_stream(self.side)
        for _, fn in bwd:
            fn()

    def capture(self, warmup: int = 1):
        """Record one step into a HIP graph (after `warmup` eager steps on a side stream)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(warmup):
                self.run()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run()
        torch.cuda.synchronize()
        self.graph = g
        return g

    def replay(self):
        self.graph.replay()

    def outputs(self):
        return dict(o=self.o, lse=self.lse, dq=self.dq, dk=self.dk, dv=self.dv, sel=self.sel)
