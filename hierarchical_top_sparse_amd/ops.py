"""LLSA as a PyTorch op: the whole hot path through the C ABI.

forward : [reorder] -> pool -> select -> sparse attention (-> inverse reorder)
backward: CSR->CSC transpose of every level (one call) -> sparse backward

With layout RASTER (the default) the reorder is folded into the kernels' addressing: the
inputs are raster-ordered pixel tokens and so are the outputs.  With layout MORTON the caller
supplies Morton-ordered tokens (llsa_reorder produces them) and gets Morton-ordered outputs.
PyTorch only allocates device memory and provides the stream.
"""
from __future__ import annotations

import torch

from . import _abi
from ._abi import (LLSA_BF16, LLSA_F32, LLSA_LAYOUT_MORTON, LLSA_LAYOUT_RASTER, Problem,
                   llsa_attn_bwd, llsa_attn_bwd_masked, llsa_attn_fwd, llsa_block_mask,
                   llsa_expand_blocks,
                   llsa_index_transpose_levels, llsa_index_transpose_levels_workspace,
                   llsa_pool_select,
                   llsa_reorder, llsa_workspace_bytes)

__all__ = ["Problem", "make_problem", "llsa_forward", "llsa_backward", "llsa_backward_masked",
           "llsa_attention", "dense_attention", "reorder", "LLSA_BF16", "LLSA_F32", "LLSA_LAYOUT_MORTON",
           "LLSA_LAYOUT_RASTER"]


def make_problem(q: torch.Tensor, height: int, width: int, levels: int, topk: int = 8,
                 enrich: bool = True, scale: float = 0.0, layout: int = LLSA_LAYOUT_RASTER,
                 enrich_levels: int = 0, coarse_unit_weight: bool = False,
                 block: int = 16, coarse_exclude_overlap: bool = False):
    b, h, n, d = q.shape
    if n != height * width:
        raise ValueError(f"token count {n} != height*width {height * width}")
    dtype = {torch.bfloat16: LLSA_BF16, torch.float32: LLSA_F32}.get(q.dtype)
    if dtype is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    return Problem(batch=b, heads=h, height=height, width=width, levels=levels, topk=topk,
                   enrich=int(enrich), head_dim=d, scale=scale, dtype=dtype, layout=layout,
                   enrich_levels=enrich_levels, coarse_unit_weight=int(coarse_unit_weight),
                   block=block, coarse_exclude_overlap=int(coarse_exclude_overlap))


def reorder(p: Problem, x: torch.Tensor, inverse: bool = False) -> torch.Tensor:
    y = torch.empty_like(x)
    llsa_reorder(p, x, y, inverse)
    return y


def llsa_forward(p: Problem, q, k, v):
    """Returns a dict: o, lse, q_lv, k_lv, v_lv (levels 1..L, v level 1 is None), sel (the
    selection of every level), fine (level 1 as 16-token blocks: sel[0] itself for B = 16)."""
    dev = q.device
    lv_shape = lambda l: (p.batch, p.heads, p.n_level(l), p.head_dim)
    f32 = dict(device=dev, dtype=torch.float32)
    q_lv = [torch.empty(lv_shape(l), **f32) for l in range(1, p.levels + 1)]
    k_lv = [torch.empty(lv_shape(l), **f32) for l in range(1, p.levels + 1)]
    # attention reads V's levels >= 2 only; level 1 is stored only where the next level is
    # pooled from it (block 64; with block 16 levels 1 and 2 both come from the tokens)
    v_lv = [torch.empty(lv_shape(1), **f32) if p.block != 16 and p.levels >= 2 else None] + [
        torch.empty(lv_shape(l), **f32) for l in range(2, p.levels + 1)]
    need_v = p.enrich and p.levels >= 2
    sel = [torch.empty((p.batch, p.heads, p.n_level(l), p.topk), device=dev, dtype=torch.int32)
           for l in range(1, p.levels + 1)]
    # pooling and selection in one call (V pooled inside the selection launches), as the step
    # runner issues them
    llsa_pool_select(p, q, k, v if need_v else None, q_lv, k_lv, v_lv, sel)
    fine = sel[0]
    if p.block != 16:
        fine = torch.empty((p.batch, p.heads, p.n // 16, p.fine_k), device=dev,
                           dtype=torch.int32)
        llsa_expand_blocks(p, sel[0], fine)
    o = torch.empty_like(q)
    lse = torch.empty((p.batch, p.heads, p.n), **f32)
    llsa_attn_fwd(p, q, k, v, k_lv, v_lv, [fine] + sel[1:], o, lse)
    return dict(o=o, lse=lse, q_lv=q_lv, k_lv=k_lv, v_lv=v_lv, sel=sel, fine=fine)


def build_csc(p: Problem, sel):
    """Per level l: CSC of the attention's selection (level 1 as 16-token blocks, sel[0] =
    the `fine` array; rows = queries, cols = keys): (off, rows), all levels in one call."""
    levels = 1 + p.coarse_levels
    dev = sel[0].device
    offs, rows = [], []
    for l in range(1, levels + 1):
        nl, kk = p.csc_dims(l)
        offs.append(torch.empty((p.batch, p.heads, nl + 1), device=dev, dtype=torch.int32))
        rows.append(torch.empty((p.batch, p.heads, nl * kk), device=dev, dtype=torch.int32))
    ws = torch.empty(llsa_index_transpose_levels_workspace(p), device=dev, dtype=torch.uint8)
    llsa_index_transpose_levels(p, sel, offs, rows, ws)
    return offs, rows


def llsa_backward(p: Problem, q, k, v, fwd: dict, dout):
    """Returns (dq, dk, dv) for the forward state `fwd`."""
    sel = [fwd.get("fine", fwd["sel"][0])] + list(fwd["sel"][1:])
    offs, rows = build_csc(p, sel)
    _, ws_bytes = llsa_workspace_bytes(p)
    ws = torch.empty(max(ws_bytes, 16), device=q.device, dtype=torch.uint8)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    llsa_attn_bwd(p, q, k, v, dout, fwd["lse"], fwd["k_lv"], fwd["v_lv"], sel, offs, rows, dq,
                  dk, dv, ws)
    return dq, dk, dv


def llsa_backward_masked(p: Problem, q, k, v, fwd: dict, dout):
    """The mask-based comparator of llsa_backward (no coarse keys): builds the dense level-1
    block mask from Sel_1 and runs the backward whose key-major pass scans it.  Returns
    (dq, dk, dv, mask)."""
    mask = torch.empty((p.batch, p.heads, p.n_level(1), p.n_level(1)), device=q.device,
                       dtype=torch.uint8)
    llsa_block_mask(p, fwd["sel"][0], mask)
    _, ws_bytes = llsa_workspace_bytes(p)
    ws = torch.empty(max(ws_bytes, 16), device=q.device, dtype=torch.uint8)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    llsa_attn_bwd_masked(p, q, k, v, dout, fwd["lse"], fwd["sel"][0], mask, dq, dk, dv, ws)
    return dq, dk, dv, mask


class _LLSAFunction(torch.autograd.Function):
    """The backward reads q, k, v, the LSE, the pooled K/V levels and the selections of the
    forward; those go through save_for_backward (freed once the backward has run).  The output
    o and the pooled Q are not kept: storing the forward's dict on ctx would make a reference
    cycle (output -> grad_fn -> ctx -> output) that only the cycle collector frees."""

    @staticmethod
    def forward(ctx, q, k, v, p):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        fwd = llsa_forward(p, q, k, v)
        ctx.p = p
        L = p.levels
        ctx.save_for_backward(q, k, v, fwd["lse"], fwd["fine"], *fwd["k_lv"], *fwd["v_lv"],
                              *fwd["sel"])
        ctx.levels = L
        return fwd["o"]

    @staticmethod
    def backward(ctx, dout):
        saved = ctx.saved_tensors
        L = ctx.levels
        q, k, v, lse, fine = saved[:5]
        k_lv = list(saved[5:5 + L])
        v_lv = list(saved[5 + L:5 + 2 * L])
        sel = list(saved[5 + 2 * L:5 + 3 * L])
        fwd = dict(lse=lse, fine=fine, k_lv=k_lv, v_lv=v_lv, sel=sel)
        dq, dk, dv = llsa_backward(ctx.p, q, k, v, fwd, dout.contiguous())
        return dq, dk, dv, None


def llsa_attention(q, k, v, height: int, width: int, levels: int, topk: int = 8,
                   enrich: bool = True, scale: float = 0.0, enrich_levels: int = 0,
                   coarse_unit_weight: bool = False, layout: int = LLSA_LAYOUT_RASTER,
                   block: int = 16):
    """Log-linear sparse attention over pixel tokens [b, H, height*width, 64] (raster order,
    or Morton order with layout LLSA_LAYOUT_MORTON).  enrich_levels / coarse_unit_weight
    select the enrichment variants (0 / False: the method as described); block 16 or 64."""
    p = make_problem(q, height, width, levels, topk, enrich, scale, layout, enrich_levels,
                     coarse_unit_weight, block)
    return _LLSAFunction.apply(q, k, v, p)


class _DenseFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, scale):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:-1], device=q.device, dtype=torch.float32)
        _abi.llsa_dense_attn_fwd(q, k, v, o, lse, scale)
        ctx.scale = scale
        ctx.save_for_backward(q, k, v, lse)
        return o

    @staticmethod
    def backward(ctx, dout):
        q, k, v, lse = ctx.saved_tensors
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        _abi.llsa_dense_attn_bwd(q, k, v, dout.contiguous(), lse, dq, dk, dv,
                                 torch.empty_like(lse), ctx.scale)
        return dq, dk, dv, None


def dense_attention(q, k, v, scale: float = 0.0):
    """The library's dense softmax attention over [..., N, 64] bf16 (the full-attention
    baseline), as an autograd op."""
    return _DenseFunction.apply(q, k, v, scale)
