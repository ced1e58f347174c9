"""The allocation-free backward (llsa_attn_bwd_noalloc), through the C ABI: bit-identical to
llsa_attn_bwd with a caller workspace (the same kernels on the library's own scratch array),
on two calls in a row, the second on a smaller problem than the first (the array keeps the
first call's contents, which the second must not read); problems whose workspace exceeds the
array are refused before anything is enqueued."""
import ctypes

import pytest
import torch

from hierarchical_top_sparse_amd import _abi, gen, ops

FAKE = 0x10000   # an aligned pointer the refused call never dereferences


def _bits(t):
    return t.contiguous().view(torch.int16).cpu()


def _run_both(batch, heads, side, levels, seed):
    x = gen.make_inputs(batch, heads, side, side, 64, torch.bfloat16, seed, with_grad=True)
    q, k, v, do = (x[t].cuda() for t in ("q", "k", "v", "do"))
    p = ops.make_problem(q, side, side, levels)
    fwd = ops.llsa_forward(p, q, k, v)
    sel = [fwd["fine"]] + list(fwd["sel"][1:])
    offs, rows = ops.build_csc(p, sel)
    _, ws_bytes = _abi.llsa_workspace_bytes(p)
    assert ws_bytes <= _abi.LLSA_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(ws_bytes, device="cuda", dtype=torch.uint8)
    want = [torch.empty_like(q) for _ in range(3)]
    _abi.llsa_attn_bwd(p, q, k, v, do, fwd["lse"], fwd["k_lv"], fwd["v_lv"], sel, offs, rows,
                       *want, ws)
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    _abi.llsa_attn_bwd_noalloc(p, q, k, v, do, fwd["lse"], fwd["k_lv"], fwd["v_lv"], sel, offs,
                               rows, *got)
    torch.cuda.synchronize()
    return want, got, ws_bytes


@pytest.mark.gpu
def test_noalloc_backward_equals_the_workspace_entry_on_two_calls():
    # first the benchmarked training shape (77 MiB of workspace), then a smaller problem
    sizes = []
    for batch, heads, side, levels, seed in ((2, 6, 256, 3, 3000), (1, 2, 128, 2, 17)):
        want, got, ws_bytes = _run_both(batch, heads, side, levels, seed)
        sizes.append(ws_bytes)
        for name, a, b in zip(("dq", "dk", "dv"), want, got):
            assert torch.equal(_bits(a), _bits(b)), f"{name} at {side}x{side} b{batch} h{heads}"
    assert sizes[1] < sizes[0]


def test_noalloc_backward_refuses_problems_beyond_its_scratch():
    """512x512 pixels, 6 heads: 154 MiB of workspace, above the 96 MiB array (host only)."""
    L = _abi.lib()
    p = _abi.Problem(batch=1, heads=6, height=512, width=512, levels=3)
    assert _abi.llsa_workspace_bytes(p)[1] > _abi.LLSA_NOALLOC_SCRATCH_BYTES
    f = ctypes.c_void_p(FAKE)
    lv = (ctypes.c_void_p * 6)(FAKE, FAKE, FAKE)
    st = L.llsa_attn_bwd_noalloc(ctypes.byref(p.c()), *([f] * 5), lv, lv, lv, lv, lv,
                                 *([f] * 3), None)
    assert st == 5 and b"allocation-free" in L.llsa_last_error()
