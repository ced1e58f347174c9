"""GPU checks of the step runner: HIP-graph replays of a whole fwd+bwd step (transposes on a
side stream) equal the one-stream eager step bit for bit (several replays, with eager work
and synchronisations in between), and the per-kernel profiling hook reports every kernel of
a step."""
import pytest
import torch

from hierarchical_top_sparse_amd import _abi, gen, ops
from hierarchical_top_sparse_amd.runtime import Step

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


def _make(h=128, w=128, levels=2, batch=1, heads=2, seed=61, fuse_prologue=True, block=16):
    x = gen.make_inputs(batch, heads, h, w, 64, torch.bfloat16, seed, with_grad=True)
    q, k, v, do = (x[t].cuda() for t in ("q", "k", "v", "do"))
    return Step(ops.make_problem(q, h, w, levels, block=block), q, k, v, do,
                fuse_prologue=fuse_prologue)


@pytest.mark.parametrize("h,w,levels,block", [(128, 128, 2, 16), (128, 256, 3, 16),
                                              (256, 256, 2, 64)])
def test_graph_replays_match_eager(h, w, levels, block):
    """The reference is the eager one-stream step with llsa_pool + llsa_select; the graph is
    the overlapped step with llsa_pool_select (with block 64 it runs the two plain calls, and
    the step expands the level-1 picks to 16-token blocks)."""
    step = _make(h, w, levels, fuse_prologue=False, block=block)
    step.run(overlap=False)    # one stream: the reference for the overlapped graph
    torch.cuda.synchronize()
    want = {k: v.clone() for k, v in step.outputs().items() if k != "sel"}
    want_sel = [s.clone() for s in step.sel]
    want_csc = [t.clone() for t in step.off + step.rows]
    step.fuse_prologue = True
    step.capture()
    other = _make(64, 64, 2, seed=62)
    for rep in range(3):
        for t in (step.o, step.dq, step.dk, step.dv, step.lse):
            t.zero_()
        for t in step.off + step.rows + step.sel:
            t.fill_(-1)
        torch.cuda.synchronize()
        step.replay()
        torch.cuda.synchronize()
        for name, ref in want.items():
            assert torch.equal(_bits(getattr(step, name)), _bits(ref)), (rep, name)
        for s, ref in zip(step.sel, want_sel):
            assert torch.equal(s, ref), rep
        for t, ref in zip(step.off + step.rows, want_csc):
            assert torch.equal(t, ref), rep
        other.run()             # unrelated eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("fuse_prologue,select_name", [(True, "select_pool_kernel"),
                                                       (False, "select_kernel")])
def test_profile_hook_reports_every_kernel(fuse_prologue, select_name):
    step = _make(fuse_prologue=fuse_prologue)
    step.run()
    torch.cuda.synchronize()
    _abi.llsa_profile_read()
    _abi.llsa_profile_enable(True)
    step.run()
    step.run()
    _abi.llsa_profile_enable(False)
    prof = _abi.llsa_profile_read()
    for name in ("pool12_kernel", select_name, "attn_fwd_kernel", "csc_radix_kernel",
                 "csc_assemble_kernel", "bwd_query_kernel", "coarse_grad_kernel",
                 "bwd_key_kernel"):
        assert name in prof, name
        cnt, ms = prof[name]
        assert cnt >= 2 and ms > 0.0
    # with 64 channels the overflow chunks lead the key-major launch: no launch of their own
    assert "bwd_key_overflow_kernel" not in prof
    assert _abi.llsa_profile_read() == {}


@pytest.mark.parametrize("cfg_name", ["px256_train", "px512_train"])
def test_benchmarked_graph_equals_the_parity_tested_path(cfg_name):
    """The step the benchmark times (HIP-graph replays of the whole step: llsa_pool_select,
    attention, transposes on the side stream, backward) at the workload's full size gives the
    same bits as ops.llsa_forward / ops.llsa_backward, which the end-to-end parity tests check
    against the oracle at the same sizes."""
    cfg = gen.CONFIGS[cfg_name]
    h, w, L = cfg["height"], cfg["width"], cfg["levels"]
    x = gen.make_inputs(cfg["batch"], cfg["heads"], h, w, 64, cfg["dtype"], cfg["seed_base"],
                        with_grad=True)
    q, k, v, do = (x[t].cuda() for t in ("q", "k", "v", "do"))
    p = ops.make_problem(q, h, w, L)
    fwd = ops.llsa_forward(p, q, k, v)
    dq, dk, dv = ops.llsa_backward(p, q, k, v, fwd, do)
    torch.cuda.synchronize()
    step = Step(p, q, k, v, do)
    step.capture()
    for _ in range(3):
        step.replay()
    torch.cuda.synchronize()
    for name, ref in (("o", fwd["o"]), ("lse", fwd["lse"]), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.equal(_bits(getattr(step, name)), _bits(ref)), name
    for a, b in zip(step.sel, fwd["sel"]):
        assert torch.equal(a, b)
