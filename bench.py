"""LLSA fwd+bwd throughput on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic pixel tokens already
resident in HBM: pooling -> coarse-to-fine selection -> sparse attention forward -> CSR->CSC
transpose of every level -> sparse backward (dQ, dK, dV); the Morton reorder is folded into
the kernels' addressing (inputs and outputs stay in raster order).  The step is captured once
into a HIP graph and replayed; `value` is batch*N tokens per second of graph replays.  A
second, eager pass with per-kernel HIP events (recorded by the library on each kernel's own
stream; this pass issues every call on one stream, so each kernel is timed alone) gives each
kernel's launch duration.  Every row of the path is priced as a unit
(`extra.units`: its algorithmic bytes per step over the summed time of its launches); the
roofline object is for the unit with the largest time (the backward: its four kernels),
against the vendor HBM peak and against the achievable peak the library's own streaming-copy
kernel reaches (`extra.calibration`, with the MFMA-only loop's bf16 rate).  The pooling,
selection and transpose kernels get their own HBM fractions (`extra.side_kernels`, units).
The CPU baseline runs the oracle over the whole workload on the host's cores first, before
the GPU is touched.  Prints one JSON line.

Beside the headline, `extra` carries:
  * configs: every workload (forward only for the three forward configs, forward + backward
    for the two training ones), each timed the same way, with the HBM and MFMA fractions of
    its attention kernels;
  * dense_baseline: the library's own dense flash attention at the same shapes (forward at
    256x256 batch 1, forward + backward at the headline shape) and the speed-up ratios.

  * single_level_top32 / mask_backward_comparator: the single-level comparators (one level,
    K = 32 over all blocks; the dense-mask backward) on the headline inputs.
--sweep prints one JSON line per side length (64..512) instead: LLSA (B = 16 and B = 64)
against dense attention and against the single-level comparators.  --dit prints one line for
the synthetic Pixel-DiT-S training step (LLSA against dense attention inside the network).

  python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config px256_train] [--no-cpu]
                  [--no-configs] [--no-dense] [--sweep] [--dit]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0   # dense bf16 MFMA
FP32_MFMA_PEAK_TFLOPS = 157.3    # fp32 (the fp32 workload runs on the fp32 MFMA)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="px256_train")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead")
    ap.add_argument("--layout", choices=("raster", "morton"), default="raster",
                    help="token order of the resident tensors: raster (the reorder is folded into "
                         "every kernel's addressing) or morton (inputs reordered once before "
                         "timing, as when the reorder is hoisted to the network entry)")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-workload table")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense baseline")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the bench line: LLSA vs the dense baseline across "
                         "resolutions 64^2 .. 512^2 (batch 1, 6 heads), one JSON line each")
    ap.add_argument("--dit", action="store_true",
                    help="time the synthetic Pixel-DiT-S training step (LLSA vs dense) instead")
    ap.add_argument("--with-copy", action="store_true",
                    help="also launch one Morton reorder (a plain copy of one token tensor) per "
                         "step, outside the timed region: the calibration kernel for HBM "
                         "byte counters")
    return ap.parse_args()


def kernel_model(p, elem_bytes=None):
    """Algorithmic (compulsory) HBM bytes and FLOPs per launch of the attention kernels.

    T = one [b, H, N, 64] token tensor.  Gathers of selected key blocks count once (the
    compulsory traffic); index arrays and pooled levels are counted in full.
    """
    bh, n, d, K, L = p.batch * p.heads, p.n, p.head_dim, p.topk, p.levels
    if elem_bytes is None:
        elem_bytes = 2 if p.torch_dtype == torch_bf16() else 4
    T = bh * n * d * elem_bytes
    kq_fine = K * 16
    n_coarse = p.coarse_levels * K
    kq = kq_fine + n_coarse
    pooled = sum(bh * (n // 16 ** l) * d * 4 * 2 for l in range(2, 2 + p.coarse_levels))
    sel_bytes = sum(bh * (n // 16 ** l) * K * 4 for l in range(1, L + 1))
    tok4 = bh * n * 4                                     # one fp32 per token (lse or D)
    n2 = n // 256
    partials = bh * n2 * n_coarse * d * 4 * 2
    csc1 = bh * ((n // 16) + 1) * 4 + bh * (n // 16) * K * 4
    return {
        "attn_fwd_kernel": dict(bytes=4 * T + tok4 + sel_bytes + pooled,
                                flops=4 * bh * n * kq * d),
        "bwd_query_kernel": dict(bytes=5 * T + 2 * tok4 + sel_bytes + pooled + partials,
                                 flops=6 * bh * n * kq * d),
        "bwd_key_kernel": dict(bytes=6 * T + 2 * tok4 + csc1,
                               flops=8 * bh * n * kq_fine * d),
    }


def torch_bf16():
    import torch
    return torch.bfloat16


def unit_model(p):
    """Algorithmic HBM bytes (and FLOPs) per step of each row of the hot path, with the kernels
    that run it inside the benchmarked step.  Returns (units, side): the units of the scope
    table's measurement section, and the pooling / selection kernels one by one.

    T = one [b, H, N, 64] token tensor, L_l = one fp32 pooled level l of one tensor.
      * forward (a5): per query token q, o and its share of K and V read once (4 d bytes of
        the token dtype) plus its fp32 LSE;
      * backward (a7): per query token Q, K, V, O, dO read and dQ, dK, dV written (8 d bytes)
        plus LSE and D (this path recomputes D and never reads O, so it moves 7 of the 8
        token tensors, but the unit is priced as stated);
      * pooling and selection (a2-a4, one llsa_pool_select call): the three token tensors
        read once, every stored level written (V's level 1 is not stored), each level >= 3
        pooled from the one below; every pooled level of Q and K read once by the selection
        and every selection written.  Its kernels: pool12 (Q and K: 2T read, levels 1-2
        written), pool_next (Q and K levels >= 3, V's >= 4) and select_pool (the two
        selection launches, which also pool V: T read, its levels 2-3 written);
      * index transpose (a6): per level, the selection read and its CSC written (offsets and
        rows).
    Attention FLOPs: forward 4 k_q d, backward 10 k_q d per query (k_q keys per query)."""
    bh, n, d, K, L = p.batch * p.heads, p.n, p.head_dim, p.topk, p.levels
    es = 2 if p.torch_dtype == torch_bf16() else 4
    tokens = bh * n
    T = tokens * d * es
    kq = 16 * p.fine_k + p.coarse_levels * K
    lvb = lambda l: bh * p.n_level(l) * d * 4 if l <= L else 0      # noqa: E731
    selection = 2 * sum(lvb(l) for l in range(1, L + 1)) + sum(
        bh * p.n_level(l) * K * 4 for l in range(1, L + 1))
    side = {
        "pool12_kernel": 2 * T + 2 * (lvb(1) + lvb(2)),
        "pool_next_kernel": sum(2 * (lvb(l - 1) + lvb(l)) for l in range(3, L + 1)) +
                            sum(lvb(l - 1) + lvb(l) for l in range(4, L + 1)),
        "select_pool_kernel": T + lvb(2) + (lvb(2) + lvb(3) if L >= 3 else 0) + selection,
    }
    units = {
        "pool_select": dict(kernels=list(side), bytes=sum(side.values()),
                            flops=2 * d * bh * (p.n_level(L) ** 2 + sum(
                                p.n_level(l) * K * p.block for l in range(1, L)))),
        "attn_fwd": dict(kernels=["attn_fwd_kernel"], bytes=tokens * (4 * d * es + 4),
                         flops=4 * tokens * kq * d),
        "index_transpose": dict(
            kernels=["csc_radix_kernel", "csc_assemble_kernel", "tile_sort_kernel",
                     "merge_kernel", "csc_bounds_kernel", "csc_offsets_kernel",
                     "csc_scatter_kernel"],
            bytes=sum(bh * (2 * nl * kk * 4 + (nl + 1) * 4)
                      for nl, kk in (p.csc_dims(l) for l in range(1, 2 + p.coarse_levels))),
            flops=0),
        "attn_bwd": dict(kernels=["bwd_query_kernel", "coarse_grad_kernel",
                                  "bwd_key_overflow_kernel", "bwd_key_kernel"],
                         bytes=tokens * (8 * d * es + 8), flops=10 * tokens * kq * d),
    }
    return units, side


def traffic_record(config):
    """Measured HBM bytes per launch of every kernel of the step, from the committed counter
    record of the workload; a kernel's entry counts only if it was taken on the current source
    of the kernel's file."""
    path = os.path.join(ROOT, "profiles", f"{config}_traffic.json")
    if not os.path.exists(path):
        return {}
    rec = json.load(open(path))
    out = {}
    for name, k in rec.get("kernels", {}).items():
        src = os.path.join(ROOT, k["source"])
        if not os.path.exists(src):
            continue
        if hashlib.sha256(open(src, "rb").read()).hexdigest() == k.get("source_sha256"):
            out[name] = k
    return out


_CPU_SLICES = None   # fp32 copies of the workload's tensors, set before the worker pool forks


def _cpu_slice(task):
    """The oracle's forward + backward on one (batch, head) slice (in a worker process, with
    single-threaded BLAS); returns the seconds it took."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import llsa_oracle as orc
    b, hh, h, w, L = task
    with threadpool_limits(1):
        r = {t: _CPU_SLICES[t][b:b + 1, hh:hh + 1].astype(np.float64)
             for t in ("q", "k", "v", "do")}
        t0 = time.perf_counter()
        res = orc.llsa_forward(r["q"], r["k"], r["v"], h, w, 16, L, 8, True)
        orc.llsa_backward(r["q"], r["k"], r["v"], r["do"], h, w, 16, L, res["sel"], True)
        return time.perf_counter() - t0


def cpu_baseline(cfg, x):
    """The oracle (as it stands) over the whole workload on the host's cores: its (batch,
    head) slices are independent, so one worker process per core runs them (single-threaded
    BLAS each; the oracle is bound by its Python loops, and threads or more BLAS threads do
    not speed it up).  Must run before anything touches the GPU: the workers are forked."""
    import multiprocessing as mp
    global _CPU_SLICES
    h, w, L = cfg["height"], cfg["width"], cfg["levels"]
    _CPU_SLICES = {t: x[t].float().numpy() for t in ("q", "k", "v", "do")}
    slices = [(b, hh, h, w, L) for b in range(cfg["batch"]) for hh in range(cfg["heads"])]
    workers = max(1, min(len(os.sched_getaffinity(0)), 16, len(slices)))
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers) as pool:
        busy = pool.map(_cpu_slice, slices, chunksize=1)
    wall = time.perf_counter() - t0
    _CPU_SLICES = None
    tokens = cfg["batch"] * h * w
    return dict(value=round(tokens / wall, 1), unit="tokens/s", cores=workers, kind="oracle",
                sample=f"the whole workload: all {len(slices)} (batch, head) slices, fwd+bwd, "
                       f"in {wall:.1f} s wall on {workers} worker processes (one per host "
                       f"core, single-threaded BLAS); {sum(busy):.1f} s of CPU work")


def _event_ms(fn, reps):
    import torch
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(reps):
        fn()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / reps


def _graph_ms(fn, reps=20, replays=5):
    """Average duration of fn() from a HIP graph of `reps` back-to-back calls."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(replays):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / (reps * replays)


def prologue_parts(step):
    """What the pooling-and-selection launches hold (graph-timed, each part alone on the step's
    buffers): Q and K's pooling, V's pooling, the selection of every level, and the fused
    llsa_pool_select the step issues (V's pooling riding in the selection launches)."""
    from hierarchical_top_sparse_amd import _abi
    s, p = step, step.p
    parts = {
        "pool_select": lambda: _abi.llsa_pool_select(p, s.q, s.k, s.v, s.q_lv, s.k_lv,
                                                     s.v_lv, s.sel),
        "pool_qk": lambda: _abi.llsa_pool(p, s.q, s.k, None, s.q_lv, s.k_lv, s.v_lv),
        "pool_v": lambda: _abi.llsa_pool(p, None, None, s.v, s.q_lv, s.k_lv, s.v_lv),
        "select": lambda: _abi.llsa_select(p, s.q_lv, s.k_lv, s.sel),
    }
    return {f"{k}_ms": round(_graph_ms(f), 4) for k, f in parts.items()}


def measure(step, steps, warmup, graph=True, with_copy=None):
    """Eager pass with per-kernel events, then the timed region (graph replays or eager
    steps).  Returns (ms_step, eager_ms, per_call, per_kernel_ms, per_step_kernel_ms)."""
    import torch

    from hierarchical_top_sparse_amd import _abi
    calls = step.calls()
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        step.run()
    torch.cuda.synchronize()
    if with_copy is not None:
        for _ in range(max(1, steps)):
            with_copy()
        torch.cuda.synchronize()
    _abi.llsa_profile_read()
    _abi.llsa_profile_enable(True)
    ev = {name: [] for name, _ in calls}
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e_start.record(stream)
    for _ in range(steps):
        for name, fn in calls:
            a0 = torch.cuda.Event(enable_timing=True)
            a1 = torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            fn()
            a1.record(stream)
            ev[name].append((a0, a1))
    e_end.record(stream)
    torch.cuda.synchronize()
    _abi.llsa_profile_enable(False)
    kprof = _abi.llsa_profile_read()
    eager_ms = e_start.elapsed_time(e_end) / steps
    per_call = {name: sum(a.elapsed_time(b) for a, b in pairs) / len(pairs)
                for name, pairs in ev.items()}
    per_kernel_ms = {name: tot / cnt for name, (cnt, tot) in kprof.items()}
    per_step_kernel_ms = {name: tot / steps for name, (cnt, tot) in kprof.items()}
    if graph:
        step.capture()
        for _ in range(warmup):
            step.replay()
        ms_step = _event_ms(step.replay, steps)
    else:
        ms_step = _event_ms(step.run, steps)
    return ms_step, eager_ms, per_call, per_kernel_ms, per_step_kernel_ms


def calibration(reps=10):
    """Achievable peaks from the library's calibration kernels: a plain streaming copy of
    2 GiB (read + write bytes over time) and an MFMA-only loop of v_mfma_f32_16x16x32_bf16
    (16 waves per CU, 8 independent chains each)."""
    import torch

    from hierarchical_top_sparse_amd import _abi
    nbytes = 2 ** 31
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    copy = lambda: _abi.llsa_calib_copy(src, dst)   # noqa: E731
    copy()
    copy_ms = _event_ms(copy, reps)
    blocks, iters = 4096, 512
    out = torch.empty(blocks * 256, device="cuda")
    mfma = lambda: _abi.llsa_calib_mfma(out, blocks, iters)   # noqa: E731
    mfma()
    mfma_ms = _event_ms(mfma, reps)
    flops = blocks * 4 * iters * 8 * 2 * 16 * 16 * 32
    del src, dst, out
    return {"copy_bytes": nbytes, "copy_ms": round(copy_ms, 4),
            "copy_GBps": round(2 * nbytes / (copy_ms / 1e3) / 1e9, 1),
            "mfma_bf16_TFLOPs": round(flops / (mfma_ms / 1e3) / 1e12, 1)}


def kernel_fractions(p, per_kernel_ms):
    model = kernel_model(p)
    bf16 = p.torch_dtype == torch_bf16()
    peak_tf = BF16_MFMA_PEAK_TFLOPS if bf16 else FP32_MFMA_PEAK_TFLOPS
    out = {}
    for kname in model:
        if kname in per_kernel_ms:
            t = per_kernel_ms[kname] / 1e3
            out[kname] = {"ms": round(per_kernel_ms[kname], 4),
                          "hbm_frac": round(model[kname]["bytes"] / t / 1e9 / HBM_PEAK_GBS, 4),
                          "mfma_frac": round(model[kname]["flops"] / t / 1e12 / peak_tf, 4)}
    return out


def make_step(cfg_name, layout="raster", backward=None, levels=None, topk=8, x=None,
              head_dim=64):
    """A runtime Step over the workload's inputs (x: the generator's CPU tensors, made here if
    not given); levels/topk override its L and K, head_dim its channels per head."""
    import torch

    from hierarchical_top_sparse_amd import gen, ops
    from hierarchical_top_sparse_amd.runtime import Step
    cfg = gen.CONFIGS[cfg_name]
    h, w = cfg["height"], cfg["width"]
    L = levels or cfg["levels"]
    bwd = cfg["backward"] if backward is None else backward
    if x is None:
        x = gen.make_inputs(cfg["batch"], cfg["heads"], h, w, head_dim, cfg["dtype"],
                            cfg["seed_base"], with_grad=bwd)
    dev = torch.device("cuda:0")
    q, k, v = (x[t].to(dev) for t in ("q", "k", "v"))
    do = x["do"].to(dev) if bwd else None
    p = ops.make_problem(q, h, w, L, topk)
    if layout == "morton":
        q, k, v = (ops.reorder(p, t) for t in (q, k, v))
        do = ops.reorder(p, do) if do is not None else None
        p = ops.make_problem(q, h, w, L, topk, layout=ops.LLSA_LAYOUT_MORTON)
    return Step(p, q, k, v, do), x, cfg


def config_table(steps, warmup):
    """tokens/s and attention-kernel roofline fractions of every workload."""
    from hierarchical_top_sparse_amd import gen
    rows = {}
    for name, cfg in gen.CONFIGS.items():
        step, _, _ = make_step(name)
        ms, _, _, per_kernel_ms, _ = measure(step, steps, warmup)
        tokens = cfg["batch"] * cfg["height"] * cfg["width"]
        rows[name] = {"pass": "fwd+bwd" if cfg["backward"] else "fwd",
                      "dtype": "bf16" if cfg["dtype"] == torch_bf16() else "f32",
                      "tokens": tokens, "ms": round(ms, 4),
                      "tokens_per_s": round(tokens / (ms / 1e3), 1),
                      "kernels": kernel_fractions(step.p, per_kernel_ms)}
        del step
    return rows


def dense_baseline(llsa_fwd_ms_256, llsa_train_ms_256):
    """The library's dense flash attention at 256x256: forward at batch 1 x 6 heads, forward +
    backward at batch 2 x 6 heads; ratios against the sparse path at the same shapes."""
    import torch

    from hierarchical_top_sparse_amd import _abi
    out = {}
    n = 256 * 256
    for name, bh, bwd in (("px256_fwd", 6, False), ("px256_train", 12, True)):
        g = torch.Generator(device="cuda").manual_seed(5)
        q, k, v, do = (torch.randn(bh, n, 64, device="cuda", generator=g).to(torch.bfloat16)
                       for _ in range(4))
        o = torch.empty_like(q)
        lse = torch.empty(bh, n, device="cuda")
        dd = torch.empty_like(lse)
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))

        def fwd():
            _abi.llsa_dense_attn_fwd(q, k, v, o, lse)

        def step():
            fwd()
            _abi.llsa_dense_attn_bwd(q, k, v, do, lse, dq, dk, dv, dd)
        fn = step if bwd else fwd
        fn()
        ms = _event_ms(fn, 2)
        flops = 4 * bh * n * n * 64 * (3.5 if bwd else 1.0)
        sparse_ms = llsa_train_ms_256 if bwd else llsa_fwd_ms_256
        out[name] = {"pass": "fwd+bwd" if bwd else "fwd", "batch_heads": bh, "ms": round(ms, 3),
                     "tflops": round(flops / (ms / 1e3) / 1e12, 1),
                     "mfma_frac": round(flops / (ms / 1e3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                     "llsa_ms": round(sparse_ms, 4),
                     "speedup_llsa_vs_dense": round(ms / sparse_ms, 2)}
        del q, k, v, do, o, lse, dd, dq, dk, dv
    return out


def single_level(cfg_name, llsa_ms, steps):
    """The single-level comparator on the same inputs: one level, top-32 key blocks per query
    block chosen over all N/16 blocks (the quadratic selection of single-level block-sparse
    attention), then the same sparse forward and backward."""
    step, _, cfg = make_step(cfg_name, levels=1, topk=32)
    ms, _, _, per_kernel_ms, per_step_kernel_ms = measure(step, steps, 2)
    tokens = cfg["batch"] * cfg["height"] * cfg["width"]
    out = {"levels": 1, "topk": 32, "ms": round(ms, 4),
           "tokens_per_s": round(tokens / (ms / 1e3), 1),
           "per_kernel_ms_per_step": {k2: round(v2, 4) for k2, v2 in
                                      sorted(per_step_kernel_ms.items(), key=lambda kv: -kv[1])},
           "llsa_ms": round(llsa_ms, 4), "speedup_llsa_vs_single_level": round(ms / llsa_ms, 2)}
    del step
    return out


def mask_comparator(q, k, v, do, height, width, reps):
    """Single level, K = 32: the CSC backward (index transpose + backward) against the
    mask-based one (dense block mask + backward whose key-major pass scans it) on the same
    forward state; per-kernel times from the library's event hook."""
    import torch

    from hierarchical_top_sparse_amd import _abi, ops
    p = ops.make_problem(q, height, width, 1, 32)
    fwd = ops.llsa_forward(p, q, k, v)
    nmat, n1 = p.batch * p.heads, p.n_level(1)
    tws = torch.empty(_abi.llsa_index_transpose_workspace(nmat, n1, n1, 32), device=q.device,
                      dtype=torch.uint8)
    off = torch.empty((p.batch, p.heads, n1 + 1), device=q.device, dtype=torch.int32)
    rows = torch.empty((p.batch, p.heads, n1 * 32), device=q.device, dtype=torch.int32)
    mask = torch.empty((p.batch, p.heads, n1, n1), device=q.device, dtype=torch.uint8)
    bws = torch.empty(max(16, _abi.llsa_workspace_bytes(p)[1]), device=q.device,
                      dtype=torch.uint8)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    sel = fwd["sel"]

    def csc():
        _abi.llsa_index_transpose(nmat, n1, n1, 32, sel[0], off, rows, tws)
        _abi.llsa_attn_bwd(p, q, k, v, do, fwd["lse"], fwd["k_lv"], fwd["v_lv"], sel, [off],
                           [rows], dq, dk, dv, bws)

    def masked():
        _abi.llsa_block_mask(p, sel[0], mask)
        _abi.llsa_attn_bwd_masked(p, q, k, v, do, fwd["lse"], sel[0], mask, dq, dk, dv, bws)
    out = {}
    pairs = int(sel[0].numel())
    for name, fn in (("csc", csc), ("mask", masked)):
        fn()
        ms = _event_ms(fn, reps)
        _abi.llsa_profile_read()
        _abi.llsa_profile_enable(True)
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        _abi.llsa_profile_enable(False)
        kp = {kn: tot / reps for kn, (cnt, tot) in _abi.llsa_profile_read().items()}
        key_ms = kp.get("bwd_key_mask_kernel" if name == "mask" else "bwd_key_kernel")
        out[name] = {"bwd_ms": round(ms, 4),
                     "kernels_ms": {kn: round(t, 4) for kn, t in sorted(kp.items())},
                     "key_pass_block_pairs_per_s": round(pairs / (key_ms / 1e3), 1)}
    out["speedup_csc_vs_mask"] = round(out["mask"]["bwd_ms"] / out["csc"]["bwd_ms"], 2)
    del mask, fwd
    return out


def dit_bench(steps, warmup, side=256, batch=2, depth=12):
    """Synthetic Pixel-DiT-S training step (hidden 384, 6 heads, patch 1x1, depth 12; random
    weights and data) with LLSA (B = 16, K = 8, L = 3, Morton order hoisted to the network's
    entry) and with the library's dense attention: images/s and the speed-up (the pages'
    Table 2 analogue: DiT training throughput with LLSA against full attention)."""
    import torch

    from hierarchical_top_sparse_amd import dit
    out = {"model": f"Pixel DiT-S depth {depth}, hidden 384, 6 heads, patch 1x1",
           "pixels": f"{side}x{side}", "batch": batch, "dtype": "bf16 autocast, fp32 master",
           "optimizer": "AdamW", "data": "synthetic"}
    levels = 3 if side >= 256 else 2
    for mode in ("llsa", "dense"):
        torch.manual_seed(0)
        model = dit.PixelDiT(side, side, depth=depth, mode=mode, levels=levels).cuda()
        opt = torch.optim.AdamW(model.parameters(), lr=1e-4)
        data = dit.synthetic_batch(batch, side, side, "cuda", seed=1)
        n = steps if mode == "llsa" else max(2, steps // 4)
        for _ in range(warmup if mode == "llsa" else 1):
            dit.train_step(model, opt, data)
        ms = _event_ms(lambda: dit.train_step(model, opt, data), n)
        out[mode] = {"ms_per_step": round(ms, 3), "images_per_s": round(batch / (ms / 1e3), 2),
                     "steps": n}
        del model, opt, data
        torch.cuda.empty_cache()
    out["speedup_llsa_vs_dense"] = round(out["dense"]["ms_per_step"] /
                                         out["llsa"]["ms_per_step"], 2)
    return out


def sweep(steps):
    """Resolution sweep (the shape of the pages' Figure 3 / Figure 4): per side length, LLSA
    forward and forward + backward against the dense baseline with blocks of 16 and of 64
    tokens, the single-level top-32 comparator, the CSC against the dense-mask key-major pass,
    and the key-major kernel's throughput (query-key block pairs per second) as N grows."""
    import torch

    from hierarchical_top_sparse_amd import _abi, gen, ops
    from hierarchical_top_sparse_amd.runtime import Step
    for side, levels in ((64, 2), (128, 2), (256, 3), (512, 3)):
        n = side * side
        x = gen.make_inputs(1, 6, side, side, 64, torch.bfloat16, 7000 + side, with_grad=True)
        q, k, v, do = (x[t].cuda() for t in ("q", "k", "v", "do"))
        p = ops.make_problem(q, side, side, levels)
        fwd_ms = measure(Step(p, q, k, v), steps, 2)[0]
        st = Step(p, q, k, v, do)
        train_ms, _, _, per_kernel_ms, _ = measure(st, steps, 2)
        pairs = int(st.sel[0].numel())   # (query block, picked key block) pairs
        # the selection alone (its launches, on the step's pooled levels): inside the step
        # the selection launches also carry V's pooling
        sel_alone = lambda s_=st: _abi.llsa_select(s_.p, s_.q_lv, s_.k_lv, s_.sel)  # noqa: E731
        sel_alone()
        llsa_select_ms = _event_ms(sel_alone, max(steps, 5))
        qd, kd, vd, dod = (t.reshape(6, n, 64) for t in (q, k, v, do))
        o = torch.empty_like(qd)
        lse = torch.empty(6, n, device="cuda")
        dd = torch.empty_like(lse)
        dq, dk, dv = (torch.empty_like(qd) for _ in range(3))
        dfwd = lambda: _abi.llsa_dense_attn_fwd(qd, kd, vd, o, lse)   # noqa: E731

        def dstep():
            dfwd()
            _abi.llsa_dense_attn_bwd(qd, kd, vd, dod, lse, dq, dk, dv, dd)
        dfwd()
        dense_fwd_ms = _event_ms(dfwd, 2)
        dstep()
        dense_train_ms = _event_ms(dstep, 2)
        key_ms = per_kernel_ms.get("bwd_key_kernel")
        # block 64 (8x8 tiles), K = 8: one level below 256x256 (N / 64^2 < 8), two above
        l64 = 1 if side < 256 else 2
        p64 = ops.make_problem(q, side, side, l64, 8, block=64)
        b64_fwd_ms = measure(Step(p64, q, k, v), steps, 2)[0]
        b64_train_ms = measure(Step(p64, q, k, v, do), steps, 2)[0]
        p1 = ops.make_problem(q, side, side, 1, 32)
        s1 = Step(p1, q, k, v, do)
        single_ms = measure(s1, steps, 2)[0]
        sel1_alone = lambda s_=s1: _abi.llsa_select(s_.p, s_.q_lv, s_.k_lv, s_.sel)  # noqa: E731
        sel1_alone()
        single_select_ms = _event_ms(sel1_alone, max(steps, 5))
        del s1
        mc = mask_comparator(q, k, v, do, side, side, steps)
        print(json.dumps({
            "side": side, "tokens": n, "batch": 1, "heads": 6, "levels": levels,
            "llsa_fwd_ms": round(fwd_ms, 4), "llsa_train_ms": round(train_ms, 4),
            "dense_fwd_ms": round(dense_fwd_ms, 3), "dense_train_ms": round(dense_train_ms, 3),
            "speedup_fwd": round(dense_fwd_ms / fwd_ms, 2),
            "speedup_train": round(dense_train_ms / train_ms, 2),
            "b64_levels": l64, "b64_fwd_ms": round(b64_fwd_ms, 4),
            "b64_train_ms": round(b64_train_ms, 4),
            "b64_speedup_fwd": round(dense_fwd_ms / b64_fwd_ms, 2),
            "b64_speedup_train": round(dense_train_ms / b64_train_ms, 2),
            "single_level_top32_train_ms": round(single_ms, 4),
            "single_level_select_ms": round(single_select_ms, 4),
            "llsa_select_ms": round(llsa_select_ms, 4),
            "speedup_vs_single_level": round(single_ms / train_ms, 2),
            "single_level_bwd_csc_ms": mc["csc"]["bwd_ms"],
            "single_level_bwd_mask_ms": mc["mask"]["bwd_ms"],
            "key_pass_csc_block_pairs_per_s": mc["csc"]["key_pass_block_pairs_per_s"],
            "key_pass_mask_block_pairs_per_s": mc["mask"]["key_pass_block_pairs_per_s"],
            "llsa_train_tokens_per_s": round(6 * n / (train_ms / 1e3), 1),
            "key_pass_ms": round(key_ms, 4) if key_ms else None,
            "key_pass_block_pairs_per_s": round(pairs / (key_ms / 1e3), 1) if key_ms else None,
        }), flush=True)
        del st, q, k, v, do, qd, kd, vd, dod, o, lse, dd, dq, dk, dv


def main():
    args = parse()
    if args.sweep:
        sweep(max(3, args.steps // 2))
        return
    if args.dit:
        print(json.dumps({"dit_training_step": dit_bench(max(3, args.steps // 2),
                                                         min(args.warmup, 3))}))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "llsa runs on one GPU: multi-GPU runs are not implemented "
                                   "(the op shards over (batch, head) with no exchange)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    from hierarchical_top_sparse_amd import gen
    cfg = gen.CONFIGS[args.config]
    h, w, L = cfg["height"], cfg["width"], cfg["levels"]
    x = gen.make_inputs(cfg["batch"], cfg["heads"], h, w, 64, cfg["dtype"], cfg["seed_base"],
                        with_grad=cfg["backward"])
    # the CPU leg first: its worker processes are forked before anything touches the GPU
    cpu = None if args.no_cpu else cpu_baseline(cfg, x)

    from hierarchical_top_sparse_amd import _abi

    step, x, cfg = make_step(args.config, args.layout, x=x)
    p = step.p
    copy = None
    if args.with_copy:
        copy_dst = torch.empty_like(step.q)
        copy = lambda: _abi.llsa_reorder(p, step.q, copy_dst, False)   # noqa: E731
    ms_step, eager_ms, per_call, per_kernel_ms, per_step_kernel_ms = measure(
        step, args.steps, args.warmup, graph=not args.no_graph, with_copy=copy)
    tokens = cfg["batch"] * h * w
    value = tokens / (ms_step / 1e3)

    # ---- rows of the hot path as units (algorithmic bytes per step / their kernels' time
    # per step); the roofline object is for the unit with the largest time
    units, side = unit_model(p)
    traffic = traffic_record(args.config)
    launches = {kn: per_step_kernel_ms[kn] / per_kernel_ms[kn] for kn in per_kernel_ms}
    unit_rows = {}
    for uname, u in units.items():
        ms = sum(per_step_kernel_ms.get(kn, 0.0) for kn in u["kernels"])
        if ms <= 0:
            continue
        ran = [kn for kn in u["kernels"] if kn in per_step_kernel_ms]
        measured = (sum(traffic[kn]["hbm_bytes_per_launch"] * launches[kn] for kn in ran)
                    if all(kn in traffic for kn in ran) else None)
        unit_rows[uname] = {
            "kernels": ran, "ms_per_step": round(ms, 4), "alg_bytes": u["bytes"],
            "achieved_GBps": round(u["bytes"] / (ms / 1e3) / 1e9, 1),
            "hbm_frac": round(u["bytes"] / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_frac": round(u["flops"] / (ms / 1e3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
            "traffic": measured}
    side_rows = {}
    for kn, nbytes in side.items():
        if kn in per_step_kernel_ms:
            ms = per_step_kernel_ms[kn]
            side_rows[kn] = {"ms_per_step": round(ms, 4), "alg_bytes": nbytes,
                             "hbm_frac": round(nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                             "traffic": (traffic[kn]["hbm_bytes_per_launch"] * launches[kn]
                                         if kn in traffic else None)}
    dominant = max(unit_rows, key=lambda u: unit_rows[u]["ms_per_step"])
    dom = unit_rows[dominant]
    launch_ms = dom["ms_per_step"]
    achieved = dom["achieved_GBps"]
    roofline = {"bound": "hbm",
                "kernel": f"{dominant} ({' + '.join(dom['kernels'])})",
                "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": dom["traffic"],
                "alg_bytes_per_launch": dom["alg_bytes"], "launch_ms": launch_ms,
                "mfma_frac": dom["mfma_frac"]}
    calib = calibration()
    roofline["achievable_peak"] = calib["copy_GBps"]
    roofline["frac_of_achievable"] = round(achieved / calib["copy_GBps"], 4)
    extra = {"graph": not args.no_graph, "eager_ms_per_step": round(eager_ms, 4),
             "calibration": calib,
             "per_call_ms": {k2: round(v2, 4) for k2, v2 in per_call.items()},
             "per_kernel_ms_per_step": {k2: round(v2, 4) for k2, v2 in
                                        sorted(per_step_kernel_ms.items(),
                                               key=lambda kv: -kv[1])},
             "units": unit_rows, "side_kernels": side_rows,
             "attention_kernels": kernel_fractions(p, per_kernel_ms)}
    if not args.no_configs:   # (kept out of the headline-only runs the profiles are taken on)
        extra["prologue"] = prologue_parts(step)
    del step
    if not args.no_configs:
        extra["configs"] = config_table(max(5, args.steps // 2), 2)
        # the core figure without the reorder: the same step on tokens already in Morton order
        # (a network hoists the reorder to its entry); in raster order the reorder is folded
        # into every kernel's addressing, so there is no separate reorder launch to leave out
        other = "morton" if args.layout == "raster" else "raster"
        s_o, _, _ = make_step(args.config, other)
        ms_o = measure(s_o, max(10, args.steps // 2), 5)[0]
        del s_o
        extra[f"{other}_layout"] = {"ms_per_step": round(ms_o, 4),
                                    "tokens_per_s": round(tokens / (ms_o / 1e3), 1)}
    if not args.no_configs:
        # the same training step with 128-channel heads (the enrichment-ablation variants of
        # the method crossed with the head width): step time and its units' fractions
        s128, _, _ = make_step(args.config, head_dim=128)
        ms128, _, _, pk128, pks128 = measure(s128, max(10, args.steps // 2), 5)
        u128, _ = unit_model(s128.p)
        rows128 = {}
        for un, u in u128.items():
            ms_u = sum(pks128.get(kn, 0.0) for kn in u["kernels"])
            if ms_u > 0:
                rows128[un] = {"ms_per_step": round(ms_u, 4), "alg_bytes": u["bytes"],
                               "hbm_frac": round(u["bytes"] / (ms_u / 1e3) / 1e9 / HBM_PEAK_GBS,
                                                 4)}
        extra["head_dim_128"] = {"ms_per_step": round(ms128, 4),
                                 "tokens_per_s": round(tokens / (ms128 / 1e3), 1),
                                 "units": rows128}
        del s128
    if not args.no_dense:
        if "configs" in extra:
            fwd256 = extra["configs"]["px256"]["ms"]
        else:
            s256, _, _ = make_step("px256")
            fwd256 = measure(s256, 10, 2)[0]
            del s256
        extra["dense_baseline"] = dense_baseline(fwd256, ms_step)
        extra["single_level_top32"] = single_level(args.config, ms_step, max(5, args.steps // 2))
        qd, kd, vd, dod = (x[t].to("cuda") for t in ("q", "k", "v", "do"))
        extra["mask_backward_comparator"] = mask_comparator(qd, kd, vd, dod, h, w,
                                                            max(5, args.steps // 2))
        del qd, kd, vd, dod
    line = {
        "metric": "LLSA fwd+bwd tokens/s at 256x256 pixels (65,536 tok); % MFMA/HBM peak",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.config}: {h}x{w} pixel tokens, batch {cfg['batch']}, "
                               f"{cfg['heads']} heads, head_dim 64, B=16, K=8, L={L}, fwd+bwd, "
                               f"{args.layout} token order",
                   "global_batch": cfg["batch"], "seq_len": h * w, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
