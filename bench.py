"""LLSA fwd+bwd throughput on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic pixel tokens already
resident in HBM: (Morton reorder folded into the kernels' addressing) -> pooling -> coarse-to-
fine selection -> sparse attention forward -> CSR->CSC transpose of every level -> sparse
backward (dQ, dK, dV).  Prints one JSON line.

  python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config px256_train] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="px256_train")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--with-copy", action="store_true",
                    help="also launch one Morton reorder (a plain copy of one token tensor) per "
                         "step, outside the timed region: the calibration kernel for HBM "
                         "byte counters")
    return ap.parse_args()


class Pipeline:
    """Preallocated buffers and the sequence of C-ABI calls of one training step."""

    def __init__(self, p, q, k, v, do):
        import torch
        from hierarchical_top_sparse_amd import _abi

        self.abi, self.p = _abi, p
        self.q, self.k, self.v, self.do = q, k, v, do
        dev, f32 = q.device, torch.float32
        lv = lambda l: torch.empty((p.batch, p.heads, p.n_level(l), p.head_dim), device=dev,
                                   dtype=f32)
        L = p.levels
        self.q_lv = [lv(l) for l in range(1, L + 1)]
        self.k_lv = [lv(l) for l in range(1, L + 1)]
        self.v_lv = [None] + [lv(l) for l in range(2, L + 1)]
        self.sel = [torch.empty((p.batch, p.heads, p.n_level(l), p.topk), device=dev,
                                dtype=torch.int32) for l in range(1, L + 1)]
        self.o = torch.empty_like(q)
        self.lse = torch.empty((p.batch, p.heads, p.n), device=dev, dtype=f32)
        nmat = p.batch * p.heads
        self.off = [torch.empty((p.batch, p.heads, p.n_level(l) + 1), device=dev,
                                dtype=torch.int32) for l in range(1, L + 1)]
        self.rows = [torch.empty((p.batch, p.heads, p.n_level(l) * p.topk), device=dev,
                                 dtype=torch.int32) for l in range(1, L + 1)]
        tws = max(_abi.llsa_index_transpose_workspace(nmat, p.n_level(l), p.n_level(l), p.topk)
                  for l in range(1, L + 1))
        self.tws = torch.empty(tws, device=dev, dtype=torch.uint8)
        _, bws = _abi.llsa_workspace_bytes(p)
        self.bws = torch.empty(bws, device=dev, dtype=torch.uint8)
        self.dq, self.dk, self.dv = (torch.empty_like(q) for _ in range(3))
        self.nmat = nmat

    def calls(self):
        """(name, thunk) for every ABI call of a step, in order."""
        a, p = self.abi, self.p
        out = [("pool", lambda: a.llsa_pool(p, self.q, self.k, self.v, self.q_lv, self.k_lv,
                                            self.v_lv)),
               ("select", lambda: a.llsa_select(p, self.q_lv, self.k_lv, self.sel)),
               ("attn_fwd", lambda: a.llsa_attn_fwd(p, self.q, self.k, self.v, self.k_lv,
                                                    self.v_lv, self.sel, self.o, self.lse))]
        for l in range(1, p.levels + 1):
            nl = p.n_level(l)
            out.append((f"transpose_l{l}", (lambda l=l, nl=nl: a.llsa_index_transpose(
                self.nmat, nl, nl, p.topk, self.sel[l - 1], self.off[l - 1], self.rows[l - 1],
                self.tws))))
        out.append(("attn_bwd", lambda: a.llsa_attn_bwd(
            p, self.q, self.k, self.v, self.do, self.lse, self.k_lv, self.v_lv,
            self.sel, self.off, self.rows, self.dq, self.dk, self.dv, self.bws)))
        return out


def algorithmic(p, elem_bytes=2):
    """Algorithmic (compulsory) HBM bytes and FLOPs per launch of each attention kernel."""
    bh, n, d, K, L = p.batch * p.heads, p.n, p.head_dim, p.topk, p.levels
    T = bh * n * d * elem_bytes
    n1 = n // 16
    kq = K * 16 + (L - 1) * K           # keys per query
    coarse = sum(bh * (n // 16 ** l) * d * 4 * 2 for l in range(2, L + 1))   # pooled K, V fp32
    sel_bytes = sum(bh * (n // 16 ** l) * K * 4 for l in range(1, L + 1))
    fwd_bytes = 4 * T + bh * n * 4 + sel_bytes + coarse
    # read q, k, v, dO (the forward's O is not needed), write dq, dk, dv
    bwd_bytes = 7 * T + 2 * bh * n * 4 + 2 * sel_bytes + coarse + bh * (n1 + 1) * 4
    return dict(T=T, kq=kq, fwd_bytes=fwd_bytes, bwd_bytes=bwd_bytes,
                fwd_flops=4 * bh * n * kq * d, bwd_flops=10 * bh * n * kq * d)


def cpu_baseline(cfg, x, seconds_budget=12.0):
    """The oracle (as it stands), single-threaded, on whole (batch, head) slices of the same
    inputs, fwd + bwd, until the time budget is used; scaled to whole-workload tokens/s."""
    import torch
    from threadpoolctl import threadpool_limits

    from oracle import llsa_oracle as orc

    h, w, L = cfg["height"], cfg["width"], cfg["levels"]
    slices = [(b, hh) for b in range(cfg["batch"]) for hh in range(cfg["heads"])]
    done, spent = 0, 0.0
    with threadpool_limits(1):
        nthreads = torch.get_num_threads()
        torch.set_num_threads(1)
        for b, hh in slices:
            r = {t: x[t][b:b + 1, hh:hh + 1].double().numpy() for t in ("q", "k", "v", "do")}
            t0 = time.perf_counter()
            res = orc.llsa_forward(r["q"], r["k"], r["v"], h, w, 16, L, 8, True)
            orc.llsa_backward(r["q"], r["k"], r["v"], r["do"], h, w, 16, L, res["sel"], True)
            spent += time.perf_counter() - t0
            done += 1
            if spent >= seconds_budget:
                break
        torch.set_num_threads(nthreads)
    tokens = cfg["batch"] * h * w * done / len(slices)
    return dict(value=round(tokens / spent, 1), unit="tokens/s", cores=1, kind="oracle",
                sample=f"{done} of {len(slices)} (batch, head) slices of the workload, fwd+bwd "
                       f"in {spent:.1f} s on one thread; tokens counted pro rata")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; multi-GPU runs are not "
                                   "part of it (the op shards over (batch, head) with no "
                                   "exchange, see the design notes)", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    from hierarchical_top_sparse_amd import _abi, gen, ops

    cfg = gen.CONFIGS[args.config]
    h, w, L = cfg["height"], cfg["width"], cfg["levels"]
    x = gen.make_inputs(cfg["batch"], cfg["heads"], h, w, 64, cfg["dtype"], cfg["seed_base"],
                        with_grad=True)
    dev = torch.device("cuda:0")
    q, k, v, do = (x[t].to(dev) for t in ("q", "k", "v", "do"))
    p = ops.make_problem(q, h, w, L)
    pipe = Pipeline(p, q, k, v, do)
    calls = pipe.calls()
    stream = torch.cuda.current_stream()

    def step():
        for _, fn in calls:
            fn()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.with_copy:
        copy_dst = torch.empty_like(q)
        for _ in range(max(1, args.steps)):
            _abi.llsa_reorder(p, q, copy_dst, False)
        torch.cuda.synchronize()
    # timed region: events around every ABI call, on the stream the kernels run on
    ev = {name: [] for name, _ in calls}
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for _ in range(args.steps):
        for name, fn in calls:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            ev[name].append((e0, e1))
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    per_call = {name: sum(a.elapsed_time(b) for a, b in pairs) / len(pairs)
                for name, pairs in ev.items()}
    tokens = cfg["batch"] * h * w
    value = tokens / (ms_step / 1e3)

    alg = algorithmic(p)
    fwd_ms = per_call["attn_fwd"]
    achieved = alg["fwd_bytes"] / (fwd_ms / 1e3) / 1e9
    roofline = {"bound": "hbm", "kernel": "attn_fwd_kernel", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None, "alg_bytes_per_launch": alg["fwd_bytes"],
                "launch_ms": round(fwd_ms, 4),
                "mfma_tflops": round(alg["fwd_flops"] / (fwd_ms / 1e3) / 1e12, 2)}
    extra = {"per_call_ms": {k2: round(v2, 4) for k2, v2 in per_call.items()},
             "attn_bwd_alg_GBps": round(alg["bwd_bytes"] / (per_call["attn_bwd"] / 1e3) / 1e9, 1),
             "attn_bwd_mfma_tflops": round(alg["bwd_flops"] / (per_call["attn_bwd"] / 1e3) / 1e12,
                                           2)}
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, x)
    line = {
        "metric": "LLSA fwd+bwd tokens/s at 256x256 pixels (65,536 tok); % MFMA/HBM peak",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{args.config}: {h}x{w} pixel tokens, batch {cfg['batch']}, "
                               f"{cfg['heads']} heads, head_dim 64, B=16, K=8, L={L}, fwd+bwd",
                   "global_batch": cfg["batch"], "seq_len": h * w, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
