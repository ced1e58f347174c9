"""Summaries of rocprofv3 output for the library's kernels (a measurement aid, not part of the
method): the per-kernel time table of a `--kernel-trace --stats` run, and the HBM traffic per
launch of every kernel from two `--pmc` runs (FETCH_SIZE, then WRITE_SIZE).

Counters are scaled by what they read for a plain copy of known size in the same run: the
benchmark's `--with-copy` launches one Morton reorder of a token tensor (T bytes read, T bytes
written) per step, so fetched bytes = FETCH_SIZE * (T / FETCH_SIZE of the copy) and likewise
for writes.

  python -m hierarchical_top_sparse_amd.profiling stats <run>_kernel_stats.csv --title ...
         --command ...                                   (markdown table on stdout)
  python -m hierarchical_top_sparse_amd.profiling traffic --fetch <fetch>_counter_collection.csv
         --write <write>_counter_collection.csv --copy-bytes T --workload px256_train
         --command ... --command ... > profiles/<workload>_traffic.json
  python -m hierarchical_top_sparse_amd.profiling timeline <run>_kernel_trace.csv --steps 3
         --title ... --command ...                       (markdown: the last steps' launches)
  python -m hierarchical_top_sparse_amd.profiling sweep <bench --sweep output> --command ...
                                                         (markdown: the resolution sweep tables)
  python -m hierarchical_top_sparse_amd.profiling sq <pass1>_counter_collection.csv
         <pass2>_counter_collection.csv --kernel ... --title ... --command ... --command ...
                                                         (markdown: SQ counters per kernel)
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = "hierarchical_top_sparse_amd/csrc"

# device symbol (without namespace and template arguments) -> the name the library's event
# profiler gives its launches, and the file the kernel is compiled from
_KERNELS = {
    "pool12_bf16_kernel": ("pool12_kernel", "pool.hip"),
    "pool12_f32_kernel": ("pool12_kernel", "pool.hip"),
    "pool_next_kernel": ("pool_next_kernel", "pool.hip"),
    "pool_next_v_kernel": ("pool_next_kernel", "select.hip"),
    "select_kernel": ("select_kernel", "select.hip"),
    "select_pool12_kernel": ("select_pool_kernel", "select.hip"),
    "select_pool_next_kernel": ("select_pool_kernel", "select.hip"),
    "expand_kernel": ("expand_kernel", "select.hip"),
    "attn_fwd_kernel": ("attn_fwd_kernel", "attn_fwd.hip"),
    "csc_radix_kernel": ("csc_radix_kernel", "transpose.hip"),
    "csc_assemble_kernel": ("csc_assemble_kernel", "transpose.hip"),
    "tile_sort_kernel": ("tile_sort_kernel", "transpose.hip"),
    "merge_kernel": ("merge_kernel", "transpose.hip"),
    "csc_bounds_kernel": ("csc_bounds_kernel", "transpose.hip"),
    "csc_offsets_kernel": ("csc_offsets_kernel", "transpose.hip"),
    "csc_scatter_kernel": ("csc_scatter_kernel", "transpose.hip"),
    "bwd_query_kernel": ("bwd_query_kernel", "attn_bwd.hip"),
    "coarse_grad_kernel": ("coarse_grad_kernel", "attn_bwd.hip"),
    "reorder_kernel": ("reorder_kernel", "reorder.hip"),
    "copy_kernel": ("copy_kernel", "calib.hip"),
    "mfma_kernel": ("mfma_kernel", "calib.hip"),
}
# bwd_key_kernel<MODE>: 0 = the CSC pass, 1 = the mask-scanning comparator, 2 = overflow chunks
_KEY_MODES = {"0": "bwd_key_kernel", "1": "bwd_key_mask_kernel", "2": "bwd_key_overflow_kernel"}


def profile_name(symbol: str):
    """(profiler name, source file) of a demangled kernel symbol, or None if not ours."""
    m = re.match(r"\s*(?:void\s+)?(?:llsa::)?(\w+)(?:<([^>]*)>)?", symbol)
    if not m:
        return None
    base, targs = m.group(1), m.group(2)
    if base == "bwd_key_kernel":
        mode = (targs or "").split(",")[0].strip()   # <MODE, head_dim>
        return _KEY_MODES.get(mode, "bwd_key_kernel"), "attn_bwd.hip"
    return _KERNELS.get(base)


def _col(row: dict, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError(f"none of {names} in {sorted(row)}")


def kernel_stats_table(path: str) -> list:
    """Rows (symbol, calls, avg_us, min_us, max_us, percent) of a rocprofv3 kernel_stats.csv."""
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append((_col(r, "Name", "KERNEL_NAME"), int(_col(r, "Calls")),
                         float(_col(r, "AverageNs")) / 1e3, float(_col(r, "MinNs")) / 1e3,
                         float(_col(r, "MaxNs")) / 1e3, float(_col(r, "Percentage"))))
    rows.sort(key=lambda t: -t[5])
    return rows


def counters_per_kernel(path: str, counter: str) -> dict:
    """Mean value of `counter` per dispatch of each profiler name (with its dispatch count)."""
    tot, cnt = defaultdict(float), defaultdict(int)
    with open(path) as f:
        for r in csv.DictReader(f):
            if _col(r, "Counter_Name") != counter:
                continue
            key = profile_name(_col(r, "Kernel_Name"))
            if key is None:
                continue
            tot[key[0]] += float(_col(r, "Counter_Value"))
            cnt[key[0]] += 1
    return {k: (tot[k] / cnt[k], cnt[k]) for k in tot}


def traffic_record(fetch_csv, write_csv, copy_bytes, workload, commands) -> dict:
    fetch = counters_per_kernel(fetch_csv, "FETCH_SIZE")
    write = counters_per_kernel(write_csv, "WRITE_SIZE")
    if "reorder_kernel" not in fetch or "reorder_kernel" not in write:
        raise SystemExit("no calibration copy (reorder_kernel) in the counter runs: run the "
                         "benchmark with --with-copy")
    kib = copy_bytes / 1024.0
    fscale = kib / fetch["reorder_kernel"][0]
    wscale = kib / write["reorder_kernel"][0]
    sources = {}   # a profiler name's first listed source (pool_next_kernel: pool.hip)
    for name, src in list(_KERNELS.values()) + [(v, "attn_bwd.hip")
                                                for v in _KEY_MODES.values()]:
        sources.setdefault(name, src)
    kernels = {}
    for name in sorted(set(fetch) & set(write)):
        if name == "reorder_kernel":
            continue
        src = f"{CSRC}/{sources[name]}"
        rd = fetch[name][0] * fscale * 1024.0
        wr = write[name][0] * wscale * 1024.0
        kernels[name] = {
            "source": src,
            "source_sha256": hashlib.sha256(open(os.path.join(ROOT, src), "rb").read())
            .hexdigest(),
            "dispatches": fetch[name][1],
            "fetch_size_kib_per_dispatch": round(fetch[name][0], 1),
            "write_size_kib_per_dispatch": round(write[name][0], 1),
            "hbm_read_bytes_per_launch": int(rd), "hbm_write_bytes_per_launch": int(wr),
            "hbm_bytes_per_launch": int(rd + wr)}
    return {"workload": workload,
            "calibration": f"reorder_kernel, a plain copy of {copy_bytes} bytes: FETCH_SIZE "
                           f"{fetch['reorder_kernel'][0]:.1f} KiB, WRITE_SIZE "
                           f"{write['reorder_kernel'][0]:.1f} KiB per dispatch",
            "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4),
            "commands": commands, "kernels": kernels}


def step_timelines(path: str, first: str = "pool12_kernel", last_steps: int = 3) -> list:
    """The last `last_steps` complete steps of a rocprofv3 kernel_trace.csv, a step starting at
    each launch of `first`: per step, rows (name, queue, start_us, end_us) relative to the
    step's first launch, for the library's own kernels other than the calibration ones."""
    ev = []
    with open(path) as f:
        for r in csv.DictReader(f):
            key = profile_name(_col(r, "Kernel_Name"))
            if key is None or key[0] in ("copy_kernel", "mfma_kernel", "reorder_kernel"):
                continue
            ev.append((int(_col(r, "Start_Timestamp")), int(_col(r, "End_Timestamp")), key[0],
                       int(_col(r, "Queue_Id"))))
    ev.sort()
    starts = [i for i, e in enumerate(ev) if e[2] == first]
    steps = []
    for a, b in zip(starts, starts[1:] + [len(ev)]):
        t0 = ev[a][0]
        steps.append([(name, q, (s - t0) / 1e3, (e - t0) / 1e3) for s, e, name, q in ev[a:b]])
    # the last step may be cut short by the end of the run: keep steps as long as the median
    full = [st for st in steps if len(st) == max(len(x) for x in steps)]
    return full[-last_steps:]


# MI355X: GRBM_GUI_ACTIVE is reported summed over the 8 XCDs; 1024 SIMDs in 256 CUs
_XCDS, _SIMDS, _CUS = 8, 1024, 256


def sq_rows(csvs, kernels) -> list:
    """Per kernel (profiler name): the SQ counters of the given passes averaged over its
    dispatches, and what they derive to (MFMA busy, bf16 MFMA FLOP, per-wave instruction
    counts, LDS activity and the share of it spent in bank conflicts)."""
    vals = defaultdict(lambda: defaultdict(list))
    for path in csvs:
        with open(path) as f:
            for r in csv.DictReader(f):
                key = profile_name(_col(r, "Kernel_Name"))
                if key is not None:
                    vals[key[0]][_col(r, "Counter_Name")].append(float(_col(r, "Counter_Value")))
    rows = []
    for kn in kernels:
        c = {name: sum(v) / len(v) for name, v in vals[kn].items()}
        gui = c["GRBM_GUI_ACTIVE"] / _XCDS
        waves = c["SQ_WAVES"]
        rows.append({
            "kernel": kn, "gui_cycles": gui,
            "mfma_busy": c["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * _SIMDS),
            "mfma_gflop": c["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / 1e9,
            "mfma_per_wave": c["SQ_INSTS_MFMA"] / waves,
            "valu_per_wave": c["SQ_INSTS_VALU"] / waves,
            "lds_per_wave": c["SQ_INSTS_LDS"] / waves,
            "lds_active": c["SQ_LDS_IDX_ACTIVE"] / (gui * _CUS),
            "bank_conflict_share": (c["SQ_LDS_BANK_CONFLICT"] / c["SQ_LDS_IDX_ACTIVE"]
                                    if c["SQ_LDS_IDX_ACTIVE"] else 0.0)})
    return rows


def sweep_tables(path: str) -> str:
    """The three tables of the resolution sweep (`bench.py --sweep`, one JSON line per side):
    LLSA (B = 16 and 64) against dense attention, LLSA against the single-level top-32
    comparator, and the CSC against the dense-mask key-major pass."""
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{") and '"side"' in line:
                rows.append(json.loads(line))
    g = lambda x: f"{x / 1e9:.2f} G"   # noqa: E731
    out = ["## LLSA against dense attention (the pages' Figure 3: B = 16 and 64)", "",
           "| side | tokens | dense fwd ms | B=16 fwd ms | B=16 fwd speed-up | B=64 fwd ms | "
           "B=64 fwd speed-up | dense fwd+bwd ms | B=16 fwd+bwd ms | B=16 speed-up | "
           "B=64 fwd+bwd ms | B=64 speed-up |",
           "|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        out.append(f"| {r['side']} | {r['tokens']} | {r['dense_fwd_ms']:.3f} | "
                   f"{r['llsa_fwd_ms']:.4f} | {r['speedup_fwd']:.1f}x | {r['b64_fwd_ms']:.4f} | "
                   f"{r['b64_speedup_fwd']:.1f}x | {r['dense_train_ms']:.3f} | "
                   f"{r['llsa_train_ms']:.4f} | {r['speedup_train']:.1f}x | "
                   f"{r['b64_train_ms']:.4f} | {r['b64_speedup_train']:.1f}x |")
    out += ["", "## Quadratic selection: LLSA against single-level top-32", "",
            "| side | LLSA select ms | single-level select ms | LLSA fwd+bwd ms | "
            "single-level fwd+bwd ms | LLSA speed-up |", "|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        out.append(f"| {r['side']} | {r['llsa_select_ms']:.4f} | "
                   f"{r['single_level_select_ms']:.4f} | {r['llsa_train_ms']:.4f} | "
                   f"{r['single_level_top32_train_ms']:.4f} | "
                   f"{r['speedup_vs_single_level']:.2f}x |")
    out += ["", "## KV backward: index transpose against a dense block mask (the pages' "
            "Figure 4)", "", "| side | CSC bwd ms | mask bwd ms | CSC key pass pairs/s | "
            "mask key pass pairs/s | LLSA (K=8) key pass pairs/s |",
            "|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        llsa = r.get("key_pass_block_pairs_per_s")
        out.append(f"| {r['side']} | {r['single_level_bwd_csc_ms']:.4f} | "
                   f"{r['single_level_bwd_mask_ms']:.4f} | "
                   f"{g(r['key_pass_csc_block_pairs_per_s'])} | "
                   f"{g(r['key_pass_mask_block_pairs_per_s'])} | "
                   f"{g(llsa) if llsa else '-'} |")
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    st = sub.add_parser("stats")
    st.add_argument("csv")
    st.add_argument("--title", required=True)
    st.add_argument("--command", required=True)
    tr = sub.add_parser("traffic")
    tr.add_argument("--fetch", required=True)
    tr.add_argument("--write", required=True)
    tr.add_argument("--copy-bytes", type=int, required=True)
    tr.add_argument("--workload", required=True)
    tr.add_argument("--command", action="append", default=[])
    tl = sub.add_parser("timeline")
    tl.add_argument("csv")
    tl.add_argument("--steps", type=int, default=3)
    tl.add_argument("--title", required=True)
    tl.add_argument("--command", required=True)
    sw = sub.add_parser("sweep")
    sw.add_argument("jsonl")
    sw.add_argument("--command", required=True)
    sq = sub.add_parser("sq")
    sq.add_argument("csv", nargs="+")
    sq.add_argument("--kernel", action="append", required=True)
    sq.add_argument("--title", required=True)
    sq.add_argument("--command", action="append", required=True)
    a = ap.parse_args(argv)
    if a.what == "stats":
        print(f"# {a.title}\n\nCommand (MI355X host, repo root; `TMPDIR=/tmp`):\n\n```\n{a.command}\n"
              f"```\n\n| kernel | calls | avg µs | min µs | max µs | % of GPU time |\n"
              f"|---|---:|---:|---:|---:|---:|")
        for sym, calls, avg, mn, mx, pct in kernel_stats_table(a.csv):
            print(f"| `{sym}` | {calls} | {avg:.2f} | {mn:.2f} | {mx:.2f} | {pct:.2f} |")
    elif a.what == "sweep":
        print(f"Command (MI355X host, repo root):\n\n```\n{a.command}\n```\n")
        print(sweep_tables(a.jsonl))
    elif a.what == "sq":
        cmds = "\n".join(a.command)
        print(f"# {a.title}\n\nCommands (MI355X host, repo root; `TMPDIR=/tmp`), one counter pass "
              f"each:\n\n```\n{cmds}\n```\n\nPer launch, averaged over the launches of each "
              f"kernel in the run.  GRBM_GUI_ACTIVE comes summed over the {_XCDS} XCDs, so GUI "
              f"cycles are that value / {_XCDS}.  MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GUI "
              f"cycles x {_SIMDS} SIMDs); MFMA GFLOP = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; LDS "
              f"active = SQ_LDS_IDX_ACTIVE / (GUI cycles x {_CUS} CUs); bank-conflict share = "
              f"SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE.  Per-wave counts divide by SQ_WAVES.\n"
              f"\n| kernel | GUI cycles | MFMA busy | MFMA GFLOP | MFMA / wave | VALU / wave | "
              f"LDS / wave | LDS active | LDS cycles in bank conflicts |\n"
              f"|---|---:|---:|---:|---:|---:|---:|---:|---:|")
        for r in sq_rows(a.csv, a.kernel):
            print(f"| `{r['kernel']}` | {r['gui_cycles']:,.0f} | {100 * r['mfma_busy']:.1f} % | "
                  f"{r['mfma_gflop']:.1f} | {r['mfma_per_wave']:,.0f} | "
                  f"{r['valu_per_wave']:,.0f} | {r['lds_per_wave']:,.0f} | "
                  f"{100 * r['lds_active']:.1f} % | {100 * r['bank_conflict_share']:.1f} % |")
    elif a.what == "timeline":
        print(f"# {a.title}\n\nCommand (MI355X host, repo root; `TMPDIR=/tmp`):\n\n```\n{a.command}\n"
              f"```\n\nThe last {a.steps} steps of the run (graph replays), each launch's start "
              f"and end relative to the step's first launch; queues are the hardware queues "
              f"the runtime put the launches on.")
        for st in step_timelines(a.csv, last_steps=a.steps):
            main_q = st[0][1]
            side = [x for x in st if x[1] != main_q]
            fwd = [x for x in st if x[0] == "attn_fwd_kernel"]
            print(f"\nStep of {max(x[3] for x in st):.1f} µs"
                  + (f": the other queue's launches end at {max(x[3] for x in side):.1f} µs, "
                     f"the forward at {fwd[0][3]:.1f} µs" if side and fwd else "")
                  + "\n\n| launch | queue | start µs | end µs | µs |\n|---|---:|---:|---:|---:|")
            for name, q, t0, t1 in st:
                print(f"| `{name}` | {q} | {t0:.1f} | {t1:.1f} | {t1 - t0:.1f} |")
    else:
        json.dump(traffic_record(a.fetch, a.write, a.copy_bytes, a.workload, a.command),
                  sys.stdout, indent=1)
        print()


if __name__ == "__main__":
    main()
