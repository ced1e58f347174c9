"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI, run the CPU
oracle on the same seeded inputs, and compare with the acceptance rules:

* reorder and index transpose: bit-exact;
* selections: identical sets, except in near-tie rows.  A row may differ from the oracle's
  only if every GPU pick scores (oracle fp64 scores) at least as high as every candidate the
  GPU left out, minus 1e-4 relative (the GPU scores in fp32): then the oracle's K-th and
  (K+1)-th scores are also within 1e-4 of each other.  Every level is checked
  teacher-forced on the GPU's parent picks;
* outputs and gradients: max-abs <= 2e-2 and mean-rel <= 5e-3 for bf16 inputs, both <= 1e-4
  for fp32 inputs (mean-rel = mean|x - ref| / mean|ref|), with the oracle attention run on
  the GPU's selection.  The max-abs bound applies to the kernel's arithmetic: a tensor stored
  in bf16 is the round-to-nearest-even image of the kernel's fp32 value, so an element passes
  iff some fp32 value that rounds to the stored bf16 number lies within the bound of the
  reference (the stored number's exact rounding interval, no more);
* the log-sum-exp is fp32 and gets no storage allowance: 1e-4 for fp32 inputs, and for bf16
  inputs the bound `lse_tolerance` derives from the arithmetic of the score.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

from oracle import llsa_oracle as orc

B = 16
GAP = 1e-4


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def tolerances(dtype: torch.dtype):
    return (2e-2, 5e-3) if dtype == torch.bfloat16 else (1e-4, 1e-4)


def _log(record: dict):
    path = os.environ.get("LLSA_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(record) + "\n")


def bf16_rounding_interval(x: np.ndarray):
    """(lo, hi): the reals that round to nearest even to the bf16 numbers x (float64 arrays
    holding bf16 values).  A finite bf16 number m > 0 takes the reals within half the gap to
    its neighbours: [m - (m - prev)/2, m + (next - m)/2]; the bounds are kept (ties may round
    either way, depending on the last bit); signs mirror, zero takes half the smallest
    subnormal on both sides."""
    x = np.asarray(x, dtype=np.float64)
    bits = (np.abs(x).astype(np.float32).view(np.uint32) >> 16).astype(np.int64)
    if not np.array_equal(np.abs(x).astype(np.float32).view(np.uint32) & 0xFFFF,
                          np.zeros(x.shape, np.uint32)):
        raise ValueError("values are not bf16 numbers")

    def val(b):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    mag = np.abs(x)
    up = val(bits + 1)
    down = np.where(bits > 0, val(np.maximum(bits - 1, 0)), -val(np.ones_like(bits)))
    above = (up - mag) / 2          # toward larger magnitude
    below = (mag - down) / 2        # toward zero (for zero: half the smallest subnormal)
    neg = x < 0
    lo = np.where(neg, x - above, x - below)
    hi = np.where(neg, x + below, x + above)
    return lo, hi


def assert_close(x, ref: np.ndarray, dtype: torch.dtype, name: str, tol_abs: float | None = None,
                 stored_bf16: bool | None = None):
    """x: the GPU tensor (or its float64 array); dtype: the input precision, which picks the
    tolerances; tol_abs overrides the max-abs bound (the LSE's).  stored_bf16 (default: x is a
    bf16 tensor, or an array of a bf16-input run) compares the stored number's rounding
    interval with the reference instead of the number itself."""
    tol_a, tol_rel = tolerances(dtype)
    if tol_abs is not None:
        tol_a = tol_abs
    if isinstance(x, torch.Tensor):
        if stored_bf16 is None:
            stored_bf16 = x.dtype == torch.bfloat16
        x = to64(x)
    elif stored_bf16 is None:
        stored_bf16 = dtype == torch.bfloat16
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, f"{name}: shape {x.shape} vs {ref.shape}"
    assert np.isfinite(x).all(), f"{name}: non-finite values"
    err = np.abs(x - ref)
    if stored_bf16:
        lo, hi = bf16_rounding_interval(x)
        dist = np.maximum(0.0, np.maximum(lo - ref, ref - hi))   # ref to the interval
    else:
        dist = err
    excess = float((dist - tol_a).max())
    max_abs = float(err.max())
    mean_rel = float(err.mean() / max(np.abs(ref).mean(), 1e-30))
    _log(dict(name=name, max_abs=max_abs, mean_rel=mean_rel, max_ref=float(np.abs(ref).max()),
              max_arith_err=float(dist.max()), worst_over_bound=excess))
    assert excess <= 0 and mean_rel <= tol_rel, (
        f"{name}: max-abs {max_abs:.3g}, arithmetic error at least {float(dist.max()):.3g} "
        f"(bound {tol_a:.3g}) mean-rel {mean_rel:.3g} (tol {tol_rel}); "
        f"max|ref| {np.abs(ref).max():.3g}")
    return max_abs, mean_rel


def lse_tolerance(q_ref: np.ndarray, k_ref: np.ndarray, dtype: torch.dtype, levels: int = 0,
                  head_dim: int = 64, block: int = 16) -> float:
    """Max-abs bound of the fp32 log-sum-exp (levels: the pooled levels whose keys enrich the
    attention come from, 0 without coarse keys).

    fp32 inputs: 1e-4 (the fp32 acceptance bound).  bf16 inputs: the LSE moves by at most the
    largest error of one of its scores (it is a smooth maximum of them).  A score
    scale * sum_c q_c k_c is computed from exact bf16 q and k (their products are exact in
    fp32) and accumulated in fp32 over head_dim products (error <= head_dim 2^-24
    sum_c |q_c k_c|).  A coarse key is an fp32 mean whose sums add at most B - 1 rounding
    errors per level (<= (B - 1) L 2^-24 of the largest |k|), entering the MFMA as bf16 hi + lo
    parts (relative error <= 2^-18 per element, taken as 2^-17).  So |error| <= scale ||q||_1
    max|k| (head_dim 2^-24 [+ 2^-17 + (B - 1) L 2^-24]), plus 1e-5 for the fp32 exponentials
    and logarithm."""
    if dtype != torch.bfloat16:
        return 1e-4
    scale = 1.0 / np.sqrt(head_dim)
    q1 = np.abs(q_ref).sum(axis=-1).max()
    kmax = np.abs(k_ref).max()
    rel = head_dim * 2.0 ** -24
    if levels >= 2:
        rel += 2.0 ** -17 + (block - 1) * levels * 2.0 ** -24
    return float(1e-5 + scale * q1 * kmax * rel)


def candidate_scores(q_l, k_l, parent, k):
    """fp64 scores of every query against its candidate list (children of its parent's picks,
    or all keys at the coarsest level).  Returns (cand [n, C], scores [n, C])."""
    n = q_l.shape[0]
    if parent is None:
        cand = np.broadcast_to(np.arange(k_l.shape[0]), (n, k_l.shape[0]))
        return cand, q_l @ k_l.T
    cand = (parent[np.arange(n) // B][:, :, None] * B + np.arange(B)).reshape(n, -1)
    scores = np.empty(cand.shape)
    for s in range(0, n, 1024):
        e = min(n, s + 1024)
        scores[s:e] = np.einsum("ad,acd->ac", q_l[s:e], k_l[cand[s:e]])
    return cand, scores


def check_level(gpu_sel, q_l, k_l, parent, k, where="", block=B):
    """Teacher-forced check of one level's selection of one head; returns #rows that differ
    from the oracle within the tie window.

    A differing row must hold K distinct candidates in ascending order, and no candidate the
    GPU left out may score more than GAP (relative) above the GPU's lowest pick: every pick is
    then a top-K pick up to the window, and the oracle's K-th and (K+1)-th scores lie within
    it too (the row is a near tie)."""
    n = q_l.shape[0]
    want = (orc.select_coarsest(q_l, k_l, k) if parent is None
            else orc.select_level(q_l, k_l, parent, block, k))
    got = np.asarray(gpu_sel, dtype=np.int64)
    assert got.shape == want.shape, where
    diff_rows = np.nonzero((got != want).any(axis=1))[0]
    if diff_rows.size == 0:
        return 0
    for a in diff_rows:
        if parent is None:
            c = np.arange(k_l.shape[0])
            s = q_l[a] @ k_l.T
        else:
            c = (parent[a // block][:, None] * block + np.arange(block)).reshape(-1)
            s = k_l[c] @ q_l[a]
        row = got[a]
        assert np.all(np.diff(row) > 0), f"{where} row {a}: not ascending/distinct: {row}"
        pos = {int(cid): i for i, cid in enumerate(c)}
        assert all(int(x) in pos for x in row), f"{where} row {a}: pick outside candidates"
        order = np.sort(s)[::-1]
        s_k, s_k1 = order[k - 1], order[k] if len(order) > k else -np.inf
        denom = max(abs(s_k), abs(s_k1) if np.isfinite(s_k1) else 0.0,
                    1e-6 * np.abs(s).max())
        picked = np.zeros(len(c), dtype=bool)
        picked[[pos[int(x)] for x in row]] = True
        low_pick = s[picked].min()
        best_left = s[~picked].max() if (~picked).any() else -np.inf
        worst = (best_left - low_pick) / denom
        assert worst < GAP, (f"{where} row {a}: GPU pick {row} vs oracle {want[a]}: a "
                             f"candidate left out scores {worst:.3g} (relative) above the "
                             f"lowest pick; the window is {GAP}")
        assert (s_k - s_k1) / denom < GAP, f"{where} row {a}: not a near-tie row"
    return int(diff_rows.size)


def check_selection(gpu_sel, q_lv, k_lv, k, where="", block=B):
    """gpu_sel: per level [b, H, n_l, K] arrays; q_lv/k_lv: oracle fp64 pooled levels."""
    levels = len(gpu_sel)
    flips = 0
    b, h = gpu_sel[0].shape[:2]
    for bi in range(b):
        for hi in range(h):
            for l in range(levels, 0, -1):
                parent = None if l == levels else gpu_sel[l][bi, hi]
                flips += check_level(gpu_sel[l - 1][bi, hi], q_lv[l - 1][bi, hi],
                                     k_lv[l - 1][bi, hi], parent, k,
                                     f"{where} b{bi} h{hi} level {l}", block)
    return flips


def gpu_sel_lists(sel, bsel=None, hsel=None):
    """[b][h] lists of per-level int64 arrays from device selections."""
    arrs = [s.cpu().numpy().astype(np.int64) for s in sel]
    b, h = arrs[0].shape[:2]
    bs = range(b) if bsel is None else bsel
    hs = range(h) if hsel is None else hsel
    return [[[a[bi, hi] for a in arrs] for hi in hs] for bi in bs]
