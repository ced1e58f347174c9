"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI, run the CPU
oracle on the same seeded inputs, and compare with the acceptance rules:

* reorder and index transpose: bit-exact;
* selections: identical sets, except that a pick may differ from the oracle's where the
  oracle's fp64 score of the GPU's pick lies within 1e-4 (relative) of the K-th best score
  (the GPU scores in fp32); every level is checked teacher-forced on the GPU's parent picks;
* outputs and gradients: max-abs <= 2e-2 and mean-rel <= 5e-3 for bf16 inputs, both <= 1e-4
  for fp32 inputs (mean-rel = mean|x - ref| / mean|ref|), with the oracle attention run on
  the GPU's selection.  The bounds apply to the arithmetic: a tensor stored in bf16 may also
  carry the rounding of its exact value to bf16 (at most half an ulp, <= 2^-8 |ref|), which
  the max-abs check adds per element (no bf16 number can be nearer than that).
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


def assert_close(x: np.ndarray, ref: np.ndarray, dtype: torch.dtype, name: str,
                 rel_slack: float | None = None):
    """dtype: input precision (picks the tolerance).  rel_slack: per-element allowance
    rel_slack*|ref| added to the max-abs bound; defaults to the bf16 storage rounding 2^-8
    for bf16 tensors and 0 for fp32 ones."""
    tol_abs, tol_rel = tolerances(dtype)
    if rel_slack is None:
        rel_slack = 2.0 ** -8 if dtype == torch.bfloat16 else 0.0
    err = np.abs(x - ref)
    allow = tol_abs + np.abs(ref) * rel_slack
    excess = float((err - allow).max())
    max_abs = float(err.max())
    mean_rel = float(err.mean() / max(np.abs(ref).mean(), 1e-30))
    _log(dict(name=name, max_abs=max_abs, mean_rel=mean_rel, max_ref=float(np.abs(ref).max()),
              worst_over_bound=excess))
    assert np.isfinite(x).all(), f"{name}: non-finite values"
    assert excess <= 0 and mean_rel <= tol_rel, (
        f"{name}: max-abs {max_abs:.3g} (bound {tol_abs} + storage; worst excess {excess:.3g}) "
        f"mean-rel {mean_rel:.3g} (tol {tol_rel}); max|ref| {np.abs(ref).max():.3g}")
    return max_abs, mean_rel


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
    from the oracle within the tie window."""
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
        picked = np.array([s[pos[int(x)]] for x in row])
        worst = (s_k - picked.min()) / denom
        assert worst < GAP, (f"{where} row {a}: GPU pick {row} vs oracle {want[a]}: "
                             f"relative gap {worst:.3g} exceeds {GAP}")
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
