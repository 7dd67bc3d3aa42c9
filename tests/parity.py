"""Comparison helpers shared by the GPU parity tests (no method arithmetic)."""
from __future__ import annotations

import sys

import numpy as np

# fp32 outputs and the final table: max relative error <= 1e-4; configs with
# bf16 inputs: <= 2e-2 (the inputs are identical bits on both sides, so the
# observed error is fp32 rounding in either case).
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def max_rel_err(x, r) -> float:
    """Per vector (last axis): ||x - r||_inf / max(||r||_inf, 1e-6 ||R||_inf), max over vectors."""
    x = np.asarray(x, np.float64).reshape(-1, np.shape(x)[-1])
    r = np.asarray(r, np.float64).reshape(-1, np.shape(r)[-1])
    floor = max(1e-6 * float(np.abs(r).max()), 1e-30)
    den = np.maximum(np.abs(r).max(axis=1), floor)
    return float((np.abs(x - r).max(axis=1) / den).max())


def compare_slots(g_idx, o_idx, o_sc, o_next, g_sc=None):
    """GPU slot lists vs the oracle's, per token-branch (last axis = the k slots).

    exact:      identical ordered lists
    reordered:  same set, different order, and the oracle scores of the GPU's
                order are non-increasing within the near-tie tolerance
    near_tie:   different set, but the oracle's k-th and (k+1)-th scores differ
                by less than 1e-6 * max(1, |S_k|)   (literal: by less than 1e-6)
    violating:  anything else
    """
    g_idx = np.asarray(g_idx).reshape(-1, np.shape(g_idx)[-1])
    o_idx = np.asarray(o_idx).reshape(-1, np.shape(o_idx)[-1])
    o_sc = np.asarray(o_sc, np.float64).reshape(-1, np.shape(o_sc)[-1])
    o_next = np.asarray(o_next, np.float64).reshape(-1)
    exact = (g_idx == o_idx).all(1)
    same_set = (np.sort(g_idx, 1) == np.sort(o_idx, 1)).all(1)
    sk = o_sc[:, -1]
    gap = sk - o_next
    tol = 1e-6 * np.maximum(1.0, np.abs(sk))
    near = gap < tol
    near_literal = gap < 1e-6
    reordered_ok = np.zeros_like(exact)
    for i in np.nonzero(same_set & ~exact)[0]:
        pos = {int(s): j for j, s in enumerate(o_idx[i])}
        s_in_gpu_order = np.array([o_sc[i, pos[int(s)]] for s in g_idx[i]])
        reordered_ok[i] = np.all(np.diff(s_in_gpu_order) <= 1e-6 * np.maximum(1.0, np.abs(s_in_gpu_order[1:])))
    res = {
        "n": int(len(exact)),
        "exact": int(exact.sum()),
        "reordered": int((same_set & ~exact & reordered_ok).sum()),
        "near_tie": int((~same_set & near).sum()),
        "near_tie_literal": int((~same_set & near_literal).sum()),
        "violating": int(((~same_set) & ~near).sum() + (same_set & ~exact & ~reordered_ok).sum()),
    }
    bad = np.nonzero((~same_set) & ~near)[0]
    if len(bad):
        res["violating_gaps"] = [float(gap[i]) for i in bad[:8]]
    return res
