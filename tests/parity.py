"""Comparison helpers shared by the GPU parity tests (no method arithmetic).

Every slot-list comparison made through ``compare_slots`` with a label is also
recorded in ``REPORT``; ``tests/conftest.py`` writes the records as JSON at the
end of the session when the environment variable SDM_PARITY_REPORT names a
file (the near-tie accounting of the end-to-end address checks).
"""
from __future__ import annotations

import sys

import numpy as np

# fp32 outputs and the final table: max relative error <= 1e-4; configs with
# bf16 inputs: <= 2e-2 (the inputs are identical bits on both sides, so the
# observed error is fp32 rounding in either case).
TOL_F32 = 1e-4
TOL_BF16 = 2e-2
# Checks whose two sides scan identical inputs (same slots, weights, gates,
# values and initial table) see only fp32 rounding order, observed near 1e-7
# relative; they assert this tighter bound as well, so that an error of a
# forwarded row or a partial sum well below the bf16 tolerance still fails.
TOL_SAME_INPUTS = 1e-5

REPORT: list = []


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


def slot_scores(half, slots) -> np.ndarray:
    """Oracle score of each slot a*n + b: the fp32 sum of the oracle's half-scores
    s_0[a] + s_1[b] (one fp32 add). half [..., 2, n], slots [..., k] -> [..., k]."""
    half = np.asarray(half, np.float32)
    n = half.shape[-1]
    slots = np.asarray(slots).astype(np.int64)
    h = half.reshape(-1, 2, n)
    s = slots.reshape(h.shape[0], -1)
    rows = np.arange(h.shape[0])[:, None]
    out = h[rows, 0, s // n] + h[rows, 1, s % n]   # float32 + float32 -> float32
    return out.reshape(slots.shape)


def _gap_hist(g) -> dict:
    g = np.asarray(g)
    return {"0": int((g == 0).sum()), "1": int((g == 1).sum()), "2-3": int(((g >= 2) & (g < 4)).sum()),
            "4-7": int(((g >= 4) & (g < 8)).sum()), "8-15": int(((g >= 8) & (g < 16)).sum()),
            ">=16": int((g >= 16).sum())}


def compare_slots(g_idx, o_idx, o_sc, o_next, o_half, label=None):
    """GPU slot lists vs the oracle's, per token-branch (last axis = the k slots).

    o_half holds the oracle's half-scores [..., 2, n] of the same token-branches,
    from which the oracle score of any slot (also of slots only the GPU picked)
    follows.

    exact:      identical ordered lists
    reordered:  same set, different order, and the oracle scores of the GPU's
                order are non-increasing within the near-tie tolerance
    near_tie:   different set, the oracle's k-th and (k+1)-th scores differ by
                less than tol = 1e-6 * max(1, |S_k|), and every slot in only one
                of the two sets has an oracle score within tol of S_k (the two
                lists differ only at the boundary)
    near_tie_literal: the near-ties whose gap is also below 1e-6 absolute
    violating:  anything else
    The gaps of the near-tie mismatches are histogrammed in fp32 ulps of |S_k|.
    """
    k = np.shape(g_idx)[-1]
    g_idx = np.asarray(g_idx).reshape(-1, k)
    o_idx = np.asarray(o_idx).reshape(-1, k)
    o_sc = np.asarray(o_sc, np.float32).reshape(-1, k)
    o_next = np.asarray(o_next, np.float32).reshape(-1)
    half = np.asarray(o_half, np.float32)
    half = half.reshape(-1, 2, half.shape[-1])
    exact = (g_idx == o_idx).all(1)
    same_set = (np.sort(g_idx, 1) == np.sort(o_idx, 1)).all(1)
    sk = o_sc[:, -1].astype(np.float64)
    gap = sk - o_next.astype(np.float64)
    tol = 1e-6 * np.maximum(1.0, np.abs(sk))
    near = np.zeros(len(exact), bool)
    boundary_ok = np.zeros(len(exact), bool)
    for i in np.nonzero(~same_set)[0]:
        if not gap[i] < tol[i]:
            continue
        near[i] = True
        gset, oset = set(g_idx[i].tolist()), set(o_idx[i].tolist())
        diff = np.array(sorted(gset ^ oset), np.int64)
        sc = slot_scores(half[i:i + 1], diff[None])[0].astype(np.float64)
        boundary_ok[i] = bool(np.all(np.abs(sc - sk[i]) <= tol[i]))
    reordered_ok = np.zeros_like(exact)
    for i in np.nonzero(same_set & ~exact)[0]:
        pos = {int(s): j for j, s in enumerate(o_idx[i])}
        s_in_gpu_order = np.array([o_sc[i, pos[int(s)]] for s in g_idx[i]], np.float64)
        reordered_ok[i] = np.all(np.diff(s_in_gpu_order) <= 1e-6 * np.maximum(1.0, np.abs(s_in_gpu_order[1:])))
    tie = ~same_set & near & boundary_ok
    ulp = np.spacing(np.abs(sk).astype(np.float32)).astype(np.float64)
    gaps_ulp = np.round(gap[tie] / ulp[tie]) if tie.any() else np.zeros(0)
    res = {
        "n": int(len(exact)),
        "exact": int(exact.sum()),
        "reordered": int((same_set & ~exact & reordered_ok).sum()),
        "near_tie": int(tie.sum()),
        "near_tie_literal": int((tie & (gap < 1e-6)).sum()),
        "violating": int((~same_set & ~tie).sum() + (same_set & ~exact & ~reordered_ok).sum()),
        "near_tie_gap_ulps": _gap_hist(gaps_ulp),
    }
    bad = np.nonzero(~same_set & ~tie)[0]
    if len(bad):
        res["violating_gaps"] = [float(gap[i]) for i in bad[:8]]
    if label is not None:
        REPORT.append({"check": label, "k": k, **res})
    return res
