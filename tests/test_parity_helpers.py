"""The slot-list comparison the end-to-end address checks use (tests/parity.py),
on hand-made cases: it must accept exact lists, reorders within equal scores
and boundary near-ties, and reject everything else, in particular a near-tie
token whose lists also differ away from the boundary."""
import numpy as np

from parity import compare_slots, slot_scores


def _case(k=4):
    # n = 4 subkeys per half; half-scores chosen so that slot a*4+b scores s0[a] + s1[b]
    half = np.zeros((1, 2, 4), np.float32)
    half[0, 0] = [10.0, 8.0, 5.0, 1.0]
    half[0, 1] = [3.0, 2.0, 1.0, 0.0]
    sc = slot_scores(half, np.arange(16)[None])[0]
    order = sorted(range(16), key=lambda s: (-sc[s], s))
    idx = np.array(order[:k])[None]
    return half, idx, sc[idx], np.array([sc[order[k]]], np.float32), order


def test_exact_and_reordered_and_violations():
    half, idx, osc, onx, order = _case()
    assert compare_slots(idx, idx, osc, onx, half)["exact"] == 1
    # a top slot swapped for a low one, no near tie: violating
    g = idx.copy(); g[0, 0] = order[15]
    assert compare_slots(g, idx, osc, onx, half)["violating"] == 1
    # same set, order breaking the scores: violating
    g = idx[:, ::-1].copy()
    assert compare_slots(g, idx, osc, onx, half)["violating"] == 1


def test_near_tie_accepted_only_at_the_boundary():
    half = np.zeros((1, 2, 4), np.float32)
    # slot scores 13, 11.0, 11.0 + 1 ulp ... : make the 4th and 5th best equal up to 1 ulp
    half[0, 0] = [10.0, 8.0, 2.0, 1.0]
    half[0, 1] = [3.0, 2.0, 1.0, 0.0]
    sc = slot_scores(half, np.arange(16)[None])[0]
    order = sorted(range(16), key=lambda s: (-sc[s], s))
    k = 4
    # bump the (k+1)-th slot's score to within tolerance below the k-th
    sk = sc[order[k - 1]]
    idx = np.array(order[:k])[None]
    osc = sc[idx]
    onx = np.array([np.nextafter(sk, np.float32(-np.inf))], np.float32)
    # GPU swapped the k-th for the (k+1)-th: accepted only if that slot scores within tol of S_k
    half_t = half.copy()
    a, b = divmod(order[k], 4)
    half_t[0, 1, b] = np.float32(onx[0] - half_t[0, 0, a])
    g = idx.copy(); g[0, k - 1] = order[k]
    r = compare_slots(g, idx, osc, onx, half_t)
    assert r["near_tie"] == 1 and r["violating"] == 0 and r["near_tie_literal"] == 1
    # the same near-tie token, but a top-ranked slot swapped for an unrelated low one: violating
    g2 = idx.copy(); g2[0, 0] = order[15]
    r2 = compare_slots(g2, idx, osc, onx, half_t)
    assert r2["near_tie"] == 0 and r2["violating"] == 1
