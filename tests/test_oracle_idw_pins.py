"""Pins of the oracle's inverse-distance (IDW) subkey score.

Fast-weight Product Key Memory notes, §2.2: FwPKM's default subkey score is
s = -log(1e-3 + ||q - K_i||^2) rather than a dot product; near subkeys score
high, and after the softmax over the selected slots the weights are the
normalised inverse squared distances. The slot score is still the sum of the
two half-scores, so the product-key selection is unchanged.

The pins below use what that section fixes and what the mathematics gives:
the exact-match value -log(1e-3) = 3 ln 10, the nearest-neighbour order from a
library distance routine, the normalised inverse-distance weights, exact
translation invariance, and brute-force full-N top-k.
"""
import numpy as np
import pytest
import scipy.spatial.distance as ssd

import oracle
from sparse_memory_linear_amd import inputs

EPS = 1e-3                      # the constant of FwPKM §2.2
THREE_LN10 = 6.907755278982137  # -log(1e-3) = 3 ln 10


def _sqdist(q, K):
    """Squared Euclidean distances [T, n] from a library routine, in float64."""
    return ssd.cdist(np.asarray(q, np.float64), np.asarray(K, np.float64), metric="sqeuclidean")


def test_exact_match_scores_three_ln10_and_ranks_first():
    rng = np.random.default_rng(1)
    H, n, dh = 1, 16, 8
    K = rng.standard_normal((H, 2, n, dh)).astype(np.float32)
    q = np.empty((1, H, n, 2, dh), np.float32)
    for t in range(n):                       # token t copies subkey t of half 0, n-1-t of half 1
        q[0, 0, t, 0] = K[0, 0, t]
        q[0, 0, t, 1] = K[0, 1, n - 1 - t]
    hs = oracle.half_scores(q, K, scoring="idw")
    for t in range(n):
        assert hs[0, 0, t, 0, t] == np.float32(THREE_LN10)
        assert hs[0, 0, t, 1, n - 1 - t] == np.float32(THREE_LN10)
        assert np.argmax(hs[0, 0, t, 0]) == t and np.sum(hs[0, 0, t, 0] == hs[0, 0, t, 0].max()) == 1
    idx, wt, sc, _ = oracle.select(hs, 1)
    assert np.array_equal(idx[0, 0, :, 0], np.arange(n) * n + (n - 1 - np.arange(n)))
    assert np.all(wt == 1.0)


@pytest.mark.parametrize("name", ["tiny", "large_table"])
def test_half_scores_follow_library_squared_distances(name):
    wl = inputs.get(name, T=24, B=1, H=1)
    x = inputs.make_inputs(wl)
    hs = oracle.half_scores(x["q_w"], x["subkeys"], scoring="idw")
    q = x["q_w"].float().numpy(); K = x["subkeys"].float().numpy()
    for j in range(2):
        d2 = _sqdist(q[0, 0, :, j], K[0, j])
        # scores fall as the distance grows: -log is strictly decreasing
        ref = -np.log(EPS + d2)
        assert np.all(np.abs(hs[0, 0, :, j] - ref) <= 2 * np.spacing(np.abs(ref).astype(np.float32)))
        # nearest-neighbour order (ties by index) equals the score order
        for t in range(wl.T):
            by_dist = np.lexsort((np.arange(wl.n_sub), d2[t]))
            by_score = np.lexsort((np.arange(wl.n_sub), -hs[0, 0, t, j].astype(np.float64)))
            close = np.isclose(np.sort(d2[t])[1:], np.sort(d2[t])[:-1], rtol=1e-6).any()
            if not close:
                assert np.array_equal(by_dist, by_score)


@pytest.mark.parametrize("name", ["tiny", "small", "large_table"])
def test_weights_are_normalised_inverse_squared_distances(name):
    """softmax(-log(eps + d0) - log(eps + d1)) over the selection = normalised 1/((eps+d0)(eps+d1))."""
    wl = inputs.get(name, T=16, B=1, H=1)
    x = inputs.make_inputs(wl)
    k = wl.W
    idx, wt, sc, _ = oracle.address(x["q_w"], x["subkeys"], k, scoring="idw")
    q = x["q_w"].float().numpy(); K = x["subkeys"].float().numpy()
    n = wl.n_sub
    d0 = _sqdist(q[0, 0, :, 0], K[0, 0]); d1 = _sqdist(q[0, 0, :, 1], K[0, 1])
    for t in range(wl.T):
        a, b = np.divmod(idx[0, 0, t].astype(np.int64), n)
        inv = 1.0 / ((EPS + d0[t, a]) * (EPS + d1[t, b]))
        assert np.allclose(wt[0, 0, t], inv / inv.sum(), rtol=2e-5, atol=0)
        # the selection holds the k largest inverse-distance products of all N slots
        full = 1.0 / np.outer(EPS + d0[t], EPS + d1[t]).reshape(-1)
        order = np.argsort(-full, kind="stable")
        kth, nxt = full[order[k - 1]], full[order[k]] if k < n * n else 0.0
        if (kth - nxt) / kth > 1e-5:          # no near tie at the boundary
            assert set(idx[0, 0, t].tolist()) == set(order[:k].tolist())


def test_translation_invariance_is_exact():
    """Shifting q and every subkey by one vector leaves every distance, hence every
    score, unchanged; values on a 1/64 grid keep each shifted input exact in fp32."""
    rng = np.random.default_rng(7)
    H, n, dh, T = 2, 16, 8, 12
    K = (rng.integers(-256, 256, (H, 2, n, dh)) / 64).astype(np.float32)
    q = (rng.integers(-256, 256, (1, H, T, 2, dh)) / 64).astype(np.float32)
    c = rng.integers(-20, 20, dh).astype(np.float32)
    hs = oracle.half_scores(q, K, scoring="idw")
    hs2 = oracle.half_scores(q + c, K + c, scoring="idw")
    assert np.array_equal(hs, hs2)
    # a dot-product score is not translation invariant (the two scorings differ)
    assert not np.array_equal(oracle.half_scores(q, K), oracle.half_scores(q + c, K + c))


@pytest.mark.parametrize("name,k", [("tiny", 8), ("small", 16), ("large_table", 8)])
def test_pkm_equals_brute_force_with_idw_scores(name, k):
    from test_oracle_pins import brute_force_topk
    wl = inputs.get(name, T=32, B=1, H=1)
    x = inputs.make_inputs(wl)
    hs = oracle.half_scores(x["q_r"], x["subkeys"], scoring="idw")
    idx, wt, sc, nxt = oracle.select(hs, k)
    for t in range(wl.T):
        bs, bsc, bn = brute_force_topk(hs[0, 0, t, 0], hs[0, 0, t, 1], k)
        assert nxt[0, 0, t] == bn
        if bsc[-1] != bn:
            assert np.array_equal(idx[0, 0, t], bs) and np.array_equal(sc[0, 0, t], bsc)


def test_unknown_scoring_is_rejected():
    with pytest.raises(ValueError):
        oracle.half_scores(np.zeros((1, 1, 1, 2, 8), np.float32), np.zeros((1, 2, 16, 8), np.float32),
                           scoring="cosine")
