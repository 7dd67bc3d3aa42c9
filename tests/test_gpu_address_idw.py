"""GPU parity of the inverse-distance (IDW) addressing against the CPU oracle.

Fast-weight Product Key Memory notes §2.2: subkey score -log(1e-3 + ||q - K||^2).
The GPU forms the squared distance as ||q||^2 + ||K||^2 - 2 <q, K> in fp32 (the
inner product on MFMA); the oracle sums the squared differences in double. The
same three stages as the dot-product addressing:
 1. half-scores within the rounding bound of the GPU's formula;
 2. the oracle's selection run on the GPU's own half-scores reproduces the
    GPU's slots bit for bit;
 3. end to end, GPU slots vs the oracle from the inputs, with differences
    allowed only at near-ties of the oracle's k-th / (k+1)-th slot scores.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_memory_linear_amd as sdm
from sparse_memory_linear_amd import inputs
from parity import compare_slots, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
U = 2.0 ** -24


def _gpu(x):
    return {k: v.to(DEV) for k, v in x.items()}


def _idw_bound(q, K, ref):
    """Bound on |GPU - oracle| of an IDW half-score. The GPU's squared distance
    d2 = qn + kn - 2 dot carries the fp32 accumulation errors of the three sums
    (dh u per term magnitude each) and three roundings of the combination; the
    logarithm turns an absolute error E of 1e-3 + d2 into E / (1e-3 + d2 - E),
    plus a few ulps of logf and of the final rounding."""
    qd = q.double().numpy(); Kd = K.double().numpy()
    dh = q.shape[-1]
    qn = np.einsum("bhtjc,bhtjc->bhtj", qd, qd)[..., None]
    kn = np.einsum("hjac,hjac->hja", Kd, Kd)[None, :, None]
    absdot = np.einsum("bhtjc,hjac->bhtja", np.abs(qd), np.abs(Kd))
    E = 2 * dh * U * (qn + kn + 2 * absdot) + 4 * U * (qn + kn + 2 * absdot) + 4 * U * 1e-3
    t = np.exp(-ref.astype(np.float64))              # 1e-3 + d2 from the oracle's score
    with np.errstate(divide="ignore"):
        b = np.where(t > E, E / np.maximum(t - E, 1e-300), np.inf)
    return b + 8 * U * np.maximum(np.abs(ref), 1.0)


CASES = [("tiny", {}), ("small", dict(B=2, H=2, T=1000)),
         ("gdn_matched", dict(B=1, H=2, T=500)), ("long_context", dict(H=2, T=300)),
         ("large_table", dict(T=150))]


@pytest.mark.parametrize("name,over", CASES, ids=[c[0] for c in CASES])
def test_idw_half_scores_match_oracle(name, over):
    wl = inputs.get(name, **over)
    say(f"[idw a1] {name} {over}")
    x = inputs.make_inputs(wl)
    g = _gpu(x)
    half = sdm.sdm_debug_half_scores(g["q_w"], g["subkeys"], scoring="idw").cpu().numpy()
    ref = oracle.half_scores(x["q_w"], x["subkeys"], scoring="idw")
    bound = _idw_bound(x["q_w"], x["subkeys"], ref)
    err = np.abs(half.astype(np.float64) - ref)
    say(f"  max |err| {err.max():.3e}, max err/bound {np.max(err / bound):.3f}")
    assert np.all(err <= bound)


@pytest.mark.parametrize("name,over", CASES, ids=[c[0] for c in CASES])
def test_idw_selection_bit_exact_on_gpu_half_scores(name, over):
    wl = inputs.get(name, **over)
    say(f"[idw a2-a4 on GPU half-scores] {name} {over}")
    x = inputs.make_inputs(wl)
    g = _gpu(x)
    idx_w, wt_w, idx_r, wt_r, sc_w, sc_r = sdm.sdm_address(
        g["q_w"], g["q_r"], g["subkeys"], g["subkeys"], wl.W, wl.R, True, scoring="idw")
    for q, k, gi, gw, gs in ((g["q_w"], wl.W, idx_w, wt_w, sc_w), (g["q_r"], wl.R, idx_r, wt_r, sc_r)):
        half = sdm.sdm_debug_half_scores(q, g["subkeys"], scoring="idw").cpu()
        oi, ow, osc, _ = oracle.select(half, k)
        gi, gw, gs = gi.cpu().numpy(), gw.cpu().numpy(), gs.cpu().numpy()
        assert np.array_equal(gi, oi)
        assert np.array_equal(gs, osc)
        rel = np.abs(gw - ow) / np.maximum(ow, 1e-30)
        say(f"  k={k}: slots identical, max weight rel err {rel.max():.2e}")
        assert rel.max() < 2e-6 or np.abs(gw - ow).max() < 1e-7


@pytest.mark.parametrize("name,over", CASES, ids=[c[0] for c in CASES])
def test_idw_slots_match_oracle_end_to_end(name, over):
    wl = inputs.get(name, **over)
    say(f"[idw end to end] {name} {over}")
    x = inputs.make_inputs(wl)
    g = _gpu(x)
    idx_w, wt_w, idx_r, wt_r = sdm.sdm_address(g["q_w"], g["q_r"], g["subkeys"], g["subkeys"],
                                               wl.W, wl.R, scoring="idw")
    for br, q, k, gi, gw in (("write", x["q_w"], wl.W, idx_w, wt_w), ("read", x["q_r"], wl.R, idx_r, wt_r)):
        ohalf = oracle.half_scores(q, x["subkeys"], scoring="idw")
        oi, ow, osc, onext = oracle.select(ohalf, k)
        gi = gi.cpu().numpy()
        res = compare_slots(gi, oi, osc, onext, ohalf, label=f"idw {name} {over} {br}")
        say(f"  k={k}: {res}")
        assert res["violating"] == 0
        same = (gi == oi).all(-1)
        gw = gw.cpu().numpy()
        assert np.max(np.abs(gw[same] - ow[same]) / np.maximum(ow[same], 1e-30)) < 1e-4


def test_idw_exact_match_selects_the_matched_slot():
    """A half-query equal to one of its subkeys is at distance 0: that subkey
    scores -log(1e-3) = 3 ln 10 (the largest possible score, within the GPU's
    cancellation error) and the matched pair is selected first."""
    rng = np.random.default_rng(3)
    H, n, dh, T = 2, 64, 32, 48
    K = (rng.integers(-16, 17, (H, 2, n, dh)) / 8).astype(np.float32)   # exact sums in fp32
    a = rng.integers(0, n, (1, H, T, 2))
    q = np.empty((1, H, T, 2, dh), np.float32)
    for h in range(H):
        for t in range(T):
            for j in range(2):
                q[0, h, t, j] = K[h, j, a[0, h, t, j]]
    qt, Kt = torch.from_numpy(q).to(DEV), torch.from_numpy(K).to(DEV)
    half = sdm.sdm_debug_half_scores(qt, Kt, scoring="idw").cpu().numpy()
    hit = np.take_along_axis(half, a[..., None], axis=-1)[..., 0]
    # d2 is exactly 0 on this grid; what is left is logf's rounding of -log(1e-3f)
    assert np.all(np.abs(hit.astype(np.float64) - 6.907755278982137) <= 4 * np.spacing(np.float32(6.9)))
    others = half.copy()
    np.put_along_axis(others, a[..., None], -np.inf, axis=-1)
    assert np.all(others.max(-1) < 5.0)           # nearest other subkey: d2 >= 1/64
    iw, ww, ir, wr = sdm.sdm_address(qt, qt, Kt, Kt, 8, 8, scoring="idw")
    assert np.array_equal(iw.cpu().numpy()[..., 0], a[..., 0] * n + a[..., 1])


@pytest.mark.parametrize("T", [1, 15, 17])
def test_idw_ragged_token_counts(T):
    wl = inputs.get("large_table", T=T)
    say(f"[idw ragged] T={T}")
    x = inputs.make_inputs(wl)
    g = _gpu(x)
    iw, ww, ir, wr = sdm.sdm_address(g["q_w"], g["q_r"], g["subkeys"], g["subkeys"], wl.W, wl.R,
                                     scoring="idw")
    half = sdm.sdm_debug_half_scores(g["q_r"], g["subkeys"], scoring="idw").cpu()
    oi, _, _, _ = oracle.select(half, wl.R)
    assert np.array_equal(ir.cpu().numpy(), oi)


@pytest.mark.parametrize("name", ["large_table", "gdn_matched"])
def test_idw_full_size_sampled_tokens(name):
    """The full workload (large_table is the FwPKM value-table size, whose
    default scoring is IDW); a seeded sample of token-branches is checked
    against the oracle (stages 2 and 3)."""
    wl = inputs.get(name)
    say(f"[idw full size] {name} B={wl.B} H={wl.H} T={wl.T}")
    x = inputs.make_inputs(wl)
    g = _gpu(x)
    iw, ww, ir, wr = sdm.sdm_address(g["q_w"], g["q_r"], g["subkeys"], g["subkeys"], wl.W, wl.R,
                                     scoring="idw")
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    nb = 2048
    bs = torch.from_numpy(rng.integers(0, wl.B, nb)); hs = torch.from_numpy(rng.integers(0, wl.H, nb))
    ts = torch.from_numpy(rng.integers(0, wl.T, nb)); ar = torch.arange(nb)
    for qn, k, gi in (("q_w", wl.W, iw), ("q_r", wl.R, ir)):
        qs = x[qn][bs, hs, ts]
        qsub = torch.zeros((1, wl.H, nb, 2, wl.d_h), dtype=qs.dtype)
        qsub[0, hs, ar] = qs
        half = sdm.sdm_debug_half_scores(qsub.to(DEV), g["subkeys"], scoring="idw").cpu()[0, hs, ar]
        oi2, _, _, _ = oracle.select(half.reshape(1, 1, nb, 2, wl.n_sub), k)
        gsel = gi[bs.to(DEV), hs.to(DEV), ts.to(DEV)].cpu().numpy()
        assert np.array_equal(gsel, oi2[0, 0])
        qq = torch.zeros((1, wl.H, nb, 2, wl.d_h), dtype=torch.float32)
        qq[0, hs, ar] = qs.float()
        ohalf = oracle.half_scores(qq, x["subkeys"], scoring="idw")
        oi, ow, osc, onext = oracle.select(ohalf, k)
        sel = (0, hs.numpy(), ar.numpy())
        res = compare_slots(gsel, oi[sel], osc[sel], onext[sel], ohalf[sel],
                            label=f"idw {name} full size, {nb} sampled token-branches, {qn}")
        say(f"  {qn}: {res}")
        assert res["violating"] == 0
