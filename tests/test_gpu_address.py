"""GPU parity of product-key addressing against the CPU oracle, through the C ABI.

Stage-decoupled, so that one rounding flip cannot hide or fake an error:
 1. the MFMA half-scores vs the oracle's double-accumulated ones (error bound);
 2. the selection logic: the oracle run on the GPU's own half-scores must
    reproduce the GPU slots bit for bit (same fp32 values, same decisions);
 3. end to end: GPU slots vs the oracle from the inputs, where the only
    allowed differences are near-ties of the oracle's k-th / (k+1)-th scores.
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


def _gpu(x):
    return {k: v.to(DEV) for k, v in x.items()}


def _half_bound(q, K):
    """Rounding bound of an fp32-accumulated dot product: dh * 2^-23 * sum |q_c K_c|."""
    qa = q.double().abs().numpy()
    Ka = K.double().abs().numpy()
    s = np.einsum("bhtjc,hjac->bhtja", qa, Ka)
    return q.shape[-1] * 2.0 ** -23 * s + 1e-30


CASES = [("tiny", {}), ("small", dict(B=2, H=2, T=1000)),
         ("gdn_matched", dict(B=1, H=2, T=500)), ("long_context", dict(H=2, T=300)),
         ("large_table", dict(T=150))]


@pytest.mark.parametrize("name,over", CASES, ids=[c[0] for c in CASES])
def test_half_scores_match_oracle(name, over):
    wl = inputs.get(name, **over)
    say(f"[address a1] {name} {over}")
    x = inputs.make_inputs(wl)
    g = _gpu(x)
    half = sdm.sdm_debug_half_scores(g["q_w"], g["subkeys"]).cpu().numpy()
    ref = oracle.half_scores(x["q_w"], x["subkeys"])
    bound = _half_bound(x["q_w"], x["subkeys"])
    err = np.abs(half.astype(np.float64) - ref)
    say(f"  max |err| {err.max():.3e}, max err/bound {np.max(err / bound):.3f}")
    assert np.all(err <= bound)


@pytest.mark.parametrize("name,over", CASES, ids=[c[0] for c in CASES])
def test_selection_bit_exact_on_gpu_half_scores(name, over):
    wl = inputs.get(name, **over)
    say(f"[address a2-a4 on GPU half-scores] {name} {over}")
    x = inputs.make_inputs(wl)
    g = _gpu(x)
    idx_w, wt_w, idx_r, wt_r, sc_w, sc_r = sdm.sdm_address(g["q_w"], g["q_r"], g["subkeys"],
                                                           g["subkeys"], wl.W, wl.R, True)
    for q, k, gi, gw, gs in ((g["q_w"], wl.W, idx_w, wt_w, sc_w), (g["q_r"], wl.R, idx_r, wt_r, sc_r)):
        half = sdm.sdm_debug_half_scores(q, g["subkeys"]).cpu()
        oi, ow, osc, _ = oracle.select(half, k)
        gi, gw, gs = gi.cpu().numpy(), gw.cpu().numpy(), gs.cpu().numpy()
        assert np.array_equal(gi, oi)
        assert np.array_equal(gs, osc)
        rel = np.abs(gw - ow) / np.maximum(ow, 1e-30)
        say(f"  k={k}: slots identical, max weight rel err {rel.max():.2e}")
        assert rel.max() < 2e-6 or np.abs(gw - ow).max() < 1e-7


@pytest.mark.parametrize("name,over", CASES, ids=[c[0] for c in CASES])
def test_slots_match_oracle_end_to_end(name, over):
    wl = inputs.get(name, **over)
    say(f"[address end to end] {name} {over}")
    x = inputs.make_inputs(wl)
    g = _gpu(x)
    idx_w, wt_w, idx_r, wt_r = sdm.sdm_address(g["q_w"], g["q_r"], g["subkeys"], g["subkeys"],
                                               wl.W, wl.R)
    for br, q, k, gi in (("write", x["q_w"], wl.W, idx_w), ("read", x["q_r"], wl.R, idx_r)):
        ohalf = oracle.half_scores(q, x["subkeys"])
        oi, ow, osc, onext = oracle.select(ohalf, k)
        res = compare_slots(gi.cpu().numpy(), oi, osc, onext, ohalf, label=f"dot {name} {over} {br}")
        say(f"  k={k}: {res}")
        assert res["violating"] == 0


def test_exact_integer_scores_with_ties():
    """One-hot half-queries and small-integer subkeys make every half-score an
    exact small integer on both sides: ties everywhere, all resolved by index."""
    rng = np.random.default_rng(5)
    B, H, T, n, dh = 1, 2, 96, 16, 32
    K = rng.integers(-3, 4, size=(H, 2, n, dh)).astype(np.float32)
    q = np.zeros((B, H, T, 2, dh), np.float32)
    cols = rng.integers(0, dh, size=(B, H, T, 2))
    np.put_along_axis(q, cols[..., None], 1.0, axis=-1)
    qt, Kt = torch.from_numpy(q).to(DEV), torch.from_numpy(K).to(DEV)
    for k in (1, 3, 8, 17, 64):
        say(f"[address ties] k={k}")
        iw, ww, ir, wr, sw, sr = sdm.sdm_address(qt, qt, Kt, Kt, k, k, True)
        oi, ow, osc, _ = oracle.address(q, K, k)
        assert np.array_equal(iw.cpu().numpy(), oi)
        assert np.array_equal(sw.cpu().numpy(), osc)
        assert np.allclose(ww.cpu().numpy(), ow, rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("T", [1, 15, 16, 17, 33])
def test_ragged_token_counts(T):
    wl = inputs.get("small", B=1, H=1, T=T)
    say(f"[address ragged] T={T}")
    x = inputs.make_inputs(wl)
    g = _gpu(x)
    iw, ww, ir, wr = sdm.sdm_address(g["q_w"], g["q_r"], g["subkeys"], g["subkeys"], wl.W, wl.R)
    half = sdm.sdm_debug_half_scores(g["q_r"], g["subkeys"]).cpu()
    oi, _, _, _ = oracle.select(half, wl.R)
    assert np.array_equal(ir.cpu().numpy(), oi)


@pytest.mark.parametrize("B,T", [(40, 1), (7, 3), (3, 17)])
def test_token_tiles_span_sequences(B, T):
    """Short calls pack tokens of several sequences of a head into one tile
    (decoding: T = 1); the half-scores, the selection and where each token's
    result lands must not depend on that."""
    wl = inputs.get("gdn_matched", B=B, H=2, T=T)
    say(f"[address tiles across sequences] B={B} T={T}")
    x = inputs.make_inputs(wl)
    g = _gpu(x)
    iw, ww, ir, wr = sdm.sdm_address(g["q_w"], g["q_r"], g["subkeys"], g["subkeys"], wl.W, wl.R)
    for q, idx, wt, k in ((g["q_w"], iw, ww, wl.W), (g["q_r"], ir, wr, wl.R)):
        half = sdm.sdm_debug_half_scores(q, g["subkeys"]).cpu()
        ref = oracle.half_scores(q.cpu(), x["subkeys"])
        assert np.all(np.abs(half.numpy().astype(np.float64) - ref) <= _half_bound(q.cpu(), x["subkeys"]))
        oi, ow, _, _ = oracle.select(half, k)
        assert np.array_equal(idx.cpu().numpy(), oi)
        gw = wt.cpu().numpy()
        assert np.max(np.abs(gw - ow) / np.maximum(ow, 1e-30)) < 2e-6 or np.abs(gw - ow).max() < 1e-7


def test_empty_input_is_a_no_op():
    wl = inputs.get("small", B=1, H=1, T=0)
    x = inputs.make_inputs(wl)
    g = _gpu(x)
    out = sdm.sdm_address(g["q_w"], g["q_r"], g["subkeys"], g["subkeys"], wl.W, wl.R)
    assert all(t.numel() == 0 for t in out)


def test_separate_write_and_read_subkeys():
    wl = inputs.get("small", B=1, H=2, T=64)
    say("[address] distinct subkey tables per branch")
    x = inputs.make_inputs(wl)
    K2 = torch.randn(x["subkeys"].shape, generator=torch.Generator().manual_seed(9))
    g = _gpu(x)
    iw, ww, ir, wr = sdm.sdm_address(g["q_w"], g["q_r"], g["subkeys"], K2.to(DEV), wl.W, wl.R)
    hr = sdm.sdm_debug_half_scores(g["q_r"], K2.to(DEV)).cpu()
    oi, _, _, _ = oracle.select(hr, wl.R)
    assert np.array_equal(ir.cpu().numpy(), oi)
    hw = sdm.sdm_debug_half_scores(g["q_w"], g["subkeys"]).cpu()
    oi, _, _, _ = oracle.select(hw, wl.W)
    assert np.array_equal(iw.cpu().numpy(), oi)


def test_deterministic_rerun():
    wl = inputs.get("gdn_matched", B=1, H=1, T=256)
    x = _gpu(inputs.make_inputs(wl))
    a = sdm.sdm_address(x["q_w"], x["q_r"], x["subkeys"], x["subkeys"], wl.W, wl.R)
    b = sdm.sdm_address(x["q_w"], x["q_r"], x["subkeys"], x["subkeys"], wl.W, wl.R)
    assert all(torch.equal(u, w) for u, w in zip(a, b))


@pytest.mark.parametrize("name", ["gdn_matched", "long_context"])
def test_full_size_sampled_tokens(name):
    """The full workload as the benchmark runs it; a seeded sample of
    token-branches is checked (stages 2 and 3) against the oracle."""
    wl = inputs.get(name)
    say(f"[address full size] {name} B={wl.B} H={wl.H} T={wl.T}")
    x = inputs.make_inputs(wl)
    g = _gpu(x)
    iw, ww, ir, wr = sdm.sdm_address(g["q_w"], g["q_r"], g["subkeys"], g["subkeys"], wl.W, wl.R)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    nb = 2048
    bs = torch.from_numpy(rng.integers(0, wl.B, nb)); hs = torch.from_numpy(rng.integers(0, wl.H, nb))
    ts = torch.from_numpy(rng.integers(0, wl.T, nb)); ar = torch.arange(nb)
    for qn, k, gi in (("q_w", wl.W, iw), ("q_r", wl.R, ir)):
        qs = x[qn][bs, hs, ts]                                   # [nb, 2, dh]
        # each sampled token as its own (b=0, h, t) row: keep its head's subkeys
        qsub = torch.zeros((1, wl.H, nb, 2, wl.d_h), dtype=qs.dtype)
        qsub[0, hs, ar] = qs
        half = sdm.sdm_debug_half_scores(qsub.to(DEV), g["subkeys"]).cpu()[0, hs, ar]
        oi2, _, _, _ = oracle.select(half.reshape(1, 1, nb, 2, wl.n_sub), k)
        gsel = gi[bs.to(DEV), hs.to(DEV), ts.to(DEV)].cpu().numpy()
        assert np.array_equal(gsel, oi2[0, 0])
        qq = torch.zeros((1, wl.H, nb, 2, wl.d_h), dtype=torch.float32)
        qq[0, hs, ar] = qs.float()
        ohalf = oracle.half_scores(qq, x["subkeys"])
        oi, ow, osc, onext = oracle.select(ohalf, k)
        sel = (0, hs.numpy(), ar.numpy())
        res = compare_slots(gsel, oi[sel], osc[sel], onext[sel], ohalf[sel],
                            label=f"dot {name} full size, {nb} sampled token-branches, {qn}")
        say(f"  {qn}: {res}")
        assert res["violating"] == 0
