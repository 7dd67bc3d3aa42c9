"""GPU parity of the glue either side of the scan against the CPU oracle.

SDM notes §2.4: the gates alpha = exp(-A softplus(W_a x + b_dt)) and
beta = sigmoid(W_b x) from the layer input (one MFMA contraction over d for
all heads), and the per-head RMS-Norm with the sigmoid output gate after the
read. Both sides get identical inputs; the GPU accumulates in fp32, the
oracle in double.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_memory_linear_amd as sdm
from sparse_memory_linear_amd import inputs
from parity import TOL_BF16, TOL_F32, max_rel_err, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
U = 2.0 ** -24


def _gate_bounds(gx):
    """|GPU - oracle| bounds of alpha and beta: the fp32 accumulation of a
    length-d dot product is off by at most d * 2u * sum|w x|; alpha and beta
    change by at most A * dz and dz / 4; plus a few ulps of expf / log1pf."""
    x = gx["x"].double().numpy(); Wa = gx["W_a"].double().numpy(); Wb = gx["W_b"].double().numpy()
    d = x.shape[-1]
    ea = d * 2 * U * np.einsum("btc,hc->bht", np.abs(x), np.abs(Wa)) + 4 * U * np.abs(gx["b_dt"].numpy())[None, :, None]
    eb = d * 2 * U * np.einsum("btc,hc->bht", np.abs(x), np.abs(Wb))
    A = gx["A"].double().numpy()[None, :, None]
    return A * ea + 16 * U, eb / 4 + 16 * U


CASES = [("tiny", {}), ("small", dict(B=2, T=333)), ("gdn_matched", dict(B=1, T=1000)),
         ("large_table", dict(T=300)), ("small", dict(B=1, T=17, H=12))]


@pytest.mark.parametrize("name,over", CASES, ids=[f"{c[0]}-{i}" for i, c in enumerate(CASES)])
def test_gates_match_oracle(name, over):
    wl = inputs.get(name, **over)
    say(f"[gates] {name} {over}")
    gx = inputs.make_glue_inputs(wl)
    g = {k: v.to(DEV) for k, v in gx.items()}
    al, be = sdm.sdm_gates(g["x"], g["W_a"], g["W_b"], g["b_dt"], g["A"])
    torch.cuda.synchronize()
    oa, ob = oracle.gates(gx["x"], gx["W_a"], gx["W_b"], gx["b_dt"], gx["A"])
    ba, bb = _gate_bounds(gx)
    ea = np.abs(al.cpu().numpy().astype(np.float64) - oa)
    eb = np.abs(be.cpu().numpy().astype(np.float64) - ob)
    ra = max_rel_err(al.cpu().numpy()[..., None], oa[..., None])
    rb = max_rel_err(be.cpu().numpy()[..., None], ob[..., None])
    say(f"  alpha: max err {ea.max():.2e} (err/bound {np.max(ea / ba):.3f}), beta: {eb.max():.2e} "
        f"({np.max(eb / bb):.3f}); max rel err {ra:.2e} / {rb:.2e}")
    assert np.all(ea <= ba) and np.all(eb <= bb)
    tol = TOL_BF16 if wl.bf16_inputs else TOL_F32
    assert ra <= tol and rb <= tol


@pytest.mark.parametrize("name,over", [("tiny", {}), ("small", dict(B=2, T=300)),
                                       ("gdn_matched", dict(B=1, T=600)), ("large_table", dict(T=200))],
                         ids=["tiny", "small", "gdn_matched", "large_table"])
def test_output_gate_matches_oracle(name, over):
    wl = inputs.get(name, **over)
    say(f"[output gate] {name} {over}")
    gx = inputs.make_glue_inputs(wl)
    y = torch.randn((wl.B, wl.H, wl.T, wl.d_v), generator=torch.Generator().manual_seed(4)) * 0.3
    o = sdm.sdm_output_gate(y.to(DEV), gx["gamma"].to(DEV), gx["g"].to(DEV), 1e-6)
    torch.cuda.synchronize()
    ref = oracle.output_gate(y, gx["gamma"], gx["g"], 1e-6)
    err = max_rel_err(o.cpu().numpy(), ref)
    say(f"  max rel err {err:.2e}")
    assert err <= 1e-5


@pytest.mark.parametrize("dv", [4, 16, 36, 128, 512, 1024])
def test_output_gate_row_widths(dv):
    """Rows narrower than a wavefront (several rows per wavefront) and wider
    (several pieces per lane, a ragged last piece group)."""
    rng = np.random.default_rng(dv)
    B, H, T = 2, 3, 37
    y = torch.from_numpy(rng.standard_normal((B, H, T, dv)).astype(np.float32))
    g = torch.from_numpy(rng.standard_normal((B, H, T, dv)).astype(np.float32))
    gamma = torch.from_numpy((1 + 0.1 * rng.standard_normal((H, dv))).astype(np.float32))
    for eps in (0.0, 1e-5):
        o = sdm.sdm_output_gate(y.to(DEV), gamma.to(DEV), g.to(DEV), eps).cpu().numpy()
        assert max_rel_err(o, oracle.output_gate(y, gamma, g, eps)) <= 1e-5


def test_glue_empty_is_a_no_op():
    wl = inputs.get("small", B=1, T=0)
    gx = {k: v.to(DEV) for k, v in inputs.make_glue_inputs(wl).items()}
    al, be = sdm.sdm_gates(gx["x"], gx["W_a"], gx["W_b"], gx["b_dt"], gx["A"])
    assert al.numel() == 0 and be.numel() == 0
    o = sdm.sdm_output_gate(torch.empty((1, wl.H, 0, wl.d_v), device=DEV), gx["gamma"], gx["g"])
    assert o.numel() == 0


@pytest.mark.parametrize("name,over,form", [("small", dict(B=2, H=2, T=700), "eq4"),
                                             ("gdn_matched", dict(B=1, H=2, T=500), "eq4"),
                                             ("gdn_matched", dict(B=1, H=2, T=300), "fig2")])
def test_layer_gates_scan_output_match_oracle(name, over, form):
    """The layer around the path: gates from x, the scan (both sides fed the
    oracle's slots and weights), then the RMS-Norm and output gate; each side
    runs its own gates, so the gate rounding differences flow through."""
    wl = inputs.get(name, **over)
    say(f"[layer glue] {name} {over} {form}")
    x = inputs.make_inputs(wl)
    gx = inputs.make_glue_inputs(wl)
    oform = oracle.EQ4 if form == "eq4" else oracle.FIG2
    iw, ww, _, _ = oracle.address(x["q_w"], x["subkeys"], wl.W)
    ir, wr, _, _ = oracle.address(x["q_r"], x["subkeys"], wl.R)
    oa, ob = oracle.gates(gx["x"], gx["W_a"], gx["W_b"], gx["b_dt"], gx["A"])
    M_in = oracle.broadcast_state(x["M0"], wl.B)
    Mo, yo = oracle.scan(iw, ww, ir, wr, oa, ob, x["v"], M_in, oform)
    oo = oracle.output_gate(yo, gx["gamma"], gx["g"], 1e-6)
    g = {k: v.to(DEV) for k, v in gx.items()}
    al, be = sdm.sdm_gates(g["x"], g["W_a"], g["W_b"], g["b_dt"], g["A"])
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    M = sdm.sdm_state_init(x["M0"].to(DEV), wl.B)
    y = sdm.sdm_scan_forward(t(iw), t(ww), t(ir), t(wr), al, be, x["v"].to(DEV), M, form)
    o = sdm.sdm_output_gate(y, g["gamma"], g["g"], 1e-6)
    torch.cuda.synchronize()
    tol = TOL_BF16 if wl.bf16_inputs else TOL_F32
    e_o, e_m = max_rel_err(o.cpu().numpy(), oo), max_rel_err(M.cpu().numpy(), Mo)
    say(f"  max rel err o {e_o:.2e}, M {e_m:.2e}")
    assert e_o <= tol and e_m <= tol


def test_glue_full_size_gdn_matched():
    """The glue at the benchmark's full size (gdn_matched: 32768 tokens, d = 1024,
    8 heads; y of 33.5 M values)."""
    wl = inputs.get("gdn_matched")
    say(f"[glue full size] B={wl.B} H={wl.H} T={wl.T} d={inputs.d_model(wl)}")
    gx = inputs.make_glue_inputs(wl)
    g = {k: v.to(DEV) for k, v in gx.items()}
    al, be = sdm.sdm_gates(g["x"], g["W_a"], g["W_b"], g["b_dt"], g["A"])
    y = torch.randn((wl.B, wl.H, wl.T, wl.d_v), generator=torch.Generator().manual_seed(8)) * 0.3
    o = sdm.sdm_output_gate(y.to(DEV), g["gamma"], g["g"], 1e-6)
    torch.cuda.synchronize()
    oa, ob = oracle.gates(gx["x"], gx["W_a"], gx["W_b"], gx["b_dt"], gx["A"])
    ea = max_rel_err(al.cpu().numpy()[..., None], oa[..., None])
    eb = max_rel_err(be.cpu().numpy()[..., None], ob[..., None])
    eo = max_rel_err(o.cpu().numpy(), oracle.output_gate(y, gx["gamma"], gx["g"], 1e-6))
    say(f"  max rel err alpha {ea:.2e}, beta {eb:.2e}, o {eo:.2e}")
    assert ea <= TOL_BF16 and eb <= TOL_BF16 and eo <= 1e-5
