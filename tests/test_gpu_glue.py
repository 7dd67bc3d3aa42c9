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


GATED = [("gdn_matched", dict(B=1, H=2, T=500), "eq4", "f32"),     # row partitions: the fused pass
         ("gdn_matched", dict(B=1, H=2, T=300), "fig2", "f32"),    # one partition: y, then the gate
         ("gdn_matched", dict(B=3, H=2, T=5), "eq4", "f32"),       # the short-call form
         ("gdn_matched", dict(B=1, H=2, T=400), "eq4", "bf16"),    # bf16 table, row partitions
         ("small", dict(B=2, H=2, T=333), "eq4", "f32"),           # fp32 gate input
         ("large_table", dict(T=200), "eq4", "f32")]               # d_v = 512: 2 pieces a lane


@pytest.mark.parametrize("name,over,form,table", GATED, ids=[f"{c[0]}-{c[2]}-{c[3]}-T{c[1]['T']}" for c in GATED])
def test_gated_scan_equals_scan_then_output_gate(name, over, form, table):
    """sdm_scan_forward_gated against sdm_scan_forward followed by
    sdm_output_gate: table, y and o bit-identical, with y returned or not."""
    wl = inputs.get(name, **over)
    say(f"[gated scan] {name} {over} {form} table={table}")
    x = inputs.make_inputs(wl)
    gx = inputs.make_glue_inputs(wl)
    g = {k: v.to(DEV) for k, v in x.items()}
    gg = {k: v.to(DEV) for k, v in gx.items()}
    iw, ww, ir, wr = sdm.sdm_address(g["q_w"], g["q_r"], g["subkeys"], g["subkeys"], wl.W, wl.R)
    M0 = sdm.sdm_state_init(g["M0"], wl.B)
    if table == "bf16":
        M0 = M0.to(torch.bfloat16)
    M1, M2, M3 = M0.clone(), M0.clone(), M0.clone()
    y1 = sdm.sdm_scan_forward(iw, ww, ir, wr, g["alpha"], g["beta"], g["v"], M1, form)
    o1 = sdm.sdm_output_gate(y1, gg["gamma"], gg["g"], 1e-6)
    o2, y2 = sdm.sdm_scan_forward_gated(iw, ww, ir, wr, g["alpha"], g["beta"], g["v"], M2, gg["gamma"], gg["g"],
                                        1e-6, form, keep_y=True)
    o3 = sdm.sdm_scan_forward_gated(iw, ww, ir, wr, g["alpha"], g["beta"], g["v"], M3, gg["gamma"], gg["g"],
                                    1e-6, form)
    torch.cuda.synchronize()
    assert torch.equal(M1, M2) and torch.equal(M1, M3)
    assert torch.equal(y1, y2)
    assert torch.equal(o1, o2) and torch.equal(o1, o3)


def test_gated_scan_layer_matches_oracle():
    """The whole layer step through the gated call against the oracle chain
    (addressing, gates, scan, RMS-Norm and gate), both sides on the oracle's
    slots and weights."""
    wl = inputs.get("gdn_matched", B=1, H=2, T=600)
    say("[gated scan vs oracle] gdn_matched B=1 H=2 T=600")
    x = inputs.make_inputs(wl)
    gx = inputs.make_glue_inputs(wl)
    iw, ww, _, _ = oracle.address(x["q_w"], x["subkeys"], wl.W)
    ir, wr, _, _ = oracle.address(x["q_r"], x["subkeys"], wl.R)
    oa, ob = oracle.gates(gx["x"], gx["W_a"], gx["W_b"], gx["b_dt"], gx["A"])
    Mo, yo = oracle.scan(iw, ww, ir, wr, oa, ob, x["v"], oracle.broadcast_state(x["M0"], wl.B), oracle.EQ4)
    oo = oracle.output_gate(yo, gx["gamma"], gx["g"], 1e-6)
    g = {k: v.to(DEV) for k, v in gx.items()}
    al, be = sdm.sdm_gates(g["x"], g["W_a"], g["W_b"], g["b_dt"], g["A"])
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    M = sdm.sdm_state_init(x["M0"].to(DEV), wl.B)
    o = sdm.sdm_scan_forward_gated(t(iw), t(ww), t(ir), t(wr), al, be, x["v"].to(DEV), M, g["gamma"], g["g"],
                                   1e-6, "eq4")
    torch.cuda.synchronize()
    e_o, e_m = max_rel_err(o.cpu().numpy(), oo), max_rel_err(M.cpu().numpy(), Mo)
    say(f"  max rel err o {e_o:.2e}, M {e_m:.2e}")
    assert e_o <= TOL_BF16 and e_m <= TOL_BF16


def test_gated_scan_full_size_gdn_matched():
    """The gated call in the benchmark's launch configuration (32 streams of
    8192 tokens: two row partitions, the fused pass) equals scan + output gate."""
    wl = inputs.get("gdn_matched")
    say(f"[gated scan full size] B={wl.B} H={wl.H} T={wl.T}")
    x = inputs.make_inputs(wl)
    gx = inputs.make_glue_inputs(wl)
    g = {k: v.to(DEV) for k, v in x.items()}
    gg = {k: v.to(DEV) for k, v in gx.items()}
    iw, ww, ir, wr = sdm.sdm_address(g["q_w"], g["q_r"], g["subkeys"], g["subkeys"], wl.W, wl.R)
    M1 = sdm.sdm_state_init(g["M0"], wl.B)
    M2 = M1.clone()
    y1 = sdm.sdm_scan_forward(iw, ww, ir, wr, g["alpha"], g["beta"], g["v"], M1, "eq4")
    o1 = sdm.sdm_output_gate(y1, gg["gamma"], gg["g"], 1e-6)
    del y1
    o2 = sdm.sdm_scan_forward_gated(iw, ww, ir, wr, g["alpha"], g["beta"], g["v"], M2, gg["gamma"], gg["g"], 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(M1, M2) and torch.equal(o1, o2)
