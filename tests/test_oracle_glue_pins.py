"""Pins of the oracle's glue either side of the scan.

SDM notes §2.4: alpha_t = exp(-A softplus(W_a x_t + b_dt)), beta_t =
sigmoid(W_b x_t); after the read each head's y_t goes through RMS-Norm and an
elementwise output gate (the gate's activation read as the sigmoid of the
FwPKM notes §2.3). Pinned by closed forms (zero input, A = 0, values whose
gates are exact dyadic rationals, the large-argument limits of softplus), a
one-hot input that isolates one projection weight, torch's rms_norm and the
scale invariance of RMS-Norm.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_memory_linear_amd import inputs


def _zeros(B=1, T=3, d=8, H=4):
    return (np.zeros((B, T, d), np.float32), np.zeros((H, d), np.float32), np.zeros((H, d), np.float32))


def test_zero_input_gives_closed_forms():
    """x = 0: alpha = (1 + e^b_dt)^-A and beta = 1/2 exactly; with b_dt = 0, A = 1
    alpha = 1/2; b_dt = ln 3, A = 2 gives (1 + 3)^-2 = 1/16; A = 0 gives 1."""
    x, Wa, Wb = _zeros()
    bdt = np.array([0.0, math.log(3.0), -1.0, 5.0], np.float32)
    A = np.array([1.0, 2.0, 0.0, 0.5], np.float32)
    al, be = oracle.gates(x, Wa, Wb, bdt, A)
    assert np.all(be == 0.5)
    assert np.all(al[:, 0] == 0.5)
    assert np.allclose(al[:, 1], 1.0 / 16.0, rtol=1e-7)
    assert np.all(al[:, 2] == 1.0)
    assert np.allclose(al[:, 3], (1.0 + math.exp(float(bdt[3]))) ** -0.5, rtol=1e-7)


def test_one_hot_input_isolates_one_weight():
    """x = e_i: the projections are W_a[h, i] and W_b[h, i]; beta = 3/4 exactly
    when W_b[h, i] = ln 3, and -log(alpha) / A = softplus(W_a[h, i] + b_dt)
    (inverted with a library expm1: z = log(expm1(softplus)))."""
    rng = np.random.default_rng(0)
    d, H = 16, 3
    Wa = rng.standard_normal((H, d)).astype(np.float32)
    Wb = rng.standard_normal((H, d)).astype(np.float32)
    Wb[1, 5] = math.log(3.0)
    bdt = rng.standard_normal(H).astype(np.float32)
    A = np.array([1.0, 0.7, 1.3], np.float32)
    x = np.eye(d, dtype=np.float32)[None]                # token i is the one-hot e_i
    al, be = oracle.gates(x, Wa, Wb, bdt, A)
    assert abs(float(be[0, 1, 5]) - 0.75) <= 1e-7
    sp = -np.log(al[0].astype(np.float64)) / A[:, None]
    z = np.log(np.expm1(sp))
    assert np.allclose(z, Wa.astype(np.float64) + bdt[:, None], rtol=1e-5, atol=1e-5)
    assert np.allclose(np.log(be[0] / (1 - be[0])), Wb, rtol=1e-5, atol=1e-5)


def test_softplus_limits():
    """softplus(z) -> z for large z (alpha -> e^{-A z}, no overflow) and -> e^z
    for very negative z (alpha -> 1 - A e^z)."""
    x, Wa, Wb = _zeros(H=2)
    bdt = np.array([40.0, -40.0], np.float32)
    A = np.array([0.25, 3.0], np.float32)
    al, _ = oracle.gates(x, Wa, Wb, bdt, A)
    assert np.allclose(al[:, 0], math.exp(-10.0), rtol=1e-7)
    assert np.allclose(al[:, 1], 1.0 - 3.0 * math.exp(-40.0), rtol=0, atol=1e-12)
    x2, Wa2, Wb2 = _zeros(H=1)
    al2, be2 = oracle.gates(x2, Wa2, Wb2, np.array([800.0], np.float32), np.array([1e-3], np.float32))
    assert np.all(np.isfinite(al2)) and np.allclose(al2, math.exp(-0.8), rtol=1e-6)


def test_gates_on_the_workload_inputs_are_in_range():
    wl = inputs.get("small", B=2, T=50)
    gx = inputs.make_glue_inputs(wl)
    al, be = oracle.gates(gx["x"], gx["W_a"], gx["W_b"], gx["b_dt"], gx["A"])
    assert al.shape == (2, wl.H, 50) and np.all((al > 0) & (al < 1)) and np.all((be > 0) & (be < 1))
    assert 0.8 < al.mean() < 0.97 and 0.4 < be.mean() < 0.6


def test_output_gate_matches_torch_rms_norm_and_sigmoid():
    rng = np.random.default_rng(2)
    B, H, T, dv = 2, 3, 7, 32
    y = rng.standard_normal((B, H, T, dv)).astype(np.float32) * 3
    g = rng.standard_normal((B, H, T, dv)).astype(np.float32)
    gamma = (1 + 0.1 * rng.standard_normal((H, dv))).astype(np.float32)
    eps = 1e-6
    o = oracle.output_gate(y, gamma, g, eps)
    yt = torch.from_numpy(y).double()
    for h in range(H):
        ref = torch.nn.functional.rms_norm(yt[:, h], (dv,), torch.from_numpy(gamma[h]).double(), eps)
        ref = ref * torch.sigmoid(torch.from_numpy(g[:, h]).double())
        assert np.allclose(o[:, h], ref.numpy(), rtol=2e-7, atol=1e-7)


def test_output_gate_closed_forms_and_scale_invariance():
    B, H, T, dv = 1, 2, 4, 8
    y = np.full((B, H, T, dv), -2.5, np.float32)
    g = np.zeros_like(y)
    gamma = np.ones((H, dv), np.float32)
    o = oracle.output_gate(y, gamma, g, 0.0)
    assert np.all(o == -0.5)                            # a constant row normalises to its sign; sigmoid(0) = 1/2
    rng = np.random.default_rng(3)
    y = rng.standard_normal((B, H, T, dv)).astype(np.float32)
    g = rng.standard_normal((B, H, T, dv)).astype(np.float32)
    gamma = rng.standard_normal((H, dv)).astype(np.float32)
    o1 = oracle.output_gate(y, gamma, g, 0.0)
    o2 = oracle.output_gate(y * 8.0, gamma, g, 0.0)     # exact power-of-two scaling
    assert np.array_equal(o1, o2)
    assert np.allclose(oracle.output_gate(y, gamma, np.full_like(g, 60.0), 0.0),
                       oracle.output_gate(y, gamma, np.full_like(g, 80.0), 0.0), rtol=1e-7)


def test_glue_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.output_gate(np.zeros((1, 1, 1, 4), np.float32), np.ones((1, 4), np.float32),
                           np.zeros((1, 1, 1, 4), np.float32), -1.0)
