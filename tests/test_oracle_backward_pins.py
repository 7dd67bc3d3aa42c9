"""Pins of the oracle's backward of the scan, against things other than itself.

The backward ([SDM] §2.9 Appendix A: tokens in reverse, written rows restored
from their pre-images) is hand-derived in the oracle; here it is checked
against (i) torch autograd through a plain float64 PyTorch forward of the
recurrence ([SDM] §2.4 Eq. (3)-(5), §2.5 Fig. 2), (ii) central finite
differences of the oracle's own (already pinned) forward, one input group at a
time, (iii) the frozen-table case (alpha = 1, beta = 0), where the read's
adjoint is an index_add and the write's value gradient vanishes, and (iv)
invariants: linearity in the cotangents, the split of a sequence into two
calls, and the single-write case where both write forms coincide.
"""
import numpy as np
import pytest
import torch

import oracle

GROUPS = ("v", "alpha", "beta", "wt_w", "wt_r", "M_in")
GRAD_OF = {"v": "dv", "alpha": "dalpha", "beta": "dbeta", "wt_w": "dwt_w", "wt_r": "dwt_r", "M_in": "dM_in"}


def _case(seed, B=1, H=2, T=24, N=16, dv=8, W=4, R=5):
    rng = np.random.default_rng(seed)
    n = B * H * T
    iw = np.stack([rng.permutation(N)[:W] for _ in range(n)]).reshape(B, H, T, W).astype(np.int32)
    ir = np.stack([rng.permutation(N)[:R] for _ in range(n)]).reshape(B, H, T, R).astype(np.int32)
    c = dict(idx_w=iw, idx_r=ir,
             wt_w=rng.dirichlet(np.ones(W), size=(B, H, T)).astype(np.float32),
             wt_r=rng.dirichlet(np.ones(R), size=(B, H, T)).astype(np.float32),
             alpha=(1 / (1 + np.exp(-rng.normal(2, .5, (B, H, T))))).astype(np.float32),
             beta=(1 / (1 + np.exp(-rng.normal(0, 1, (B, H, T))))).astype(np.float32),
             v=rng.standard_normal((B, H, T, dv)).astype(np.float32),
             M_in=(rng.standard_normal((B, H, N, dv)) * 0.5).astype(np.float32))
    dy = rng.standard_normal((B, H, T, dv)).astype(np.float32)
    dM = rng.standard_normal((B, H, N, dv)).astype(np.float32)
    return c, dy, dM


def _torch_forward(c, form, leaves):
    """The recurrence written with differentiable torch ops in float64 (gather,
    index_copy); returns (final tables, y) for every (b, h)."""
    B, H, T, W = c["idx_w"].shape
    Ms, ys = [], []
    for b in range(B):
        for h in range(H):
            M = leaves["M_in"][b, h]
            yl = []
            for t in range(T):
                iw = torch.from_numpy(c["idx_w"][b, h, t].astype(np.int64))
                ir = torch.from_numpy(c["idx_r"][b, h, t].astype(np.int64))
                a, be = leaves["alpha"][b, h, t], leaves["beta"][b, h, t]
                w, r, v = leaves["wt_w"][b, h, t], leaves["wt_r"][b, h, t], leaves["v"][b, h, t]
                mt = a * M[iw]
                pred = mt if form == oracle.EQ4 else (w[:, None] * mt).sum(0, keepdim=True)
                M = M.index_copy(0, iw, mt + be * w[:, None] * (v[None] - pred))
                yl.append((r[:, None] * M[ir]).sum(0))
            Ms.append(M)
            ys.append(torch.stack(yl))
    return Ms, ys


def _autograd(c, dy, dM, form):
    leaves = {k: torch.from_numpy(c[k].astype(np.float64)).requires_grad_(True) for k in GROUPS}
    Ms, ys = _torch_forward(c, form, leaves)
    B, H = c["idx_w"].shape[:2]
    loss = 0
    for s in range(B * H):
        b, h = divmod(s, H)
        loss = loss + (ys[s] * torch.from_numpy(dy[b, h].astype(np.float64))).sum() \
            + (Ms[s] * torch.from_numpy(dM[b, h].astype(np.float64))).sum()
    loss.backward()
    return {GRAD_OF[k]: leaves[k].grad.numpy() for k in GROUPS}


def _rel(x, r):
    return np.max(np.abs(x.astype(np.float64) - r)) / max(np.max(np.abs(r)), 1e-30)


@pytest.mark.parametrize("form", [oracle.EQ4, oracle.FIG2], ids=["eq4", "fig2"])
@pytest.mark.parametrize("seed", [0, 1])
def test_backward_matches_autograd(form, seed):
    c, dy, dM = _case(seed)
    got = oracle.scan_backward(**c, dy=dy, dM_out=dM, form=form)
    ref = _autograd(c, dy, dM, form)
    for k, r in ref.items():
        # the oracle differentiates at the fp32 states its forward stores; the
        # float64 forward differs from them by rounding only
        assert _rel(got[k], r) < 2e-5, (k, _rel(got[k], r))


def _loss(c, dy, dM, form):
    M, y = oracle.scan(**c, form=form)
    return float(np.sum(y.astype(np.float64) * dy) + np.sum(M.astype(np.float64) * dM))


@pytest.mark.parametrize("form", [oracle.EQ4, oracle.FIG2], ids=["eq4", "fig2"])
@pytest.mark.parametrize("group", GROUPS)
def test_backward_matches_finite_differences(form, group):
    """Directional derivative along a random direction in one input group vs a
    central difference of the oracle's fp32 forward."""
    c, dy, dM = _case(7, T=16)
    g = oracle.scan_backward(**c, dy=dy, dM_out=dM, form=form)[GRAD_OF[group]].astype(np.float64)
    rng = np.random.default_rng(hash(group) % 1000)
    d = rng.standard_normal(c[group].shape)
    h = 1e-3 * np.max(np.abs(c[group]))
    cp, cm = dict(c), dict(c)
    cp[group] = (c[group] + h * d).astype(np.float32)
    cm[group] = (c[group] - h * d).astype(np.float32)
    # the step actually taken after fp32 rounding of the perturbed inputs
    step = (cp[group].astype(np.float64) - cm[group].astype(np.float64)) / 2
    fd = (_loss(cp, dy, dM, form) - _loss(cm, dy, dM, form)) / 2
    an = float(np.sum(g * step))
    assert abs(fd - an) <= 2e-3 * abs(an) + 1e-6, (group, fd, an)


def test_frozen_table_read_adjoint_is_an_index_add():
    """alpha = 1, beta = 0: the table never changes, so the adjoint of M0 is
    dM_out plus the read weights times dy scattered to the read rows, the read
    weight gradients are <dy_t, M0[j]>, and v and the write weights get exactly
    zero gradient."""
    c, dy, dM = _case(3)
    c["alpha"] = np.ones_like(c["alpha"]); c["beta"] = np.zeros_like(c["beta"])
    for form in (oracle.EQ4, oracle.FIG2):
        g = oracle.scan_backward(**c, dy=dy, dM_out=dM, form=form)
        assert not g["dv"].any() and not g["dwt_w"].any()
        B, H, T, R = c["idx_r"].shape
        for b in range(B):
            for h in range(H):
                ir = torch.from_numpy(c["idx_r"][b, h].reshape(-1).astype(np.int64))
                src = torch.from_numpy((c["wt_r"][b, h][..., None].astype(np.float64)
                                        * dy[b, h][:, None, :]).reshape(T * R, -1))
                ref = torch.from_numpy(dM[b, h].astype(np.float64)).index_add(0, ir, src).numpy()
                assert np.array_equal(g["dM_in"][b, h], ref.astype(np.float32))
                M0 = c["M_in"][b, h].astype(np.float64)
                dr = np.einsum("tc,tqc->tq", dy[b, h].astype(np.float64), M0[c["idx_r"][b, h]])
                assert np.array_equal(g["dwt_r"][b, h], dr.astype(np.float32))


@pytest.mark.parametrize("form", [oracle.EQ4, oracle.FIG2], ids=["eq4", "fig2"])
def test_backward_linear_in_cotangents(form):
    c, dy1, dM1 = _case(11)
    _, dy2, dM2 = _case(12)
    g1 = oracle.scan_backward(**c, dy=dy1, dM_out=dM1, form=form)
    g2 = oracle.scan_backward(**c, dy=dy2, dM_out=dM2, form=form)
    g12 = oracle.scan_backward(**c, dy=dy1 + dy2, dM_out=dM1 + dM2, form=form)
    for k in g1:
        ref = g1[k].astype(np.float64) + g2[k]
        assert _rel(g12[k], ref) < 1e-6, k


@pytest.mark.parametrize("form", [oracle.EQ4, oracle.FIG2], ids=["eq4", "fig2"])
def test_backward_split_into_two_calls(form):
    """Chunk [T1, T) first, from the state at T1, then chunk [0, T1) with the
    first call's state gradient as its final-state gradient: the same as one call."""
    c, dy, dM = _case(13, T=30)
    T1 = 11
    whole = oracle.scan_backward(**c, dy=dy, dM_out=dM, form=form)
    first = {k: (v[:, :, :T1] if k not in ("M_in",) else v) for k, v in c.items()}
    second = {k: (v[:, :, T1:] if k not in ("M_in",) else v) for k, v in c.items()}
    M_T1, _ = oracle.scan(**first, form=form)
    second["M_in"] = M_T1
    g2 = oracle.scan_backward(**second, dy=dy[:, :, T1:], dM_out=dM, form=form)
    g1 = oracle.scan_backward(**first, dy=dy[:, :, :T1], dM_out=g2["dM_in"], form=form)
    for k in ("dv", "dalpha", "dbeta", "dwt_w", "dwt_r"):
        joined = np.concatenate([g1[k], g2[k]], axis=2)
        assert _rel(joined, whole[k].astype(np.float64)) < 1e-6, k
    assert _rel(g1["dM_in"], whole["dM_in"].astype(np.float64)) < 1e-6


def test_single_write_forms_share_all_but_the_write_weight_gradient():
    """W = 1 with weight 1: both forms compute the same forward, so every
    gradient except that of the write weight (through which Fig. 2's shared
    prediction also depends on w) agrees."""
    c, dy, dM = _case(17, W=1)
    c["wt_w"] = np.ones_like(c["wt_w"])
    g4 = oracle.scan_backward(**c, dy=dy, dM_out=dM, form=oracle.EQ4)
    g2 = oracle.scan_backward(**c, dy=dy, dM_out=dM, form=oracle.FIG2)
    for k in ("dv", "dalpha", "dbeta", "dwt_r", "dM_in"):
        assert _rel(g2[k], g4[k].astype(np.float64)) < 1e-6, k
    assert _rel(g2["dwt_w"], g4["dwt_w"].astype(np.float64)) > 1e-3


def test_backward_rejects_bad_indices():
    c, dy, dM = _case(19)
    c["idx_w"] = c["idx_w"].copy()
    c["idx_w"][0, 0, 0, 1] = c["idx_w"][0, 0, 0, 0]
    with pytest.raises(ValueError):
        oracle.scan_backward(**c, dy=dy, dM_out=dM)
