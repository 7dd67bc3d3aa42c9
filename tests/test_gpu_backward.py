"""GPU parity of the training path (forward with pre-images, backward that
undoes it) against the CPU oracle's backward, through the C ABI.

Both sides get the same indices, weights, gates, values, initial table and
cotangents (dy, dL/dM of the final state). The oracle differentiates the
recurrence in double at the fp32 states its forward stores; the GPU keeps the
adjoint table in fp32. The undo must give back the initial table bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_memory_linear_amd as sdm
from sparse_memory_linear_amd import inputs
from parity import TOL_BF16, TOL_F32, TOL_SAME_INPUTS, max_rel_err, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
FORMS = [("eq4", oracle.EQ4), ("fig2", oracle.FIG2)]
GRADS = ("dv", "dalpha", "dbeta", "dwt_w", "dwt_r")


def _t(a):
    return (a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a))).to(DEV)


def _cotangents(seed, B, H, T, N, dv):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn((B, H, T, dv), generator=g).numpy(),
            torch.randn((B, H, N, dv), generator=g).numpy() * 0.1)


def _gpu_train(c, dy, dM_out, form):
    """forward_save then backward on the GPU; returns the forward's (M, y, snap),
    the gradients, the restored table and dL/dM of the initial state."""
    a = {k: _t(v) for k, v in c.items()}
    M = a["M_in"].float().contiguous().clone()
    args = (a["idx_w"].int(), a["wt_w"].float(), a["idx_r"].int(), a["wt_r"].float(),
            a["alpha"].float(), a["beta"].float(), a["v"])
    y, snap = sdm.sdm_scan_forward_save(*args, M, form)
    M_after = M.clone()
    dM = _t(dM_out).float().contiguous().clone()
    g = sdm.sdm_scan_backward(*args, snap, _t(dy).float().contiguous(), M, dM, form)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in g.items()}
    out["dM_in"] = dM.cpu().numpy()
    return M_after.cpu().numpy(), y.cpu().numpy(), snap, out, M.cpu().numpy()


def _check_grads(name, got, ref, tol, tight=None):
    """tight: a second, smaller bound asserted where both sides take identical
    inputs (only fp32 rounding order differs); the result is reported against tol."""
    errs = {k: max_rel_err(got[k], ref[k]) for k in GRADS + ("dM_in",)}
    say(f"  {name}: " + ", ".join(f"{k} {e:.1e}" for k, e in errs.items())
        + f" (tolerance {tol:g}" + (f", asserted {tight:g})" if tight is not None else ")"))
    for k, e in errs.items():
        assert e <= tol, (k, e)
        if tight is not None:
            assert e <= tight, (k, e)


def _oracle_case(name, over):
    wl = inputs.get(name, **over)
    x = inputs.make_inputs(wl)
    iw, ww, _, _ = oracle.address(x["q_w"], x["subkeys"], wl.W)
    ir, wr, _, _ = oracle.address(x["q_r"], x["subkeys"], wl.R)
    c = dict(idx_w=iw, wt_w=ww, idx_r=ir, wt_r=wr, alpha=x["alpha"].numpy(), beta=x["beta"].numpy(),
             v=x["v"], M_in=oracle.broadcast_state(x["M0"], wl.B))
    return wl, c


CASES = [("tiny", {}), ("small", dict(T=600)), ("gdn_matched", dict(B=1, H=2, T=400)),
         ("long_context", dict(H=2, T=800)), ("large_table", dict(T=200))]


@pytest.mark.parametrize("name,over", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("form,oform", FORMS, ids=["eq4", "fig2"])
def test_backward_matches_oracle(name, over, form, oform):
    say(f"[backward] {name} {over} form={form}")
    wl, c = _oracle_case(name, over)
    dy, dM = _cotangents(1, wl.B, wl.H, wl.T, wl.N, wl.d_v)
    ref = oracle.scan_backward(**c, dy=dy, dM_out=dM, form=oform)
    _, _, _, got, M_back = _gpu_train(c, dy, dM, form)
    _check_grads(name, got, ref, TOL_BF16 if wl.bf16_inputs else TOL_F32)
    # the undo restores the initial table bit for bit
    assert np.array_equal(M_back.view(np.uint32), np.asarray(c["M_in"], np.float32).view(np.uint32))


def _random_case(seed, B, H, T, N, dv, W, R, bf16=False):
    rng = np.random.default_rng(seed)
    iw = np.stack([rng.permutation(N)[:W] for _ in range(B * H * T)]).reshape(B, H, T, W).astype(np.int32)
    ir = np.stack([rng.permutation(N)[:R] for _ in range(B * H * T)]).reshape(B, H, T, R).astype(np.int32)
    ww = rng.dirichlet(np.ones(W), size=(B, H, T)).astype(np.float32)
    wr = rng.dirichlet(np.ones(R), size=(B, H, T)).astype(np.float32)
    a = (1 / (1 + np.exp(-rng.normal(2, .5, (B, H, T))))).astype(np.float32)
    b = (1 / (1 + np.exp(-rng.normal(0, 1, (B, H, T))))).astype(np.float32)
    v = torch.from_numpy(rng.standard_normal((B, H, T, dv)).astype(np.float32))
    if bf16:
        v = v.to(torch.bfloat16)
    M0 = (rng.standard_normal((B, H, N, dv)) * 0.5).astype(np.float32)
    return dict(idx_w=iw, wt_w=ww, idx_r=ir, wt_r=wr, alpha=a, beta=b, v=v, M_in=M0)


HAZARD = [  # small tables: rows written and read by nearby tokens and by the same token
    dict(B=1, H=3, T=300, N=256, dv=128, W=64, R=64, bf16=True),
    dict(B=2, H=1, T=400, N=64, dv=32, W=16, R=16),
    dict(B=1, H=1, T=300, N=16, dv=512, W=8, R=8),
    dict(B=1, H=2, T=200, N=300, dv=16, W=200, R=256),
]


@pytest.mark.parametrize("case", HAZARD, ids=[f"N{c['N']}W{c['W']}dv{c['dv']}" for c in HAZARD])
@pytest.mark.parametrize("form,oform", FORMS, ids=["eq4", "fig2"])
def test_backward_hazard_stress(case, form, oform):
    say(f"[backward hazards] {case} form={form}")
    c = _random_case(2, **case)
    dy, dM = _cotangents(3, case["B"], case["H"], case["T"], case["N"], case["dv"])
    ref = oracle.scan_backward(**c, dy=dy, dM_out=dM, form=oform)
    _, _, _, got, M_back = _gpu_train(c, dy, dM, form)
    _check_grads("hazard", got, ref, TOL_F32)
    assert np.array_equal(M_back.view(np.uint32), c["M_in"].view(np.uint32))


BWD_SWEEP = [("eq4", 32, 1), ("eq4", 32, 2), ("eq4", 32, 4), ("eq4", 32, 16), ("eq4", 16, 8), ("eq4", 8, 2),
             ("eq4", 4, 1), ("fig2", 32, 1), ("fig2", 16, 1), ("fig2", 8, 1), ("fig2", 4, 1)]


@pytest.mark.parametrize("form,slab,parts", BWD_SWEEP, ids=[f"{f}-S{s}P{p}" for f, s, p in BWD_SWEEP])
def test_backward_slabs_and_row_partitions(form, slab, parts, monkeypatch):
    monkeypatch.setenv("SDM_BWD_SLAB", str(slab))
    monkeypatch.setenv("SDM_BWD_PARTS", str(parts))
    oform = oracle.EQ4 if form == "eq4" else oracle.FIG2
    case = dict(B=1, H=2, T=250, N=4096, dv=128, W=64, R=64, bf16=True)
    say(f"[backward S={slab} P={parts}] form={form}")
    c = _random_case(4, **case)
    dy, dM = _cotangents(5, 1, 2, 250, 4096, 128)
    ref = oracle.scan_backward(**c, dy=dy, dM_out=dM, form=oform)
    _, _, _, got, M_back = _gpu_train(c, dy, dM, form)
    _check_grads(f"S{slab}P{parts}", got, ref, TOL_F32)
    assert np.array_equal(M_back.view(np.uint32), c["M_in"].view(np.uint32))


SAVE_CFG = [("eq4", 0), ("eq4", 1), ("eq4", 2), ("fig2", 0)]


@pytest.mark.parametrize("form,parts", SAVE_CFG, ids=[f"{f}-P{p or 'auto'}" for f, p in SAVE_CFG])
def test_forward_save_table_and_pre_images(form, parts, monkeypatch):
    """The training forward's table equals sdm_scan_forward's bit for bit, its
    y agrees to rounding, and every stored row is the oracle's table row before
    that token's write (row partitions: the default 8, forced 1 and 2)."""
    if parts:
        monkeypatch.setenv("SDM_SCAN_PARTS", str(parts))
    oform = oracle.EQ4 if form == "eq4" else oracle.FIG2
    c = _random_case(6, B=1, H=2, T=48, N=128, dv=32, W=16, R=8)
    a = {k: _t(v) for k, v in c.items()}
    args = (a["idx_w"], a["wt_w"], a["idx_r"], a["wt_r"], a["alpha"], a["beta"], a["v"])
    M1 = a["M_in"].clone()
    y1 = sdm.sdm_scan_forward(*args, M1, form)
    M2 = a["M_in"].clone()
    y2, snap = sdm.sdm_scan_forward_save(*args, M2, form)
    torch.cuda.synchronize()
    assert torch.equal(M1, M2)
    assert max_rel_err(y2.cpu().numpy(), y1.cpu().numpy()) <= 1e-6
    # the oracle's table before each token
    B, H, T, W = c["idx_w"].shape
    Mo = c["M_in"].copy()
    pre = np.empty((B, H, T, W, Mo.shape[-1]), np.float32)
    for t in range(T):
        for b in range(B):
            for h in range(H):
                pre[b, h, t] = Mo[b, h, c["idx_w"][b, h, t]]
        step = {k: (v[:, :, t:t + 1] if k != "M_in" else Mo) for k, v in c.items()}
        Mo, _ = oracle.scan(**step, form=oform)
    e = max_rel_err(snap.cpu().numpy(), pre)
    say(f"  pre-images vs oracle: {e:.1e}")
    assert e <= TOL_F32


@pytest.mark.parametrize("form", ["eq4", "fig2"])
def test_backward_of_two_calls_equals_one(form):
    """A sequence split into two forward calls, differentiated last call first
    with M and dM passed along: the same bits as one call."""
    c = _random_case(7, B=2, H=2, T=300, N=512, dv=64, W=32, R=32)
    dy, dM_out = _cotangents(8, 2, 2, 300, 512, 64)
    _, _, _, one, M_one = _gpu_train(c, dy, dM_out, form)
    a = {k: _t(v) for k, v in c.items()}
    T1 = 123
    part = lambda lo, hi: tuple(a[k][:, :, lo:hi].contiguous() for k in
                                ("idx_w", "wt_w", "idx_r", "wt_r", "alpha", "beta", "v"))
    M = a["M_in"].clone()
    _, s1 = sdm.sdm_scan_forward_save(*part(0, T1), M, form)
    _, s2 = sdm.sdm_scan_forward_save(*part(T1, 300), M, form)
    dM = _t(dM_out).clone()
    dyt = _t(dy)
    g2 = sdm.sdm_scan_backward(*part(T1, 300), s2, dyt[:, :, T1:].contiguous(), M, dM, form)
    g1 = sdm.sdm_scan_backward(*part(0, T1), s1, dyt[:, :, :T1].contiguous(), M, dM, form)
    torch.cuda.synchronize()
    for k in GRADS:
        joined = torch.cat([g1[k], g2[k]], dim=2).cpu().numpy()
        assert np.array_equal(joined, one[k]), k
    assert np.array_equal(dM.cpu().numpy(), one["dM_in"])
    assert np.array_equal(M.cpu().numpy(), M_one)


def test_backward_short_and_ragged_calls():
    for T in (1, 2, 7, 33):
        c = _random_case(9 + T, B=3, H=2, T=T, N=1024, dv=64, W=32, R=16)
        dy, dM = _cotangents(T, 3, 2, T, 1024, 64)
        for form, oform in FORMS:
            say(f"[backward short] T={T} form={form}")
            ref = oracle.scan_backward(**c, dy=dy, dM_out=dM, form=oform)
            _, _, _, got, M_back = _gpu_train(c, dy, dM, form)
            _check_grads(f"T{T}", got, ref, TOL_F32)
            assert np.array_equal(M_back, c["M_in"])


def test_backward_empty_call_is_a_no_op():
    z = lambda *shape, dt=torch.float32: torch.zeros(shape, dtype=dt, device=DEV)
    M = torch.randn((1, 1, 64, 16), device=DEV)
    M_in = M.clone()
    dM = torch.ones_like(M)
    g = sdm.sdm_scan_backward(z(1, 1, 0, 4, dt=torch.int32), z(1, 1, 0, 4), z(1, 1, 0, 4, dt=torch.int32),
                              z(1, 1, 0, 4), z(1, 1, 0), z(1, 1, 0), z(1, 1, 0, 16), z(1, 1, 0, 4, 16),
                              z(1, 1, 0, 16), M, dM)
    torch.cuda.synchronize()
    assert all(t.numel() == 0 for t in g.values())
    assert torch.equal(M, M_in) and torch.equal(dM, torch.ones_like(M))


def test_state_init_backward_sums_sequences():
    g = torch.Generator().manual_seed(12)
    dM = torch.randn((5, 3, 700, 64), generator=g)
    got = sdm.sdm_state_init_backward(dM.to(DEV)).cpu()
    ref = dM.double().sum(0)
    assert max_rel_err(got.numpy(), ref.numpy()) <= 1e-6


def test_backward_full_size_sampled_streams():
    """gdn_matched at full size in the benchmark's launch configuration (all 32
    streams, one forward_save and one backward call); two streams take the
    oracle's own slots and weights and are checked in full against the oracle."""
    wl = inputs.get("gdn_matched")
    streams = [(0, 0), (3, 6)]
    say(f"[backward full size] gdn_matched B={wl.B} H={wl.H} T={wl.T} streams={streams}")
    x = inputs.make_inputs(wl)
    g = {k: v.to(DEV) for k, v in x.items()}
    iw, ww, ir, wr = sdm.sdm_address(g["q_w"], g["q_r"], g["subkeys"], g["subkeys"], wl.W, wl.R)
    orc = {}
    for (b, h) in streams:
        q = lambda k: x[k][b:b + 1, h:h + 1]
        sub = x["subkeys"][h:h + 1]
        oi, ow, _, _ = oracle.address(q("q_w"), sub, wl.W)
        ri, rw, _, _ = oracle.address(q("q_r"), sub, wl.R)
        orc[(b, h)] = (oi, ow, ri, rw)
        iw[b, h] = _t(oi[0, 0]); ww[b, h] = _t(ow[0, 0]); ir[b, h] = _t(ri[0, 0]); wr[b, h] = _t(rw[0, 0])
    dy, dM_out = _cotangents(13, wl.B, wl.H, wl.T, wl.N, wl.d_v)
    M = sdm.sdm_state_init(g["M0"], wl.B)
    args = (iw, ww, ir, wr, g["alpha"], g["beta"], g["v"])
    y, snap = sdm.sdm_scan_forward_save(*args, M, "eq4")
    dM = _t(dM_out)
    grads = sdm.sdm_scan_backward(*args, snap, _t(dy), M, dM, "eq4")
    torch.cuda.synchronize()
    del snap
    for (b, h) in streams:
        oi, ow, ri, rw = orc[(b, h)]
        sl = lambda t: t[b:b + 1, h:h + 1]
        M0 = x["M0"][h:h + 1][None].numpy()
        ref = oracle.scan_backward(oi, ow, ri, rw, sl(x["alpha"]), sl(x["beta"]), sl(x["v"]), M0,
                                   sl(dy), sl(dM_out), form=oracle.EQ4)
        got = {k: sl(v).cpu().numpy() for k, v in grads.items()}
        got["dM_in"] = sl(dM).cpu().numpy()
        _check_grads(f"stream ({b},{h})", got, ref, TOL_BF16, TOL_SAME_INPUTS)
        assert np.array_equal(sl(M).cpu().numpy(), M0)


@pytest.mark.parametrize("B,H", [(5, 1), (7, 1), (3, 3), (3, 4)], ids=["NS5", "NS7", "NS9", "NS12"])
@pytest.mark.parametrize("form,oform", [("eq4", oracle.EQ4), ("fig2", oracle.FIG2)], ids=["eq4", "fig2"])
def test_backward_stream_counts_around_one_round_of_xcds(B, H, form, oform):
    """Fewer than 8 streams deal each stream's workgroups over all XCDs; 8 or
    more keep a stream on one XCD and round the grid up to whole rounds of 8:
    stream counts on both sides of that boundary, every stream checked."""
    say(f"[backward streams] B={B} H={H} form={form}")
    case = dict(B=B, H=H, T=90, N=512, dv=64, W=16, R=16)
    c = _random_case(21, **case)
    dy, dM = _cotangents(22, B, H, 90, 512, 64)
    ref = oracle.scan_backward(**c, dy=dy, dM_out=dM, form=oform)
    _, _, _, got, M_back = _gpu_train(c, dy, dM, form)
    _check_grads(f"NS={B * H}", got, ref, TOL_F32)
    assert np.array_equal(M_back.view(np.uint32), c["M_in"].view(np.uint32))


@pytest.mark.parametrize("form,oform", [("eq4", oracle.EQ4), ("fig2", oracle.FIG2)], ids=["eq4", "fig2"])
def test_training_call_split_into_launch_chunks(form, oform):
    """W = 256 write rows of d_v = 512 fp32 values: 512 KiB of pre-images per
    token, so the training forward and the backward each split the call into
    launches of at most 2^31 bytes of pre-images (4095 + 105 tokens); the
    backward walks the chunks last to first and must match the oracle across
    the boundary, with the table restored bit for bit."""
    say(f"[backward launch chunks] W=256 d_v=512 T=4200 form={form}")
    case = dict(B=1, H=1, T=4200, N=2048, dv=512, W=256, R=16)
    c = _random_case(31, **case)
    dy, dM = _cotangents(32, 1, 1, 4200, 2048, 512)
    ref = oracle.scan_backward(**c, dy=dy, dM_out=dM, form=oform)
    _, _, _, got, M_back = _gpu_train(c, dy, dM, form)
    _check_grads(f"chunks {form}", got, ref, TOL_F32)
    assert np.array_equal(M_back.view(np.uint32), c["M_in"].view(np.uint32))


@pytest.mark.parametrize("T", [1, 6])
@pytest.mark.parametrize("form,oform", [("eq4", oracle.EQ4), ("fig2", oracle.FIG2)], ids=["eq4", "fig2"])
def test_training_short_calls(T, form, oform):
    """Calls of at most 8 tokens take the direct form, also for the training
    forward (its pre-image stores); the backward then runs with fewer tokens
    than its unrolled loop holds (its tail loop only). Both against the oracle."""
    say(f"[backward short call] T={T} form={form}")
    c = _random_case(41 + T, B=2, H=3, T=T, N=512, dv=64, W=16, R=16)
    dy, dM = _cotangents(42 + T, 2, 3, T, 512, 64)
    ref = oracle.scan_backward(**c, dy=dy, dM_out=dM, form=oform)
    _, _, _, got, M_back = _gpu_train(c, dy, dM, form)
    _check_grads(f"T={T} {form}", got, ref, TOL_F32)
    assert np.array_equal(M_back.view(np.uint32), c["M_in"].view(np.uint32))


def test_backward_long_context_layout():
    """The long-context shape's backward layout (8 streams: 8-column slabs in 2
    row partitions): with T = 8192 one stream takes the oracle's own slots and
    is checked in full against the oracle; at the full T = 131072 (the launch
    the training bench times) the undo must give back the initial table bit
    for bit on every stream, with finite gradients."""
    for T in (8192, 131072):
        wl = inputs.get("long_context", T=T)
        say(f"[backward long_context layout] B={wl.B} H={wl.H} T={wl.T}")
        x = inputs.make_inputs(wl)
        g = {k: v.to(DEV) for k, v in x.items()}
        iw, ww, ir, wr = sdm.sdm_address(g["q_w"], g["q_r"], g["subkeys"], g["subkeys"], wl.W, wl.R)
        b, h = 0, 5
        if T == 8192:
            q = lambda k: x[k][b:b + 1, h:h + 1]
            oi, ow, _, _ = oracle.address(q("q_w"), x["subkeys"][h:h + 1], wl.W)
            ri, rw, _, _ = oracle.address(q("q_r"), x["subkeys"][h:h + 1], wl.R)
            iw[b, h] = _t(oi[0, 0]); ww[b, h] = _t(ow[0, 0]); ir[b, h] = _t(ri[0, 0]); wr[b, h] = _t(rw[0, 0])
        dy, dM_out = _cotangents(17, wl.B, wl.H, wl.T, wl.N, wl.d_v)
        M = sdm.sdm_state_init(g["M0"], wl.B)
        M_in = M.cpu()
        args = (iw, ww, ir, wr, g["alpha"], g["beta"], g["v"])
        y, snap = sdm.sdm_scan_forward_save(*args, M, "eq4")
        dM = _t(dM_out)
        grads = sdm.sdm_scan_backward(*args, snap, _t(dy), M, dM, "eq4")
        torch.cuda.synchronize()
        del snap, y
        assert torch.equal(M.cpu(), M_in)
        assert all(bool(torch.isfinite(v).all()) for v in grads.values()) and bool(torch.isfinite(dM).all())
        if T == 8192:
            sl = lambda t: t[b:b + 1, h:h + 1]
            ref = oracle.scan_backward(oi, ow, ri, rw, sl(x["alpha"]), sl(x["beta"]), sl(x["v"]),
                                       x["M0"][h:h + 1][None].numpy(), sl(dy), sl(dM_out), form=oracle.EQ4)
            got = {k: sl(v).cpu().numpy() for k, v in grads.items()}
            got["dM_in"] = sl(dM).cpu().numpy()
            _check_grads(f"long_context T={T} stream ({b},{h})", got, ref, TOL_BF16, TOL_SAME_INPUTS)
        del grads, dM, M, g
        torch.cuda.empty_cache()
