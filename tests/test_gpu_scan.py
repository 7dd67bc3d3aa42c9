"""GPU parity of the sparse gated delta scan against the CPU oracle, through the C ABI.

Both sides receive identical indices, weights, gates, values and initial table
(bit for bit), so y and the final table must agree to fp32 rounding; rows no
token writes must stay bit-identical to M0.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_memory_linear_amd as sdm
from sparse_memory_linear_amd import inputs
from parity import TOL_BF16, TOL_F32, TOL_SAME_INPUTS, compare_slots, max_rel_err, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
FORMS = [("eq4", oracle.EQ4), ("fig2", oracle.FIG2)]


def _run_gpu(idx_w, wt_w, idx_r, wt_r, alpha, beta, v, M_in, form):
    t = lambda a, dt=None: (a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a))).to(DEV)
    M = t(M_in).float().contiguous().clone()
    y = sdm.sdm_scan_forward(t(idx_w).int(), t(wt_w).float(), t(idx_r).int(), t(wt_r).float(),
                             t(alpha).float(), t(beta).float(), t(v), M, form)
    torch.cuda.synchronize()
    return M.cpu().numpy(), y.cpu().numpy()


def _check(name, Mg, yg, Mo, yo, M_in, idx_w, tol, tight=None):
    """tight: a second, smaller bound asserted where both sides scan identical
    inputs (only fp32 rounding order differs); the result is reported against tol."""
    ey, em = max_rel_err(yg, yo), max_rel_err(Mg, Mo)
    say(f"  {name}: max rel err y {ey:.2e}, M {em:.2e} (tolerance {tol:g}"
        + (f", asserted {tight:g})" if tight is not None else ")"))
    assert ey <= tol and em <= tol
    if tight is not None:
        assert ey <= tight and em <= tight
    # rows never selected for writing are bit-identical to the initial table
    M_in = np.asarray(M_in)
    iw = np.asarray(idx_w)
    B, H = iw.shape[:2]
    for b in range(B):
        for h in range(H):
            written = np.zeros(M_in.shape[2], bool)
            written[iw[b, h].reshape(-1)] = True
            assert np.array_equal(Mg[b, h, ~written].view(np.uint32), M_in[b, h, ~written].view(np.uint32))


CASES = [("tiny", {}), ("tiny_dense", {}), ("small", {}),
         ("gdn_matched", dict(B=1, H=2, T=1000)), ("long_context", dict(H=2, T=3000)),
         ("large_table", dict(T=1500))]


_ADDR = {}


def _oracle_inputs(name, over):
    key = (name, tuple(sorted(over.items())))
    if key not in _ADDR:
        wl = inputs.get(name, **over)
        x = inputs.make_inputs(wl)
        iw, ww, _, _ = oracle.address(x["q_w"], x["subkeys"], wl.W)
        ir, wr, _, _ = oracle.address(x["q_r"], x["subkeys"], wl.R)
        _ADDR.clear()
        _ADDR[key] = (wl, x, iw, ww, ir, wr)
    return _ADDR[key]


@pytest.mark.parametrize("name,over", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("form,oform", FORMS, ids=["eq4", "fig2"])
def test_scan_matches_oracle(name, over, form, oform):
    say(f"[scan] {name} {over} form={form}")
    wl, x, iw, ww, ir, wr = _oracle_inputs(name, over)
    M_in = oracle.broadcast_state(x["M0"], wl.B)
    Mo, yo = oracle.scan(iw, ww, ir, wr, x["alpha"], x["beta"], x["v"], M_in, oform)
    Mg, yg = _run_gpu(iw, ww, ir, wr, x["alpha"], x["beta"], x["v"], M_in, form)
    _check(name, Mg, yg, Mo, yo, M_in, iw, TOL_BF16 if wl.bf16_inputs else TOL_F32)


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
    M0 = (rng.standard_normal((B, H, N, dv)) * 0.02).astype(np.float32)
    return dict(idx_w=iw, wt_w=ww, idx_r=ir, wt_r=wr, alpha=a, beta=b, v=v, M_in=M0)


HAZARD = [  # small tables: rows are rewritten by nearby tokens all the time
    dict(B=1, H=3, T=700, N=256, dv=128, W=64, R=64, bf16=True),   # 64-slot sets in 256 rows
    dict(B=2, H=1, T=400, N=64, dv=32, W=16, R=16),                  # every other token overlaps
    dict(B=1, H=1, T=300, N=16, dv=512, W=8, R=8),
    dict(B=1, H=2, T=500, N=300, dv=16, W=200, R=256),              # wide sets, one slab
]


@pytest.mark.parametrize("case", HAZARD, ids=[f"N{c['N']}W{c['W']}dv{c['dv']}" for c in HAZARD])
@pytest.mark.parametrize("form,oform", FORMS, ids=["eq4", "fig2"])
def test_scan_hazard_stress(case, form, oform):
    """Heavy row reuse: read-after-write within a token and across every
    prefetch distance must be forwarded correctly."""
    say(f"[scan hazards] {case} form={form}")
    c = _random_case(1, **case)
    Mo, yo = oracle.scan(**c, form=oform)
    Mg, yg = _run_gpu(**c, form=form)
    _check("hazard", Mg, yg, Mo, yo, c["M_in"], c["idx_w"], TOL_F32)


# (slab width, row partitions) forced through the library's tuning variables;
# every form of the launch must give the oracle's result
SWEEP = [(32, 1), (32, 2), (32, 4), (32, 8), (16, 2), (16, 8), (8, 4), (4, 8)]


@pytest.mark.parametrize("slab,parts", SWEEP, ids=[f"S{s}P{p}" for s, p in SWEEP])
def test_scan_slabs_and_row_partitions_match_oracle(slab, parts, monkeypatch):
    monkeypatch.setenv("SDM_SCAN_SLAB", str(slab))
    monkeypatch.setenv("SDM_SCAN_PARTS", str(parts))
    say(f"[scan slab/partitions] S={slab} P={parts}")
    for case in (HAZARD[0], dict(B=2, H=1, T=300, N=64, dv=32, W=16, R=16), dict(B=1, H=2, T=77, N=4096, dv=64, W=64, R=32)):
        if case["dv"] % slab:
            continue
        c = _random_case(7, **case)
        Mo, yo = oracle.scan(**c, form=oracle.EQ4)
        Mg, yg = _run_gpu(**c, form="eq4")
        _check(f"S={slab} P={parts} N={case['N']}", Mg, yg, Mo, yo, c["M_in"], c["idx_w"], TOL_F32)
        M2, y2 = _run_gpu(**c, form="eq4")
        assert np.array_equal(M2, Mg) and np.array_equal(y2, yg)       # bit-exact rerun


# Who adds the reader wavefronts' partial sums of a token and stores y:
# reader 0 when every reader runs, the last reader when the planner's counts
# leave it idle, an added wavefront when the layout has one reader wavefront
# and room for another, reader 0 again when it has no room.
SUMMERS = [
    ("reader0_all_run", 32, 1, dict(B=1, H=2, T=200, N=4096, dv=64, W=64, R=64)),
    ("idle_last_reader", 32, 4, dict(B=1, H=2, T=200, N=4096, dv=64, W=64, R=64)),
    ("added_wavefront", 16, 1, dict(B=2, H=1, T=300, N=512, dv=64, W=16, R=16)),
    ("added_wavefront_partitioned", 16, 4, dict(B=2, H=1, T=300, N=512, dv=64, W=16, R=16)),
    ("one_reader_no_room", 16, 1, dict(B=1, H=1, T=200, N=1024, dv=64, W=112, R=16)),
]


@pytest.mark.parametrize("label,slab,parts,case", SUMMERS, ids=[c[0] for c in SUMMERS])
def test_partial_sum_wavefront_arrangements(label, slab, parts, case, monkeypatch):
    monkeypatch.setenv("SDM_SCAN_SLAB", str(slab))
    monkeypatch.setenv("SDM_SCAN_PARTS", str(parts))
    say(f"[partial sums] {label} S={slab} P={parts}")
    c = _random_case(11, **case)
    Mo, yo = oracle.scan(**c, form=oracle.EQ4)
    Mg, yg = _run_gpu(**c, form="eq4")
    _check(label, Mg, yg, Mo, yo, c["M_in"], c["idx_w"], TOL_F32)
    M2, y2 = _run_gpu(**c, form="eq4")
    assert np.array_equal(M2, Mg) and np.array_equal(y2, yg)


def test_wide_writer_sets_take_a_slab_whose_ring_fits_lds():
    # W = 120 with 32 streams: the 32-column layout fits 16 wavefronts but its
    # forwarding ring would need 210 KiB of LDS; the rule must pick a narrower
    # slab (and the call must succeed) for both forms
    c = _random_case(13, B=4, H=8, T=40, N=2048, dv=128, W=120, R=8)
    for form, oform in FORMS:
        say(f"[wide W] form={form}")
        Mo, yo = oracle.scan(**c, form=oform)
        Mg, yg = _run_gpu(**c, form=form)
        _check(f"W=120 {form}", Mg, yg, Mo, yo, c["M_in"], c["idx_w"], TOL_F32)


@pytest.mark.parametrize("case", HAZARD + [dict(B=2, H=2, T=130, N=4096, dv=64, W=64, R=32, bf16=True)],
                         ids=[f"N{c['N']}W{c['W']}dv{c['dv']}" for c in HAZARD] + ["N4096W64dv64"])
@pytest.mark.parametrize("form,oform", FORMS, ids=["eq4", "fig2"])
def test_direct_short_scan_matches_oracle(case, form, oform, monkeypatch):
    """The planner-free form used for short calls, forced for whole sequences:
    every token's loads follow the previous token's barrier, so heavy row
    reuse must still give the oracle's result."""
    monkeypatch.setenv("SDM_SCAN_DIRECT_T", "100000")
    say(f"[scan direct] {case} form={form}")
    c = _random_case(5, **case)
    Mo, yo = oracle.scan(**c, form=oform)
    Mg, yg = _run_gpu(**c, form=form)
    _check("direct", Mg, yg, Mo, yo, c["M_in"], c["idx_w"], TOL_F32)


@pytest.mark.parametrize("overlap", ["all", "half"])
@pytest.mark.parametrize("form,oform", FORMS, ids=["eq4", "fig2"])
def test_direct_reads_of_rows_the_token_writes(overlap, form, oform, monkeypatch):
    """Direct form with reads on the rows the same token writes: every read
    (read set a permutation of the write set) or half of them. The reader
    loads its row with the writers, before they store, so each such read must
    take the token's new row from the writers instead (read-after-write within
    a token, SDM notes §2.4)."""
    monkeypatch.setenv("SDM_SCAN_DIRECT_T", "100000")
    say(f"[scan direct, reads on written rows] overlap={overlap} form={form}")
    rng = np.random.default_rng(11)
    c = _random_case(12, B=2, H=2, T=60, N=512, dv=64, W=32, R=32)
    B, H, T, W = c["idx_w"].shape
    for b in range(B):
        for h in range(H):
            for t in range(T):
                w = c["idx_w"][b, h, t]
                if overlap == "all":
                    c["idx_r"][b, h, t] = rng.permutation(w)
                else:
                    others = np.setdiff1d(np.arange(512), w)
                    c["idx_r"][b, h, t] = rng.permutation(np.concatenate([w[:16], rng.choice(others, 16, False)]))
    Mo, yo = oracle.scan(**c, form=oform)
    Mg, yg = _run_gpu(**c, form=form)
    _check("direct read-on-write", Mg, yg, Mo, yo, c["M_in"], c["idx_w"], TOL_F32)


@pytest.mark.parametrize("B,H", [(5, 1), (7, 1), (3, 3), (3, 4)], ids=["NS5", "NS7", "NS9", "NS12"])
@pytest.mark.parametrize("form,oform", FORMS, ids=["eq4", "fig2"])
def test_stream_counts_around_one_round_of_xcds(B, H, form, oform):
    """Fewer than 8 streams deal each stream's workgroups over all XCDs; 8 or
    more keep a stream on one XCD and round the grid up to whole rounds of 8:
    stream counts on both sides of that boundary, every stream checked, for the
    pipelined scan and the direct short-call form."""
    say(f"[scan streams] B={B} H={H} form={form}")
    c = _random_case(23, B=B, H=H, T=120, N=512, dv=64, W=16, R=16)
    Mo, yo = oracle.scan(**c, form=oform)
    Mg, yg = _run_gpu(**c, form=form)
    _check(f"NS={B * H}", Mg, yg, Mo, yo, c["M_in"], c["idx_w"], TOL_F32)
    c2 = {k: v if k == "M_in" else (v[:, :, :6].contiguous() if isinstance(v, torch.Tensor) else
                                     np.ascontiguousarray(v[:, :, :6])) for k, v in c.items()}
    Mo2, yo2 = oracle.scan(**c2, form=oform)
    Mg2, yg2 = _run_gpu(**c2, form=form)   # 6 tokens: the direct form
    _check(f"NS={B * H} direct", Mg2, yg2, Mo2, yo2, c2["M_in"], c2["idx_w"], TOL_F32)


def test_decode_one_token_per_call_matches_one_scan():
    """Decoding: T = 1 per call, the table carried between calls, equals the
    oracle's scan over the whole sequence."""
    c = _random_case(9, B=8, H=2, T=40, N=4096, dv=64, W=16, R=16, bf16=True)
    Mo, yo = oracle.scan(**c, form=oracle.EQ4)
    t = lambda a: (a if isinstance(a, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(a))).to(DEV)
    M = t(c["M_in"]).float().contiguous().clone()
    ys = []
    for k in range(40):
        sl = lambda a: t(a)[:, :, k:k + 1].contiguous()
        ys.append(sdm.sdm_scan_forward(sl(c["idx_w"]).int(), sl(c["wt_w"]).float(), sl(c["idx_r"]).int(),
                                       sl(c["wt_r"]).float(), sl(c["alpha"]).float(), sl(c["beta"]).float(),
                                       sl(c["v"]), M, "eq4"))
    torch.cuda.synchronize()
    yg = torch.cat(ys, 2).cpu().numpy()
    _check("decode", M.cpu().numpy(), yg, Mo, yo, c["M_in"], c["idx_w"], TOL_F32)


@pytest.mark.parametrize("T", [1, 2, 5, 6, 7, 10, 11, 13, 61])
def test_scan_short_and_ragged_sequences(T):
    say(f"[scan ragged] T={T}")
    for case in (dict(B=3, H=1, N=128, dv=128, W=64, R=64), dict(B=1, H=5, N=64, dv=64, W=16, R=16)):
        c = _random_case(T, T=T, **case)
        for form, oform in FORMS:
            Mo, yo = oracle.scan(**c, form=oform)
            Mg, yg = _run_gpu(**c, form=form)
            _check(f"T={T} {form}", Mg, yg, Mo, yo, c["M_in"], c["idx_w"], TOL_F32)


def test_scan_empty_sequence_is_a_no_op():
    c = _random_case(0, B=1, H=1, T=1, N=64, dv=16, W=4, R=4)
    z = {k: (v[:, :, :0] if k != "M_in" else v) for k, v in c.items()}
    Mg, yg = _run_gpu(**z, form="eq4")
    assert yg.shape == (1, 1, 0, 16) and np.array_equal(Mg, c["M_in"])


def test_scan_deterministic_split_and_column_permutation():
    c = _random_case(3, B=2, H=2, T=500, N=512, dv=128, W=64, R=64, bf16=True)
    for form in ("eq4", "fig2"):
        M1, y1 = _run_gpu(**c, form=form)
        M2, y2 = _run_gpu(**c, form=form)
        assert np.array_equal(M1, M2) and np.array_equal(y1, y2)          # bit-exact rerun
        t1 = 211
        first = {k: (v[:, :, :t1] if k != "M_in" else v) for k, v in c.items()}
        Ma, ya = _run_gpu(**first, form=form)
        second = {k: (v[:, :, t1:] if k != "M_in" else Ma) for k, v in c.items()}
        Mb, yb = _run_gpu(**second, form=form)
        assert np.array_equal(Mb, M1) and np.array_equal(np.concatenate([ya, yb], 2), y1)
        perm = np.random.default_rng(0).permutation(128)
        cp = dict(c); cp["v"] = c["v"][..., torch.from_numpy(perm)].contiguous()
        cp["M_in"] = np.ascontiguousarray(c["M_in"][..., perm])
        Mp, yp = _run_gpu(**cp, form=form)
        assert np.array_equal(Mp, M1[..., perm]) and np.array_equal(yp, y1[..., perm])


def test_state_init_broadcasts_M0():
    M0 = torch.randn(3, 1000, 64)
    M = sdm.sdm_state_init(M0.to(DEV), 5).cpu()
    assert all(torch.equal(M[b], M0) for b in range(5))


FULL = [("gdn_matched", "eq4", [(0, 0), (1, 3), (2, 5), (3, 7)]), ("gdn_matched", "fig2", [(0, 2), (3, 6)]),
        ("long_context", "eq4", [(0, 5), (0, 2)])]


@pytest.mark.parametrize("name,form,streams", FULL, ids=[f"{n}-{f}" for n, f, _ in FULL])
def test_full_pipeline_full_size_sampled_streams(name, form, streams):
    """The whole hot path at full size, in the benchmark's launch configuration
    (state init, addressing, scan). The sampled (b, h) streams take the oracle's
    own slots and weights (written over the GPU's before the scan), so both
    sides scan identical inputs that come from the oracle; those streams are
    checked in full against the oracle scan, to the workload's tolerance and to
    the fp32-rounding bound of identical inputs."""
    wl = inputs.get(name)
    say(f"[pipeline full size] {name} {form} B={wl.B} H={wl.H} T={wl.T} streams={streams}")
    x = inputs.make_inputs(wl)
    g = {k: v.to(DEV) for k, v in x.items()}
    iw, ww, ir, wr = sdm.sdm_address(g["q_w"], g["q_r"], g["subkeys"], g["subkeys"], wl.W, wl.R)
    orc = {}
    for (b, h) in streams:
        q = lambda k: x[k][b:b + 1, h:h + 1]
        oi, ow, _, _ = oracle.address(q("q_w"), x["subkeys"][h:h + 1], wl.W)
        ri, rw, _, _ = oracle.address(q("q_r"), x["subkeys"][h:h + 1], wl.R)
        orc[(b, h)] = (oi, ow, ri, rw)
        for dst, src in ((iw, oi), (ww, ow), (ir, ri), (wr, rw)):
            dst[b, h] = torch.from_numpy(src[0, 0]).to(DEV)
    M = sdm.sdm_state_init(g["M0"], wl.B)
    y = sdm.sdm_scan_forward(iw, ww, ir, wr, g["alpha"], g["beta"], g["v"], M, form)
    torch.cuda.synchronize()
    for (b, h) in streams:
        sl = lambda t: t[b:b + 1, h:h + 1].cpu()
        oi, ow, ri, rw = orc[(b, h)]
        Mo, yo = oracle.scan(oi, ow, ri, rw, sl(x["alpha"]), sl(x["beta"]), sl(x["v"]),
                             x["M0"][h:h + 1][None].numpy(), oracle.EQ4 if form == "eq4" else oracle.FIG2)
        _check(f"stream ({b},{h})", sl(M).numpy(), sl(y).numpy(), Mo, yo,
               x["M0"][h:h + 1][None].numpy(), oi, TOL_BF16, TOL_SAME_INPUTS)


@pytest.mark.parametrize("form,oform", FORMS, ids=["eq4", "fig2"])
def test_large_table_full_size(form, oform):
    """The FwPKM-sized workload at full size (one stream, T=65536, N=262144,
    d_v=512, W=R=8, fp32): GPU addressing end to end against the oracle (near-
    tie accounting), then both scans fed the oracle's slots, the whole y and
    table checked."""
    wl = inputs.get("large_table")
    say(f"[large_table full size] T={wl.T} N={wl.N} d_v={wl.d_v} form={form}")
    x = inputs.make_inputs(wl)
    g = {k: v.to(DEV) for k, v in x.items()}
    iw, ww, ir, wr = sdm.sdm_address(g["q_w"], g["q_r"], g["subkeys"], g["subkeys"], wl.W, wl.R)
    hw, hr = oracle.half_scores(x["q_w"], x["subkeys"]), oracle.half_scores(x["q_r"], x["subkeys"])
    oiw, oww, osw, onw = oracle.select(hw, wl.W)
    oir, owr, osr, onr = oracle.select(hr, wl.R)
    if form == "eq4":  # the addressing does not depend on the form: account for it once
        for br, gi, oi, osc, onx, oh in (("write", iw, oiw, osw, onw, hw), ("read", ir, oir, osr, onr, hr)):
            res = compare_slots(gi.cpu().numpy(), oi, osc, onx, oh, label=f"dot large_table full size {br}")
            say(f"  slots: {res}")
            assert res["violating"] == 0
    M_in = oracle.broadcast_state(x["M0"], wl.B)
    Mo, yo = oracle.scan(oiw, oww, oir, owr, x["alpha"], x["beta"], x["v"], M_in, oform)
    Mg, yg = _run_gpu(oiw, oww, oir, owr, x["alpha"], x["beta"], x["v"], M_in, form)
    _check("large_table", Mg, yg, Mo, yo, M_in, oiw, TOL_F32, TOL_SAME_INPUTS)
