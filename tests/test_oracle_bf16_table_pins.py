"""Pins of the oracle's bf16-table variant of the scan.

The SDM notes give the per-layer state as 211 MB for 110.6 M elements (§4.5
Table 3 with the element count of §2.8), i.e. 2-byte table elements. The
variant keeps the recurrence of §2.4 Eq. (3)-(5) / §2.5 Fig. 2 (computed in
double, as the fp32-table oracle does) and rounds every stored element once
to the nearest bfloat16, ties to even. Pinned here against torch's own
bfloat16 rounding, the (separately pinned) fp32-table oracle, an
embedding_bag lookup, and the scan's invariants.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_memory_linear_amd import inputs


def _rand_case(seed, B=1, H=2, T=48, N=64, dv=16, W=4, R=5, beta_scale=1.0):
    rng = np.random.default_rng(seed)
    iw = np.stack([rng.permutation(N)[:W] for _ in range(B * H * T)]).reshape(B, H, T, W).astype(np.int32)
    ir = rng.integers(0, N, (B, H, T, R)).astype(np.int32)
    ww = rng.dirichlet(np.ones(W), (B, H, T)).astype(np.float32)
    wr = rng.dirichlet(np.ones(R), (B, H, T)).astype(np.float32)
    al = (1 / (1 + np.exp(-rng.normal(2, 0.5, (B, H, T))))).astype(np.float32)
    be = (beta_scale / (1 + np.exp(-rng.normal(0, 1, (B, H, T))))).astype(np.float32)
    v = rng.standard_normal((B, H, T, dv)).astype(np.float32)
    M0 = torch.from_numpy(rng.normal(0, 0.5, (B, H, N, dv)).astype(np.float32)).to(torch.bfloat16)
    return iw, ww, ir, wr, al, be, v, M0


def test_full_overwrite_stores_torch_rounding_of_v():
    """beta = 1, one write of weight 1: the row becomes v, rounded to bfloat16
    exactly as torch rounds (nearest, ties to even); the read returns it."""
    rng = np.random.default_rng(0)
    T, dv = 64, 32
    v = rng.standard_normal((1, 1, T, dv)).astype(np.float32)
    # exact ties between two bfloat16 neighbours, below and above even; values
    # below the normal range (bfloat16 subnormals are 2^-133 apart)
    v[0, 0, 0, :6] = [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(2 + 2 ** -7), 2 ** -130, 5 * 2.0 ** -136, -3 * 2.0 ** -134]
    idx = (np.arange(T) % 7).astype(np.int32).reshape(1, 1, T, 1)
    one = np.ones((1, 1, T, 1), np.float32)
    M0 = torch.zeros((1, 1, 8, dv), dtype=torch.bfloat16)
    for form in (oracle.EQ4, oracle.FIG2):
        M, y = oracle.scan_bf16(idx, one, idx, one, np.full((1, 1, T), 0.9, np.float32),
                                np.ones((1, 1, T), np.float32), v, M0, form)
        ref = torch.from_numpy(v).to(torch.bfloat16)
        assert torch.equal(torch.from_numpy(y).to(torch.bfloat16), ref[0:1])
        assert np.array_equal(y, ref.float().numpy())
        for r in range(7):
            last = max(t for t in range(T) if t % 7 == r)
            assert torch.equal(M[0, 0, r], ref[0, 0, last])


def test_frozen_table_is_bit_identical_and_a_weighted_lookup():
    iw, ww, ir, wr, al, be, v, M0 = _rand_case(1)
    M, y = oracle.scan_bf16(iw, ww, ir, wr, np.ones_like(al), np.zeros_like(be), v, M0)
    assert torch.equal(M, M0)
    B, H, T, R = ir.shape
    tab = M0.float()
    for b in range(B):
        for h in range(H):
            ref = torch.nn.functional.embedding_bag(
                torch.from_numpy(ir[b, h]).long(), tab[b, h].double(), mode="sum",
                per_sample_weights=torch.from_numpy(wr[b, h]).double())
            assert np.allclose(y[b, h], ref.numpy(), rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("form", [oracle.EQ4, oracle.FIG2])
def test_each_token_is_the_fp32_recurrence_then_one_rounding(form):
    """Token by token from the same bfloat16 table: the fp32-table oracle's
    update rounded by torch to bfloat16 equals the bf16-table oracle's row,
    except where the fp32 value lies on a bfloat16 rounding tie (the fp32 step
    is a second rounding); there the two differ by one bfloat16 ulp."""
    iw, ww, ir, wr, al, be, v, M0 = _rand_case(2, T=40)
    M = M0.clone()
    mism = total = 0
    for t in range(iw.shape[2]):
        s = (slice(None), slice(None), slice(t, t + 1))
        Mb, yb = oracle.scan_bf16(iw[s], ww[s], ir[s], wr[s], al[s], be[s], v[s], M, form)
        Mf, yf = oracle.scan(iw[s], ww[s], ir[s], wr[s], al[s], be[s], v[s], M.float(), form)
        ref = torch.from_numpy(Mf).to(torch.bfloat16)
        diff = Mb.view(torch.int16).int() - ref.view(torch.int16).int()
        assert diff.abs().max() <= 1
        mism += int((diff != 0).sum()); total += diff.numel()
        if (diff != 0).any():
            # the fp32 value sits within one fp32 ulp of a bfloat16 tie
            f = torch.from_numpy(Mf)[diff != 0]
            lo = f.to(torch.bfloat16).float()
            nb = torch.nextafter(lo, torch.where(f > lo, torch.full_like(f, np.inf), torch.full_like(f, -np.inf)))
            nb = nb.to(torch.bfloat16).float()
            assert torch.all(torch.abs(2 * f - lo - nb) <= 2 * torch.abs(torch.nextafter(f, f * 2) - f))
        # the read is the fp32 read of the rounded table
        Mr = Mb.float().numpy()
        B, H = iw.shape[:2]
        for b in range(B):
            for h in range(H):
                ref_y = (wr[b, h, t][:, None].astype(np.float64) * Mr[b, h, ir[b, h, t]]).sum(0)
                assert np.allclose(yb[b, h, 0], ref_y, rtol=1e-6, atol=1e-7)
        M = Mb
    assert mism <= total * 1e-3


def test_unselected_rows_bit_identical_and_split_in_time():
    iw, ww, ir, wr, al, be, v, M0 = _rand_case(3, T=60, N=256)
    M, y = oracle.scan_bf16(iw, ww, ir, wr, al, be, v, M0, oracle.EQ4)
    written = np.zeros((iw.shape[0], iw.shape[1], 256), bool)
    for b in range(iw.shape[0]):
        for h in range(iw.shape[1]):
            written[b, h, np.unique(iw[b, h])] = True
    untouched = torch.from_numpy(~written)
    assert torch.equal(M[untouched], M0[untouched])
    s1 = (slice(None), slice(None), slice(0, 23)); s2 = (slice(None), slice(None), slice(23, None))
    Ma, ya = oracle.scan_bf16(iw[s1], ww[s1], ir[s1], wr[s1], al[s1], be[s1], v[s1], M0)
    Mb, yb = oracle.scan_bf16(iw[s2], ww[s2], ir[s2], wr[s2], al[s2], be[s2], v[s2], Ma)
    assert torch.equal(Mb, M) and np.array_equal(np.concatenate([ya, yb], 2), y)


def test_long_run_stays_within_bf16_storage_noise_of_the_fp32_table():
    wl = inputs.get("tiny")
    x = inputs.make_inputs(wl)
    iw, ww, _, _ = oracle.address(x["q_w"], x["subkeys"], wl.W)
    ir, wr, _, _ = oracle.address(x["q_r"], x["subkeys"], wl.R)
    M0 = oracle.broadcast_state(x["M0"], 1)
    M0b = torch.from_numpy(M0.copy()).to(torch.bfloat16)
    Mb, yb = oracle.scan_bf16(iw, ww, ir, wr, x["alpha"], x["beta"], x["v"], M0b)
    Mf, yf = oracle.scan(iw, ww, ir, wr, x["alpha"], x["beta"], x["v"], M0b.float())
    err = np.abs(yb - yf).max() / np.abs(yf).max()
    assert 0 < err < 2e-2
    assert np.abs(Mb.float().numpy() - Mf).max() / np.abs(Mf).max() < 2e-2


def test_bf16_table_rejects_bad_indices():
    iw, ww, ir, wr, al, be, v, M0 = _rand_case(4)
    bad = iw.copy(); bad[0, 0, 0, 0] = 64
    with pytest.raises(ValueError):
        oracle.scan_bf16(bad, ww, ir, wr, al, be, v, M0)
    dup = iw.copy(); dup[0, 0, 0, 1] = dup[0, 0, 0, 0]
    with pytest.raises(ValueError):
        oracle.scan_bf16(dup, ww, ir, wr, al, be, v, M0)
