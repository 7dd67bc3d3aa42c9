"""The scan entry point that allocates nothing (sdm_scan_forward_noalloc, for
callers that cannot allocate): through the C ABI, its y and final table must
equal sdm_scan_forward's on the same inputs bit for bit (it runs the same
kernels, in launch chunks that fit its per-GPU scratch, and a sequence split
over launches is exact). Two calls in a row, the second on a smaller input, so
the scratch's leftover contents from the first must not matter."""
import numpy as np
import pytest
import torch

import sparse_memory_linear_amd as sdm
from sparse_memory_linear_amd import inputs
from parity import say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
SCRATCH = 64 << 20


def _case(B, H, T, seed, name="gdn_matched"):
    wl = inputs.get(name, B=B, H=H, T=T)
    x = {k: v.to(DEV) for k, v in inputs.make_inputs(wl, seed=seed).items()}
    iw, ww, ir, wr = sdm.sdm_address(x["q_w"], x["q_r"], x["subkeys"], x["subkeys"], wl.W, wl.R)
    return wl, x, (iw, ww, ir, wr)


def _both(wl, x, slots, form, table=torch.float32):
    iw, ww, ir, wr = slots
    M1 = sdm.sdm_state_init(x["M0"], wl.B, dtype=table)
    M2 = M1.clone()
    y1 = sdm.sdm_scan_forward(iw, ww, ir, wr, x["alpha"], x["beta"], x["v"], M1, form)
    y2 = sdm.sdm_scan_forward_noalloc(iw, ww, ir, wr, x["alpha"], x["beta"], x["v"], M2, form)
    torch.cuda.synchronize()
    return (M1, y1), (M2, y2)


@pytest.mark.parametrize("form", ["eq4", "fig2"])
def test_noalloc_equals_workspace_entry_point_on_two_calls(form):
    # first call: 16 streams x 3000 tokens, whose workspace exceeds the scratch
    # (so several launch chunks); second call: a smaller input
    for B, H, T, seed in ((2, 8, 3000, 21), (1, 3, 700, 22)):
        wl, x, slots = _case(B, H, T, seed)
        need = sdm.sdm_scan_workspace_bytes(B, H, T, wl.W, wl.R, wl.d_v)
        say(f"[no-alloc scan] {form} B={B} H={H} T={T}: workspace of the other entry point {need} bytes")
        if (B, H, T) == (2, 8, 3000):
            assert need > SCRATCH
        (M1, y1), (M2, y2) = _both(wl, x, slots, form)
        assert torch.equal(y1, y2), float((y1 - y2).abs().max())
        assert torch.equal(M1, M2)


def test_noalloc_bf16_table_and_short_calls():
    wl, x, slots = _case(2, 8, 2500, 23)
    (M1, y1), (M2, y2) = _both(wl, x, slots, "eq4", torch.bfloat16)
    assert torch.equal(y1, y2) and torch.equal(M1.view(torch.int16), M2.view(torch.int16))
    # a decode-style call (one token: the short-call form, no scratch) after it
    wl, x, slots = _case(3, 2, 1, 24)
    (M1, y1), (M2, y2) = _both(wl, x, slots, "eq4")
    assert torch.equal(y1, y2) and torch.equal(M1, M2)
