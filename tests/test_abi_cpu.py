"""Host-side checks of the C ABI (no GPU): the library loads, exports every
declared symbol, and rejects invalid arguments before any launch."""
import ctypes
import os
import re

import pytest

from sparse_memory_linear_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdm_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return binding.lib()


def test_header_declares_the_hot_path_calls():
    names = declared_functions()
    for f in ("sdm_address", "sdm_scan_forward", "sdm_state_init", "sdm_debug_half_scores",
              "sdm_scan_workspace_bytes", "sdm_status_string", "sdm_last_error", "sdm_abi_version",
              "sdm_scan_forward_save", "sdm_scan_snapshot_bytes", "sdm_scan_backward",
              "sdm_scan_backward_workspace_bytes", "sdm_state_init_backward", "sdm_address_idw",
              "sdm_debug_half_scores_idw", "sdm_gates", "sdm_output_gate", "sdm_scan_forward_noalloc",
              "sdm_scan_forward_gated", "sdm_scan_gated_workspace_bytes"):
        assert f in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(binding._SIGS) == set(declared_functions())


def test_abi_version_and_status_strings(lib):
    assert binding.sdm_abi_version() == 7
    assert binding.sdm_status_string(0) == "ok"
    assert binding.sdm_status_string(7).startswith("workspace")
    assert binding.sdm_status_string(99) == "unknown status"


def test_workspace_size_is_pure_host_logic(lib):
    # W = R = 64, dv = 128, 32 streams. The per-slot form uses 32-column slabs
    # (8 rows per wavefront, 8 writer + 8 reader wavefronts; a token record holds
    # 64 writer entries of 16 bytes and 64 reader entries of 8 bytes) with the
    # rows split into 2 partitions (32 * 4 slabs * 2 = 256 workgroups), plus the
    # two partitions' partial y. The shared-residual form (16-column slabs, one
    # partition) needs less, and the workspace covers both.
    # and the largest per-token count of each (stream, partition, branch)
    # The workspace also covers a bf16 table (32-column slabs, 2 partitions for
    # 32 streams; 16-column slabs, 8 partitions for 8): the same sizes here.
    rec = 64 * 16 + 64 * 8
    assert binding.sdm_scan_workspace_bytes(4, 8, 8192, 64, 64, 128) == \
        32 * 2 * 8192 * rec + 2 * 32 * 8192 * 128 * 4 + 32 * 2 * 2 * 4
    # 8 streams (the long-context shape): 8 partitions
    assert binding.sdm_scan_workspace_bytes(1, 8, 1000, 64, 64, 128) == \
        8 * 8 * 1000 * rec + 8 * 8 * 1000 * 128 * 4 + 8 * 8 * 2 * 4
    assert binding.sdm_scan_workspace_bytes(0, 8, 8192, 64, 64, 128) == 0
    # W = 120, R = 8, 32 streams: 32-column slabs would fit 16 wavefronts, but
    # their forwarding ring (14 tokens x 120 rows x 128 B) exceeds the 160 KiB of
    # LDS, and 16-column ones need 9 wavefronts; every form and table dtype takes
    # 8-column slabs (4 writer + 1 reader wavefronts of 32 rows), one partition
    assert binding.sdm_scan_workspace_bytes(4, 8, 1000, 120, 8, 128) == \
        32 * 1000 * (4 * 32 * 16 + 32 * 8) + 32 * 2 * 4
    assert lib.sdm_scan_workspace_bytes(1, 1, 1, 0, 1, 16) == -1
    assert lib.sdm_scan_workspace_bytes(1, 1, 1, 300, 1, 16) == -1


P = ctypes.c_void_p


def test_address_rejects_bad_arguments_before_launch(lib):
    fake = P(4096)  # never dereferenced: every call below fails validation first
    args = lambda **kw: dict(dict(q_w=fake, q_r=fake, qd=1, kw=fake, kr=fake, kd=1, B=1, H=1, T=16,
                                  n=256, dh=64, W=64, R=64, iw=fake, ww=fake, ir=fake, wr=fake,
                                  sw=None, sr=None, st=None), **kw)
    call = lambda a: lib.sdm_address(*a.values())
    assert call(args(q_w=None)) == 1
    assert call(args(qd=5)) == 3
    assert call(args(kd=0)) == 3                 # subkey dtype must match q
    assert call(args(T=-1)) == 2
    assert call(args(n=250)) == 5                # not a multiple of 16
    assert call(args(dh=48)) == 5                # bf16 needs multiples of 32
    assert call(args(W=0)) == 2
    assert call(args(W=65)) == 5                 # GPU covers k <= 64
    assert call(args(iw=P(4100))) == 4           # misaligned
    assert "aligned" in binding.sdm_last_error()
    assert call(args(B=1 << 16, T=1 << 16)) == 5  # 2^32 tokens: token numbers are 32-bit on the GPU
    assert "2^32" in binding.sdm_last_error()


def test_scan_rejects_bad_arguments_before_launch(lib):
    fake = P(4096)
    base = dict(iw=fake, ww=fake, W=64, ir=fake, wr=fake, R=64, a=fake, b=fake, v=fake, vd=1,
                M=fake, md=0, y=fake, B=1, H=1, T=8, N=65536, dv=128, form=0, ws=fake, wsb=1 << 30,
                st=None)
    call = lambda **kw: lib.sdm_scan_forward(*dict(base, **kw).values())
    assert call(iw=None) == 1
    assert call(iw=None, ww=None, M=None, T=0) == 0                     # empty: valid no-op
    assert call(vd=2) == 3
    assert call(md=2) == 3                       # unknown table dtype
    assert call(md=1, dv=132) == 5               # a bf16 table needs dv % 8 == 0
    assert call(md=1, M=None) == 1
    assert call(form=2) == 3
    assert call(W=65537) == 2                    # W > N
    assert call(N=(1 << 18) + 1, W=64) == 5
    assert call(dv=130) == 5
    assert call(N=1 << 18, W=64, dv=2048) == 5   # one stream's table would reach 2 GiB
    assert call(ws=None) == 7
    assert call(wsb=100) == 7
    assert call(y=P(4104)) == 4
    assert "workspace" in binding.sdm_last_error() or "aligned" in binding.sdm_last_error()


def test_training_sizes_are_pure_host_logic(lib):
    # pre-images: one fp32 row per write
    assert binding.sdm_scan_snapshot_bytes(4, 8, 8192, 64, 128) == 4 * 8 * 8192 * 64 * 128 * 4
    assert lib.sdm_scan_snapshot_bytes(1, 1, 1, 0, 16) == -1
    # backward partial sums: per (slab, stream, token) W + R weight gradients, per
    # (slab, partition, stream, token) 2 gate gradients, with P > 1 row
    # partitions a partial dv per partition, and per (stream, token) the
    # prefetch plan's W + 2R source words; the workspace covers both forms.
    def bwd(NS, T, S, P, W=64, R=64, dv=128):
        nslab = dv // S
        return 4 * (nslab * NS * T * (W + R) + nslab * P * NS * T * 2 + (P * NS * T * dv if P > 1 else 0)
                    + NS * T * (W + 2 * R))
    # the per-slot form takes the widest slab that fills 256 workgroups in at most
    # 2 partitions (32 streams: 32-column slabs in 2; 8 streams: 8-column slabs in
    # 2), the shared-residual form the widest with at most 8 wavefronts and at
    # least 128 workgroups (32 streams: 16-column slabs; 8 streams: 8-column
    # slabs), and the workspace is the larger of the two; chunks of at most
    # 2^31 / (W dv 4) tokens
    assert bwd(32, 8192, 16, 1) > bwd(32, 8192, 32, 2)
    assert binding.sdm_scan_backward_workspace_bytes(4, 8, 8192, 64, 64, 128) == bwd(32, 8192, 16, 1)
    assert binding.sdm_scan_backward_workspace_bytes(1, 8, 1000, 64, 64, 128) == bwd(8, 1000, 8, 2)
    Tc = 0x7FFFFFFF // (64 * 128 * 4)
    assert binding.sdm_scan_backward_workspace_bytes(1, 8, 131072, 64, 64, 128) == bwd(8, Tc, 8, 2)
    # small W, large R: the chunk is bounded by the W + 2R plan words per token, not
    # by the pre-images (1 x 4 x 4 bytes): 2^31 / ((1 + 512) x 4) tokens
    Tc = 0x7FFFFFFF // ((1 + 2 * 256) * 4)
    assert binding.sdm_scan_backward_workspace_bytes(1, 1, 2_000_000, 1, 256, 4) == \
        bwd(1, Tc, 4, 1, W=1, R=256, dv=4)
    # one stream of d_v = 512, W = R = 8: only 4-column slabs reach 128 workgroups
    assert binding.sdm_scan_backward_workspace_bytes(1, 1, 500, 8, 8, 512) == bwd(1, 500, 4, 1, W=8, R=8, dv=512)
    assert binding.sdm_scan_backward_workspace_bytes(0, 8, 100, 64, 64, 128) == 0
    assert lib.sdm_scan_backward_workspace_bytes(1, 1, 1, 300, 1, 16) == -1


def test_training_calls_reject_bad_arguments_before_launch(lib):
    fake = P(4096)
    fwd = dict(iw=fake, ww=fake, W=64, ir=fake, wr=fake, R=64, a=fake, b=fake, v=fake, vd=1,
               M=fake, y=fake, snap=fake, B=1, H=1, T=8, N=65536, dv=128, form=0, ws=fake,
               wsb=1 << 30, st=None)
    call = lambda **kw: lib.sdm_scan_forward_save(*dict(fwd, **kw).values())
    assert call(snap=None) == 1
    assert call(snap=P(4100)) == 4
    assert call(snap=None, T=0) == 0
    assert call(form=3) == 3
    bwd = dict(iw=fake, ww=fake, W=64, ir=fake, wr=fake, R=64, a=fake, b=fake, v=fake, vd=1,
               snap=fake, dy=fake, M=fake, dM=fake, dv=fake, da=fake, db=fake, dww=fake, dwr=fake,
               B=1, H=1, T=8, N=65536, dvs=128, form=0, ws=fake, wsb=1 << 30, st=None)
    callb = lambda **kw: lib.sdm_scan_backward(*dict(bwd, **kw).values())
    for k in ("snap", "dy", "M", "dM", "dv", "da", "db", "dww", "dwr"):
        assert callb(**{k: None}) == 1, k
    assert callb(dy=P(4104)) == 4
    assert callb(ws=None) == 7
    assert callb(wsb=16) == 7
    assert callb(dvs=130) == 5
    assert callb(W=0) == 2
    assert callb(snap=None, dy=None, T=0) == 0
    assert lib.sdm_state_init_backward(None, fake, 2, 1, 16, 16, None) == 1
    assert lib.sdm_state_init_backward(fake, fake, 0, 1, 16, 16, None) == 2
    assert lib.sdm_state_init_backward(fake, fake, 2, 1, 16, 18, None) == 5


def test_state_init_rejects_bad_arguments(lib):
    fake = P(4096)
    assert lib.sdm_state_init(None, fake, 0, 1, 1, 16, 16, None) == 1
    assert lib.sdm_state_init(None, None, 0, 0, 1, 16, 16, None) == 0   # empty: no storage needed
    assert lib.sdm_state_init(fake, fake, 0, 1, 1, 16, 18, None) == 5
    assert lib.sdm_state_init(fake, fake, 1, 1, 1, 16, 18, None) == 5
    assert lib.sdm_state_init(fake, fake, 0, -1, 1, 16, 16, None) == 2
    assert lib.sdm_state_init(fake, fake, 3, 1, 1, 16, 16, None) == 3   # unknown table dtype


def test_binding_refuses_cpu_tensors(lib):
    import torch
    x = torch.zeros(1, 1, 16, 2, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 256, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        binding.sdm_address(x, x, k, k, 8, 8)


def test_glue_calls_reject_bad_arguments_before_launch(lib):
    fake = P(4096)  # never dereferenced: every call below fails validation first
    g = lambda x_dtype=1, w_dtype=1, B=2, T=16, d=1024, H=8: lib.sdm_gates(
        fake, x_dtype, fake, fake, w_dtype, fake, fake, B, T, d, H, fake, fake, None)
    assert g(x_dtype=5) == 3
    assert g(w_dtype=0) == 3                      # weights in the dtype of x
    assert g(d=1000) == 5                         # bf16 needs d % 32 == 0
    assert g(H=5000) == 5
    assert g(B=1 << 16, T=1 << 16) == 5           # 2^32 tokens: token numbers are 32-bit on the GPU
    assert "2^32" in binding.sdm_last_error()
    og = lambda B=2, H=8, T=16, dv=128, eps=1e-6: lib.sdm_output_gate(
        fake, fake, fake, 0, ctypes.c_float(eps), B, H, T, dv, fake, None)
    assert og(dv=130) == 5
    assert og(eps=-1.0) == 2
    assert og(B=1 << 12, H=1 << 10, T=1 << 10) == 5   # 2^32 rows
    assert "2^32" in binding.sdm_last_error()


def test_noalloc_scan_rejects_bad_arguments_before_launch(lib):
    """The scan entry point without a workspace validates like sdm_scan_forward
    and rejects stream counts whose scan needs more than its 64 MiB scratch for
    a single token per launch, all before any HIP call."""
    fake = P(4096)
    base = dict(iw=fake, ww=fake, W=64, ir=fake, wr=fake, R=64, a=fake, b=fake, v=fake, vd=1,
                M=fake, md=0, y=fake, B=1, H=1, T=100, N=4096, dv=128, form=0, st=None)
    call = lambda **kw: lib.sdm_scan_forward_noalloc(*dict(base, **kw).values())
    assert call(iw=None) == 1
    assert call(iw=None, ww=None, M=None, T=0) == 0                     # empty: valid no-op
    assert call(form=2) == 3
    assert call(y=P(4104)) == 4
    # 65536 streams: one token's plan records alone take 65536 x 1536 bytes
    assert call(B=65536) == 5
    assert "scratch" in binding.sdm_last_error()


def test_gated_scan_rejects_bad_arguments_before_launch(lib):
    """The scan with the output step validates the scan's arguments like
    sdm_scan_forward, then its own (gate dtype, eps, gamma/g/o, o not aliasing
    y, the larger workspace), all before any HIP call; y may be NULL."""
    fake = P(4096)
    B, H, T, dv = 1, 2, 100, 128
    need = binding.sdm_scan_gated_workspace_bytes(B, H, T, 64, 64, dv)
    assert need >= binding.sdm_scan_workspace_bytes(B, H, T, 64, 64, dv) + B * H * T * dv * 4
    assert binding.sdm_scan_gated_workspace_bytes(0, H, T, 64, 64, dv) == 0
    assert lib.sdm_scan_gated_workspace_bytes(B, H, T, 64, 64, 6) == -1
    base = dict(iw=fake, ww=fake, W=64, ir=fake, wr=fake, R=64, a=fake, b=fake, v=fake, vd=1, M=fake, md=0,
                y=None, gamma=fake, g=fake, gd=1, eps=ctypes.c_float(1e-6), o=P(8192), B=B, H=H, T=T, N=4096,
                dv=dv, form=0, ws=fake, wsb=need, st=None)
    call = lambda **kw: lib.sdm_scan_forward_gated(*dict(base, **kw).values())
    assert call(iw=None) == 1                                  # SDM_ERR_NULL
    assert call(gamma=None) == 1
    assert call(o=None) == 1
    assert call(iw=None, ww=None, M=None, T=0) == 0           # empty: valid no-op
    assert call(gd=5) == 3                                     # SDM_ERR_DTYPE
    assert call(form=2) == 3
    assert call(eps=ctypes.c_float(-1.0)) == 2                 # SDM_ERR_SHAPE
    assert call(y=P(8192)) == 2                                # o aliases y
    assert call(o=P(8200)) == 4                                # SDM_ERR_ALIGN
    assert call(wsb=need - 16) == 7                            # SDM_ERR_WORKSPACE
