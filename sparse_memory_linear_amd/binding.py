"""Thin Python binding of libsdm.so (include/sdm.h), same names as the C ABI.

Argument marshalling only: tensors are checked (device, dtype, shape,
contiguity), outputs are allocated with torch on the tensors' device, and the
raw device pointers plus the current torch stream are handed to the C ABI.
Every step of the hot path runs in the library's HIP kernels; there is no
fallback. If the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsdm.so")

SDM_F32, SDM_BF16 = 0, 1
SDM_DELTA_EQ4, SDM_DELTA_FIG2 = 0, 1
FORMS = {"eq4": SDM_DELTA_EQ4, "fig2": SDM_DELTA_FIG2}

# int sdm_*(...) signatures, in the order of include/sdm.h
_P, _I64, _I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
_SIGS = {
    "sdm_abi_version": (_I, []),
    "sdm_status_string": (ctypes.c_char_p, [_I]),
    "sdm_last_error": (ctypes.c_char_p, []),
    "sdm_address": (_I, [_P, _P, _I, _P, _P, _I, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                         _P, _P, _P, _P, _P, _P, _P]),
    "sdm_debug_half_scores": (_I, [_P, _I, _P, _I, _I64, _I64, _I64, _I64, _I64, _P, _P]),
    "sdm_address_idw": (_I, [_P, _P, _I, _P, _P, _I, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                             _P, _P, _P, _P, _P, _P, _P]),
    "sdm_debug_half_scores_idw": (_I, [_P, _I, _P, _I, _I64, _I64, _I64, _I64, _I64, _P, _P]),
    "sdm_state_init": (_I, [_P, _P, _I, _I64, _I64, _I64, _I64, _P]),
    "sdm_scan_workspace_bytes": (_I64, [_I64, _I64, _I64, _I64, _I64, _I64]),
    "sdm_scan_forward": (_I, [_P, _P, _I64, _P, _P, _I64, _P, _P, _P, _I, _P, _I, _P,
                              _I64, _I64, _I64, _I64, _I64, _I, _P, _I64, _P]),
    "sdm_scan_gated_workspace_bytes": (_I64, [_I64, _I64, _I64, _I64, _I64, _I64]),
    "sdm_scan_forward_gated": (_I, [_P, _P, _I64, _P, _P, _I64, _P, _P, _P, _I, _P, _I, _P,
                                    _P, _P, _I, ctypes.c_float, _P,
                                    _I64, _I64, _I64, _I64, _I64, _I, _P, _I64, _P]),
    "sdm_scan_forward_noalloc": (_I, [_P, _P, _I64, _P, _P, _I64, _P, _P, _P, _I, _P, _I, _P,
                                      _I64, _I64, _I64, _I64, _I64, _I, _P]),
    "sdm_scan_snapshot_bytes": (_I64, [_I64, _I64, _I64, _I64, _I64]),
    "sdm_scan_forward_save": (_I, [_P, _P, _I64, _P, _P, _I64, _P, _P, _P, _I, _P, _P, _P,
                                   _I64, _I64, _I64, _I64, _I64, _I, _P, _I64, _P]),
    "sdm_scan_backward_workspace_bytes": (_I64, [_I64, _I64, _I64, _I64, _I64, _I64]),
    "sdm_scan_backward": (_I, [_P, _P, _I64, _P, _P, _I64, _P, _P, _P, _I, _P, _P, _P, _P,
                               _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I, _P, _I64, _P]),
    "sdm_state_init_backward": (_I, [_P, _P, _I64, _I64, _I64, _I64, _P]),
    "sdm_gates": (_I, [_P, _I, _P, _P, _I, _P, _P, _I64, _I64, _I64, _I64, _P, _P, _P]),
    "sdm_output_gate": (_I, [_P, _P, _P, _I, ctypes.c_float, _I64, _I64, _I64, _I64, _P, _P]),
}

_lib = None


class SdmError(RuntimeError):
    def __init__(self, fn: str, code: int, detail: str):
        super().__init__(f"{fn} failed with status {code}: {detail}")
        self.code = code


def lib() -> ctypes.CDLL:
    """The loaded libsdm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(fn: str, rc: int):
    if rc != 0:
        raise SdmError(fn, rc, lib().sdm_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dev(*ts: torch.Tensor) -> torch.device:
    d = ts[0].device
    for t in ts:
        if t.device.type != "cuda" or t.device != d:
            raise ValueError("all tensors must be on the same GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return d


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SDM_F32
    if t.dtype == torch.bfloat16:
        return SDM_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


def sdm_abi_version() -> int:
    return lib().sdm_abi_version()


def sdm_status_string(code: int) -> str:
    return lib().sdm_status_string(code).decode()


def sdm_last_error() -> str:
    return lib().sdm_last_error().decode()


SCORINGS = ("dot", "idw")


def sdm_address(q_w: torch.Tensor, q_r: torch.Tensor, subkeys_w: torch.Tensor,
                subkeys_r: torch.Tensor, W: int, R: int, return_scores: bool = False,
                out: Optional[Tuple[torch.Tensor, ...]] = None, scoring: str = "dot"):
    """Product-key addressing of both branches.

    q_w, q_r [B,H,T,2,dh]; subkeys [H,2,n_sub,dh] (same dtype, fp32 or bf16).
    Returns (idx_w, wt_w, idx_r, wt_r) and, with return_scores, (score_w, score_r).
    ``out`` may pass preallocated (idx_w, wt_w, idx_r, wt_r) tensors. ``scoring``
    "dot" calls sdm_address, "idw" sdm_address_idw (inverse-distance half-scores).
    """
    if scoring not in SCORINGS:
        raise ValueError(f"unknown scoring {scoring!r}")
    fn = "sdm_address" if scoring == "dot" else "sdm_address_idw"
    d = _dev(q_w, q_r, subkeys_w, subkeys_r)
    B, H, T, two, dh = q_w.shape
    n = subkeys_w.shape[2]
    if two != 2 or q_r.shape != q_w.shape or subkeys_w.shape != (H, 2, n, dh) \
            or subkeys_r.shape != subkeys_w.shape:
        raise ValueError("shape mismatch in sdm_address")
    kw = dict(device=d)
    if out is not None:
        idx_w, wt_w, idx_r, wt_r = out
        for t, shp, dt in ((idx_w, (B, H, T, W), torch.int32), (wt_w, (B, H, T, W), torch.float32),
                           (idx_r, (B, H, T, R), torch.int32), (wt_r, (B, H, T, R), torch.float32)):
            if tuple(t.shape) != shp or t.dtype != dt:
                raise ValueError("preallocated address output has the wrong shape or dtype")
        _dev(q_w, idx_w, wt_w, idx_r, wt_r)
    else:
        idx_w = torch.empty((B, H, T, W), dtype=torch.int32, **kw)
        wt_w = torch.empty((B, H, T, W), dtype=torch.float32, **kw)
        idx_r = torch.empty((B, H, T, R), dtype=torch.int32, **kw)
        wt_r = torch.empty((B, H, T, R), dtype=torch.float32, **kw)
    sc_w = torch.empty((B, H, T, W), dtype=torch.float32, **kw) if return_scores else None
    sc_r = torch.empty((B, H, T, R), dtype=torch.float32, **kw) if return_scores else None
    _check(fn, getattr(lib(), fn)(
        _ptr(q_w), _ptr(q_r), _dtype_code(q_w), _ptr(subkeys_w), _ptr(subkeys_r),
        _dtype_code(subkeys_w), B, H, T, n, dh, W, R, _ptr(idx_w), _ptr(wt_w), _ptr(idx_r),
        _ptr(wt_r), _ptr(sc_w), _ptr(sc_r), _stream(d)))
    out = (idx_w, wt_w, idx_r, wt_r)
    return out + (sc_w, sc_r) if return_scores else out


def sdm_debug_half_scores(q: torch.Tensor, subkeys: torch.Tensor, scoring: str = "dot") -> torch.Tensor:
    """Half-scores [B,H,T,2,n_sub] fp32 of one branch (the contraction of sdm_address,
    or with scoring "idw" the inverse-distance scores of sdm_address_idw)."""
    if scoring not in SCORINGS:
        raise ValueError(f"unknown scoring {scoring!r}")
    fn = "sdm_debug_half_scores" if scoring == "dot" else "sdm_debug_half_scores_idw"
    d = _dev(q, subkeys)
    B, H, T, _, dh = q.shape
    n = subkeys.shape[2]
    half = torch.empty((B, H, T, 2, n), dtype=torch.float32, device=d)
    _check(fn, getattr(lib(), fn)(
        _ptr(q), _dtype_code(q), _ptr(subkeys), _dtype_code(subkeys), B, H, T, n, dh,
        _ptr(half), _stream(d)))
    return half


def sdm_state_init(M0: torch.Tensor, B: int, out: Optional[torch.Tensor] = None,
                   dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """Per-sequence table [B,H,N,dv] initialised from M0 [H,N,dv] fp32, stored in
    ``dtype`` (float32, or bfloat16: rounded to nearest even)."""
    d = _dev(M0)
    H, N, dv = M0.shape
    if M0.dtype != torch.float32:
        raise ValueError("M0 must be fp32")
    M = out if out is not None else torch.empty((B, H, N, dv), dtype=dtype, device=d)
    if M.shape != (B, H, N, dv) or M.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("state tensor has the wrong shape or dtype")
    _dev(M0, M)
    _check("sdm_state_init", lib().sdm_state_init(_ptr(M0), _ptr(M), _dtype_code(M), B, H, N, dv,
                                                  _stream(d)))
    return M


def sdm_scan_workspace_bytes(B: int, H: int, T: int, W: int, R: int, dv: int) -> int:
    n = lib().sdm_scan_workspace_bytes(B, H, T, W, R, dv)
    if n < 0:
        raise ValueError("invalid sizes for the scan workspace")
    return n


def _scan_inputs(fn, idx_w, wt_w, idx_r, wt_r, alpha, beta, v, M, table_dtypes=(torch.float32,)):
    d = _dev(idx_w, wt_w, idx_r, wt_r, alpha, beta, v, M)
    B, H, T, W = idx_w.shape
    R = idx_r.shape[3]
    N, dv = M.shape[2], M.shape[3]
    shapes = {"wt_w": (wt_w, (B, H, T, W)), "idx_r": (idx_r, (B, H, T, R)),
              "wt_r": (wt_r, (B, H, T, R)), "alpha": (alpha, (B, H, T)),
              "beta": (beta, (B, H, T)), "v": (v, (B, H, T, dv)), "M": (M, (B, H, N, dv))}
    for name, (t, shp) in shapes.items():
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
    if idx_w.dtype != torch.int32 or idx_r.dtype != torch.int32 or wt_w.dtype != torch.float32 \
            or wt_r.dtype != torch.float32 or alpha.dtype != torch.float32 \
            or beta.dtype != torch.float32 or M.dtype not in table_dtypes:
        raise ValueError(f"dtype mismatch in {fn}")
    return d, (B, H, T, W, R, N, dv)


def _f32_out(t: Optional[torch.Tensor], shape, d, name: str) -> torch.Tensor:
    if t is None:
        return torch.empty(shape, dtype=torch.float32, device=d)
    if tuple(t.shape) != tuple(shape) or t.dtype != torch.float32:
        raise ValueError(f"{name} has the wrong shape or dtype")
    _dev(t)
    if t.device != d:
        raise ValueError("all tensors must be on the same GPU")
    return t


def _workspace(ws: Optional[torch.Tensor], nbytes: int, d) -> torch.Tensor:
    if ws is None:
        return torch.empty((max(nbytes, 16),), dtype=torch.uint8, device=d)
    if ws.dtype != torch.uint8 or ws.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 tensor")
    _dev(ws)
    return ws


def sdm_scan_forward(idx_w: torch.Tensor, wt_w: torch.Tensor, idx_r: torch.Tensor,
                     wt_r: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor,
                     v: torch.Tensor, M: torch.Tensor, form: str = "eq4",
                     y: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Sparse gated delta scan over all T tokens; M [B,H,N,dv] (float32 or
    bfloat16 storage) is updated in place.

    Returns y [B,H,T,dv] fp32.
    """
    d, (B, H, T, W, R, N, dv) = _scan_inputs("sdm_scan_forward", idx_w, wt_w, idx_r, wt_r,
                                             alpha, beta, v, M, (torch.float32, torch.bfloat16))
    y = _f32_out(y, (B, H, T, dv), d, "y")
    workspace = _workspace(workspace, sdm_scan_workspace_bytes(B, H, T, W, R, dv), d)
    _check("sdm_scan_forward", lib().sdm_scan_forward(
        _ptr(idx_w), _ptr(wt_w), W, _ptr(idx_r), _ptr(wt_r), R, _ptr(alpha), _ptr(beta),
        _ptr(v), _dtype_code(v), _ptr(M), _dtype_code(M), _ptr(y), B, H, T, N, dv, FORMS[form],
        _ptr(workspace), workspace.numel(), _stream(d)))
    return y


def sdm_scan_gated_workspace_bytes(B: int, H: int, T: int, W: int, R: int, dv: int) -> int:
    n = lib().sdm_scan_gated_workspace_bytes(B, H, T, W, R, dv)
    if n < 0:
        raise ValueError("invalid sizes for the gated scan workspace")
    return n


def sdm_scan_forward_gated(idx_w: torch.Tensor, wt_w: torch.Tensor, idx_r: torch.Tensor,
                           wt_r: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor,
                           v: torch.Tensor, M: torch.Tensor, gamma: torch.Tensor, g: torch.Tensor,
                           eps: float = 1e-6, form: str = "eq4", y: Optional[torch.Tensor] = None,
                           keep_y: bool = False, out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None):
    """The scan followed by the output step (RMS-Norm, gamma, sigmoid gate).
    M is updated in place. Returns o [B,H,T,dv] fp32, or (o, y) when y is given
    or keep_y is set (otherwise y is not stored where the scan need not)."""
    d, (B, H, T, W, R, N, dv) = _scan_inputs("sdm_scan_forward_gated", idx_w, wt_w, idx_r, wt_r,
                                             alpha, beta, v, M, (torch.float32, torch.bfloat16))
    if gamma.shape != (H, dv) or gamma.dtype != torch.float32 or g.shape != (B, H, T, dv):
        raise ValueError("shape or dtype mismatch of gamma or g in sdm_scan_forward_gated")
    _dev(idx_w, gamma, g)
    if y is not None or keep_y:
        y = _f32_out(y, (B, H, T, dv), d, "y")
    o = _f32_out(out, (B, H, T, dv), d, "o")
    workspace = _workspace(workspace, sdm_scan_gated_workspace_bytes(B, H, T, W, R, dv), d)
    _check("sdm_scan_forward_gated", lib().sdm_scan_forward_gated(
        _ptr(idx_w), _ptr(wt_w), W, _ptr(idx_r), _ptr(wt_r), R, _ptr(alpha), _ptr(beta),
        _ptr(v), _dtype_code(v), _ptr(M), _dtype_code(M), _ptr(y),
        _ptr(gamma), _ptr(g), _dtype_code(g), float(eps), _ptr(o), B, H, T, N, dv, FORMS[form],
        _ptr(workspace), workspace.numel(), _stream(d)))
    return (o, y) if y is not None else o


def sdm_scan_forward_noalloc(idx_w: torch.Tensor, wt_w: torch.Tensor, idx_r: torch.Tensor,
                             wt_r: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor,
                             v: torch.Tensor, M: torch.Tensor, form: str = "eq4",
                             y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """sdm_scan_forward with the library's own per-GPU scratch instead of a
    workspace (the C call allocates nothing; pass y to keep this binding from
    allocating it). M is updated in place. Returns y [B,H,T,dv] fp32."""
    d, (B, H, T, W, R, N, dv) = _scan_inputs("sdm_scan_forward_noalloc", idx_w, wt_w, idx_r, wt_r,
                                             alpha, beta, v, M, (torch.float32, torch.bfloat16))
    y = _f32_out(y, (B, H, T, dv), d, "y")
    _check("sdm_scan_forward_noalloc", lib().sdm_scan_forward_noalloc(
        _ptr(idx_w), _ptr(wt_w), W, _ptr(idx_r), _ptr(wt_r), R, _ptr(alpha), _ptr(beta),
        _ptr(v), _dtype_code(v), _ptr(M), _dtype_code(M), _ptr(y), B, H, T, N, dv, FORMS[form],
        _stream(d)))
    return y


def sdm_scan_snapshot_bytes(B: int, H: int, T: int, W: int, dv: int) -> int:
    n = lib().sdm_scan_snapshot_bytes(B, H, T, W, dv)
    if n < 0:
        raise ValueError("invalid sizes for the pre-image buffer")
    return n


def sdm_scan_forward_save(idx_w: torch.Tensor, wt_w: torch.Tensor, idx_r: torch.Tensor,
                          wt_r: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor,
                          v: torch.Tensor, M: torch.Tensor, form: str = "eq4",
                          y: Optional[torch.Tensor] = None, snap: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None
                          ) -> Tuple[torch.Tensor, torch.Tensor]:
    """The training forward: sdm_scan_forward that also stores the pre-image of
    every write. M is updated in place. Returns (y [B,H,T,dv], snap [B,H,T,W,dv])."""
    d, (B, H, T, W, R, N, dv) = _scan_inputs("sdm_scan_forward_save", idx_w, wt_w, idx_r, wt_r,
                                             alpha, beta, v, M)
    y = _f32_out(y, (B, H, T, dv), d, "y")
    snap = _f32_out(snap, (B, H, T, W, dv), d, "snap")
    workspace = _workspace(workspace, sdm_scan_workspace_bytes(B, H, T, W, R, dv), d)
    _check("sdm_scan_forward_save", lib().sdm_scan_forward_save(
        _ptr(idx_w), _ptr(wt_w), W, _ptr(idx_r), _ptr(wt_r), R, _ptr(alpha), _ptr(beta),
        _ptr(v), _dtype_code(v), _ptr(M), _ptr(y), _ptr(snap), B, H, T, N, dv, FORMS[form],
        _ptr(workspace), workspace.numel(), _stream(d)))
    return y, snap


def sdm_scan_backward_workspace_bytes(B: int, H: int, T: int, W: int, R: int, dv: int) -> int:
    n = lib().sdm_scan_backward_workspace_bytes(B, H, T, W, R, dv)
    if n < 0:
        raise ValueError("invalid sizes for the backward workspace")
    return n


def sdm_scan_backward(idx_w: torch.Tensor, wt_w: torch.Tensor, idx_r: torch.Tensor,
                      wt_r: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor,
                      v: torch.Tensor, snap: torch.Tensor, dy: torch.Tensor, M: torch.Tensor,
                      dM: torch.Tensor, form: str = "eq4", out: Optional[dict] = None,
                      workspace: Optional[torch.Tensor] = None) -> dict:
    """Backward of one sdm_scan_forward_save call, undoing its writes in place.

    M [B,H,N,dv] (in: after the forward call, out: before it) and dM (in: dL/dM
    after the call, out: before it) are updated in place. Returns a dict with dv
    [B,H,T,dv], dalpha, dbeta [B,H,T], dwt_w [B,H,T,W], dwt_r [B,H,T,R]; ``out``
    may pass those tensors preallocated.
    """
    d, (B, H, T, W, R, N, dv) = _scan_inputs("sdm_scan_backward", idx_w, wt_w, idx_r, wt_r,
                                             alpha, beta, v, M)
    for name, t, shp in (("snap", snap, (B, H, T, W, dv)), ("dy", dy, (B, H, T, dv)),
                         ("dM", dM, (B, H, N, dv))):
        if tuple(t.shape) != shp or t.dtype != torch.float32:
            raise ValueError(f"{name} has the wrong shape or dtype")
        _dev(M, t)
    out = dict(out or {})
    shapes = {"dv": (B, H, T, dv), "dalpha": (B, H, T), "dbeta": (B, H, T),
              "dwt_w": (B, H, T, W), "dwt_r": (B, H, T, R)}
    for k, shp in shapes.items():
        out[k] = _f32_out(out.get(k), shp, d, k)
    workspace = _workspace(workspace, sdm_scan_backward_workspace_bytes(B, H, T, W, R, dv), d)
    _check("sdm_scan_backward", lib().sdm_scan_backward(
        _ptr(idx_w), _ptr(wt_w), W, _ptr(idx_r), _ptr(wt_r), R, _ptr(alpha), _ptr(beta),
        _ptr(v), _dtype_code(v), _ptr(snap), _ptr(dy), _ptr(M), _ptr(dM), _ptr(out["dv"]),
        _ptr(out["dalpha"]), _ptr(out["dbeta"]), _ptr(out["dwt_w"]), _ptr(out["dwt_r"]),
        B, H, T, N, dv, FORMS[form], _ptr(workspace), workspace.numel(), _stream(d)))
    return out


def sdm_gates(x: torch.Tensor, W_a: torch.Tensor, W_b: torch.Tensor, b_dt: torch.Tensor,
              A: torch.Tensor, out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None
              ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Scan gates from the layer input: alpha = exp(-A softplus(W_a x + b_dt)),
    beta = sigmoid(W_b x). x [B,T,d], W_a/W_b [H,d] (same dtype, fp32 or bf16),
    b_dt/A [H] fp32. Returns (alpha, beta) [B,H,T] fp32."""
    d_ = _dev(x, W_a, W_b, b_dt, A)
    B, T, d = x.shape
    H = W_a.shape[0]
    if W_a.shape != (H, d) or W_b.shape != (H, d) or b_dt.shape != (H,) or A.shape != (H,):
        raise ValueError("shape mismatch in sdm_gates")
    if b_dt.dtype != torch.float32 or A.dtype != torch.float32:
        raise ValueError("b_dt and A must be fp32")
    al, be = out if out is not None else (None, None)
    al = _f32_out(al, (B, H, T), d_, "alpha")
    be = _f32_out(be, (B, H, T), d_, "beta")
    _check("sdm_gates", lib().sdm_gates(
        _ptr(x), _dtype_code(x), _ptr(W_a), _ptr(W_b), _dtype_code(W_a), _ptr(b_dt), _ptr(A),
        B, T, d, H, _ptr(al), _ptr(be), _stream(d_)))
    return al, be


def sdm_output_gate(y: torch.Tensor, gamma: torch.Tensor, g: torch.Tensor, eps: float = 1e-6,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-head RMS-Norm of y [B,H,T,dv] times gamma [H,dv] and sigmoid(g) (g
    [B,H,T,dv], fp32 or bf16). Returns o [B,H,T,dv] fp32."""
    d_ = _dev(y, gamma, g)
    B, H, T, dv = y.shape
    if gamma.shape != (H, dv) or g.shape != y.shape or y.dtype != torch.float32 \
            or gamma.dtype != torch.float32:
        raise ValueError("shape or dtype mismatch in sdm_output_gate")
    o = _f32_out(out, (B, H, T, dv), d_, "o")
    if o.data_ptr() == y.data_ptr() and o.numel() > 0:
        raise ValueError("o may not alias y")
    _check("sdm_output_gate", lib().sdm_output_gate(
        _ptr(y), _ptr(gamma), _ptr(g), _dtype_code(g), float(eps), B, H, T, dv, _ptr(o), _stream(d_)))
    return o


def sdm_state_init_backward(dM: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Gradient of the shared initial state: dM0 [H,N,dv] = sum over b of dM [B,H,N,dv]."""
    d = _dev(dM)
    B, H, N, dv = dM.shape
    if dM.dtype != torch.float32:
        raise ValueError("dM must be fp32")
    dM0 = _f32_out(out, (H, N, dv), d, "dM0")
    _check("sdm_state_init_backward", lib().sdm_state_init_backward(
        _ptr(dM), _ptr(dM0), B, H, N, dv, _stream(d)))
    return dM0
