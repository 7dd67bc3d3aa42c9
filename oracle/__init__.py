"""CPU oracle of the SDM hot path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package. The product path never does.

Thin numpy/ctypes wrapper over ``liboracle_sdm.so`` (plain C, see
``oracle_sdm.c``). Inputs are converted to contiguous fp32 / int32 host arrays
(bf16 tensors are widened exactly); outputs are fresh numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# SDM_ORACLE_SANITIZE=1 loads a build with AddressSanitizer and UBSan instead
# (the process must then preload the ASan runtime, see tests/test_oracle_sanitized.py)
SANITIZE = os.environ.get("SDM_ORACLE_SANITIZE") == "1"
LIB_PATH = os.path.join(HERE, "liboracle_sdm_san.so" if SANITIZE else "liboracle_sdm.so")
SRC = os.path.join(HERE, "oracle_sdm.c")

EQ4 = 0
FIG2 = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle_sdm.so with gcc (no fast-math, no FMA contraction), or
    with SDM_ORACLE_SANITIZE=1 the same source with AddressSanitizer and
    UndefinedBehaviorSanitizer (every UB report aborts) into liboracle_sdm_san.so."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"] \
            if SANITIZE else []
        cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-ffp-contract=off", "-fno-fast-math", *san,
               "-fPIC", "-shared", "-pthread", SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.oracle_half_scores.argtypes = [P, P, I64, I64, I64, I64, I64, P, I]
        lib.oracle_half_scores_idw.argtypes = [P, P, I64, I64, I64, I64, I64, P, I]
        lib.oracle_select.argtypes = [P, I64, I64, I64, I64, I64, P, P, P, P, I]
        lib.oracle_scan.argtypes = [P, P, I64, P, P, I64, P, P, P, P, P,
                                    I64, I64, I64, I64, I64, I, I]
        lib.oracle_scan_bf16.argtypes = [P, P, I64, P, P, I64, P, P, P, P, P,
                                         I64, I64, I64, I64, I64, I, I]
        lib.oracle_gates.argtypes = [P, P, P, P, P, I64, I64, I64, I64, P, P, I]
        lib.oracle_output_gate.argtypes = [P, P, P, ctypes.c_double, I64, I64, I64, I64, P, I]
        lib.oracle_scan_backward.argtypes = [P, P, I64, P, P, I64, P, P, P, P, P, P,
                                             P, P, P, P, P, P, I64, I64, I64, I64, I64, I, I]
        for f in (lib.oracle_half_scores, lib.oracle_half_scores_idw, lib.oracle_select,
                  lib.oracle_scan, lib.oracle_scan_bf16, lib.oracle_scan_backward,
                  lib.oracle_gates, lib.oracle_output_gate):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float32).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(x, dtype=np.float32)


def _i32(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.int32).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(x, dtype=np.int32)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


SCORINGS = ("dot", "idw")


def half_scores(q, subkeys, nthreads: Optional[int] = None, scoring: str = "dot") -> np.ndarray:
    """A1: q [B,H,T,2,dh], subkeys [H,2,n,dh] -> half-scores [B,H,T,2,n] fp32.

    scoring "dot": <q_j, K_j[a]> (SDM notes §2.3); "idw": -log(1e-3 + ||q_j - K_j[a]||^2)
    (FwPKM notes §2.2, inverse-distance weighting).
    """
    if scoring not in SCORINGS:
        raise ValueError(f"unknown scoring {scoring!r}")
    q = _f32(q); K = _f32(subkeys)
    B, H, T, two, dh = q.shape
    assert two == 2 and K.shape[0] == H and K.shape[1] == 2 and K.shape[3] == dh
    n = K.shape[2]
    out = np.empty((B, H, T, 2, n), np.float32)
    fn = _load().oracle_half_scores if scoring == "dot" else _load().oracle_half_scores_idw
    _check(fn(_p(q), _p(K), B, H, T, n, dh, _p(out), nthreads or default_threads()), "half_scores")
    return out


def select(half, k: int, nthreads: Optional[int] = None
           ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """A2-A4 on half-scores [B,H,T,2,n]: returns (idx, wt, score, score_next)."""
    half = _f32(half)
    B, H, T, two, n = half.shape
    assert two == 2
    idx = np.empty((B, H, T, k), np.int32)
    wt = np.empty((B, H, T, k), np.float32)
    sc = np.empty((B, H, T, k), np.float32)
    nxt = np.empty((B, H, T), np.float32)
    _check(_load().oracle_select(_p(half), B, H, T, n, k, _p(idx), _p(wt), _p(sc), _p(nxt),
                                 nthreads or default_threads()), "select")
    return idx, wt, sc, nxt


def address(q, subkeys, k: int, nthreads: Optional[int] = None, scoring: str = "dot"):
    """A1-A4: product-key addressing of one branch. Returns (idx, wt, score, score_next)."""
    return select(half_scores(q, subkeys, nthreads, scoring), k, nthreads)


def scan(idx_w, wt_w, idx_r, wt_r, alpha, beta, v, M_in, form: int = EQ4,
         nthreads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """A5-A6 over all tokens. M_in [B,H,N,dv] is not modified.

    Returns (M_out [B,H,N,dv], y [B,H,T,dv]).
    """
    iw = _i32(idx_w); ww = _f32(wt_w); ir = _i32(idx_r); wr = _f32(wt_r)
    a = _f32(alpha); b = _f32(beta); vv = _f32(v)
    M = np.array(_f32(M_in), dtype=np.float32, copy=True, order="C")
    B, H, T, W = iw.shape
    R = ir.shape[3]
    N, dv = M.shape[2], M.shape[3]
    assert M.shape[:2] == (B, H) and vv.shape == (B, H, T, dv)
    y = np.empty((B, H, T, dv), np.float32)
    _check(_load().oracle_scan(_p(iw), _p(ww), W, _p(ir), _p(wr), R, _p(a), _p(b), _p(vv),
                               _p(M), _p(y), B, H, T, N, dv, form,
                               nthreads or default_threads()), "scan")
    return M, y


def bf16_bits(x) -> np.ndarray:
    """The raw 16-bit patterns of a bfloat16 tensor (or a uint16 array as is)."""
    import torch
    if isinstance(x, torch.Tensor):
        if x.dtype != torch.bfloat16:
            raise ValueError("expected a bfloat16 tensor")
        return np.ascontiguousarray(x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))
    x = np.asarray(x)
    if x.dtype != np.uint16:
        raise ValueError("expected bfloat16 bits as uint16")
    return np.ascontiguousarray(x)


def bits_to_bf16(bits: np.ndarray):
    """uint16 bit patterns -> a CPU bfloat16 tensor (no rounding: the same bits)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16)


def scan_bf16(idx_w, wt_w, idx_r, wt_r, alpha, beta, v, M_in, form: int = EQ4,
              nthreads: Optional[int] = None):
    """A5-A6 with the table stored in bfloat16 (each stored element rounded once,
    to nearest even, from the double-precision update). M_in [B,H,N,dv] is a
    bfloat16 tensor (or its uint16 bits) and is not modified.

    Returns (M_out as a CPU bfloat16 tensor, y [B,H,T,dv] fp32).
    """
    iw = _i32(idx_w); ww = _f32(wt_w); ir = _i32(idx_r); wr = _f32(wt_r)
    a = _f32(alpha); b = _f32(beta); vv = _f32(v)
    Mb = np.array(bf16_bits(M_in), dtype=np.uint16, copy=True, order="C")
    B, H, T, W = iw.shape
    R = ir.shape[3]
    N, dv = Mb.shape[2], Mb.shape[3]
    assert Mb.shape[:2] == (B, H) and vv.shape == (B, H, T, dv)
    y = np.empty((B, H, T, dv), np.float32)
    _check(_load().oracle_scan_bf16(_p(iw), _p(ww), W, _p(ir), _p(wr), R, _p(a), _p(b), _p(vv),
                                    _p(Mb), _p(y), B, H, T, N, dv, form,
                                    nthreads or default_threads()), "scan_bf16")
    return bits_to_bf16(Mb), y


def scan_backward(idx_w, wt_w, idx_r, wt_r, alpha, beta, v, M_in, dy, dM_out=None,
                  form: int = EQ4, nthreads: Optional[int] = None) -> dict:
    """Reverse-mode derivatives of the scan ([SDM] §2.9 Appendix A: the tokens in
    reverse, each written row restored from its pre-image).

    M_in [B,H,N,dv] is the state before token 0, dy [B,H,T,dv] the gradient of y
    and dM_out [B,H,N,dv] (or None: zero) that of the final state. Returns a dict
    with dv [B,H,T,dv], dalpha, dbeta [B,H,T], dwt_w [B,H,T,W], dwt_r [B,H,T,R]
    and dM_in [B,H,N,dv]; inputs are not modified.
    """
    iw = _i32(idx_w); ww = _f32(wt_w); ir = _i32(idx_r); wr = _f32(wt_r)
    a = _f32(alpha); b = _f32(beta); vv = _f32(v); M = _f32(M_in); g = _f32(dy)
    gM = None if dM_out is None else _f32(dM_out)
    B, H, T, W = iw.shape
    R = ir.shape[3]
    N, dv = M.shape[2], M.shape[3]
    assert M.shape[:2] == (B, H) and vv.shape == (B, H, T, dv) and g.shape == vv.shape
    assert gM is None or gM.shape == M.shape
    out = {"dv": np.empty((B, H, T, dv), np.float32), "dalpha": np.empty((B, H, T), np.float32),
           "dbeta": np.empty((B, H, T), np.float32), "dwt_w": np.empty((B, H, T, W), np.float32),
           "dwt_r": np.empty((B, H, T, R), np.float32), "dM_in": np.empty((B, H, N, dv), np.float32)}
    _check(_load().oracle_scan_backward(
        _p(iw), _p(ww), W, _p(ir), _p(wr), R, _p(a), _p(b), _p(vv), _p(M), _p(g),
        None if gM is None else _p(gM), _p(out["dv"]), _p(out["dalpha"]), _p(out["dbeta"]),
        _p(out["dwt_w"]), _p(out["dwt_r"]), _p(out["dM_in"]), B, H, T, N, dv, form,
        nthreads or default_threads()), "scan_backward")
    return out


def gates(x, W_a, W_b, b_dt, A, nthreads: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """alpha, beta [B,H,T] from the layer input x [B,T,d] (SDM notes §2.4):
    alpha = exp(-A softplus(W_a x + b_dt)), beta = sigmoid(W_b x); W_a, W_b [H,d];
    b_dt, A [H]."""
    x = _f32(x); Wa = _f32(W_a); Wb = _f32(W_b); bd = _f32(b_dt); Af = _f32(A)
    B, T, d = x.shape
    H = Wa.shape[0]
    assert Wa.shape == (H, d) and Wb.shape == (H, d) and bd.shape == (H,) and Af.shape == (H,)
    al = np.empty((B, H, T), np.float32); be = np.empty((B, H, T), np.float32)
    _check(_load().oracle_gates(_p(x), _p(Wa), _p(Wb), _p(bd), _p(Af), B, T, d, H, _p(al), _p(be),
                                nthreads or default_threads()), "gates")
    return al, be


def output_gate(y, gamma, g, eps: float, nthreads: Optional[int] = None) -> np.ndarray:
    """o = y / sqrt(mean(y^2) + eps) * gamma[h] * sigmoid(g), per row of y [B,H,T,dv]."""
    yy = _f32(y); gm = _f32(gamma); gg = _f32(g)
    B, H, T, dv = yy.shape
    assert gm.shape == (H, dv) and gg.shape == yy.shape
    o = np.empty_like(yy)
    _check(_load().oracle_output_gate(_p(yy), _p(gm), _p(gg), float(eps), B, H, T, dv, _p(o),
                                      nthreads or default_threads()), "output_gate")
    return o


def broadcast_state(M0, B: int) -> np.ndarray:
    """The per-sequence initial state: M0 [H,N,dv] copied for each of B sequences."""
    M0 = _f32(M0)
    return np.ascontiguousarray(np.broadcast_to(M0[None], (B,) + M0.shape))
