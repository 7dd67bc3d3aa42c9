"""Seeded synthetic inputs for the SDM hot path (addressing + sparse delta scan).

This module only draws random numbers with fixed seeds and shapes. It holds
none of the method's arithmetic, so the CPU oracle and the HIP path can both
take their inputs from it.

Workloads (one per entry of ``WORKLOADS``). Shapes follow the SDM layer of the
Sparse Delta Memory notes, §2.2 (notation table: per head an N x d_v table,
W write and R read slots, scalar gates) and §2.3 (two half-queries of length
sqrt(N) scores each, realised here as half-queries of width d_h scored against
sqrt(N) subkeys). The large-table workload takes its sizes from the
Fast-weight Product Key Memory notes, §2.1 (512 x 256 subkey tables, a
262144 x 512 value table, top-8, one head).

Draw order for every workload (one ``torch.Generator`` seeded with the
workload's seed, fp32 draws):

1. subkeys ``[H, 2, n_sub, d_h]`` ~ N(0, 1)
2. (mixture workload only) centroids ``[H, n_centroids, 2*d_h]`` ~ N(0, 1),
   component ids ``[B, H, T]`` ~ Uniform{0..n_centroids-1}
3. q_w ``[B, H, T, 2, d_h]``: N(0, 1), or centroid + sigma * N(0, 1)
4. q_r ``[B, H, T, 2, d_h]``: same distribution (same component as q_w)
5. v ``[B, H, T, d_v]`` ~ N(0, 1)
6. alpha ``[B, H, T]`` = sigmoid(N(alpha_mu, 0.5))
7. beta ``[B, H, T]`` = sigmoid(N(0, 1))
8. M0 ``[H, N, d_v]`` ~ N(0, m0_std^2), or zeros when m0_std == 0

Tensors marked bf16 are drawn in fp32 and rounded to nearest-even bf16; both
sides of a parity check receive the same bits (the oracle widens them
exactly to fp32).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    n_sub: int          # subkeys per half; N = n_sub ** 2 slots per head
    d_v: int
    d_h: int            # half-query / subkey width
    W: int
    R: int
    bf16_inputs: bool   # q, v and subkeys stored as bf16
    m0_std: float
    alpha_mu: float
    seed: int
    n_centroids: int = 0   # > 0: addressing vectors drawn from a Gaussian mixture
    sigma: float = 0.5     # mixture noise scale

    @property
    def N(self) -> int:
        return self.n_sub * self.n_sub

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    # tiny oracle check; the dense variant selects every slot (W = R = N)
    "tiny": Workload("tiny", 1, 1, 256, 16, 16, 8, 8, 8, False, 0.02, 2.0, 0),
    "tiny_dense": Workload("tiny_dense", 1, 1, 256, 16, 16, 8, 256, 256, False, 0.02, 2.0, 0),
    # small layer, fp32 everywhere, zero initial table
    "small": Workload("small", 4, 4, 4096, 64, 64, 32, 16, 16, False, 0.0, 2.0, 1),
    # GDN-matched layer: N = 65536, W = R = 64, d_v = 128, bf16 q/v/subkeys
    "gdn_matched": Workload("gdn_matched", 4, 8, 8192, 256, 128, 64, 64, 64, True, 0.02, 2.0, 2),
    # long-context scan with skewed slot reuse (1024-centroid mixture keys)
    "long_context": Workload("long_context", 1, 8, 131072, 256, 128, 64, 64, 64, True, 0.02, 2.0, 3,
                             n_centroids=1024, sigma=0.5),
    # large table at the FwPKM value-table size (512 MB fp32 table)
    "large_table": Workload("large_table", 1, 1, 65536, 512, 512, 256, 8, 8, False, 0.02, 3.0, 4),
    # decoding: 256 sequences of the GDN-matched layer, one token per sequence
    # per call (T = the number of calls), the 64 GiB state kept between calls
    "decode": Workload("decode", 256, 8, 32, 256, 128, 64, 64, 64, True, 0.02, 2.0, 5),
}


def get(name: str, **overrides) -> Workload:
    """Workload ``name`` with optional field overrides (e.g. a shorter T)."""
    return WORKLOADS[name].with_(**overrides) if overrides else WORKLOADS[name]


def make_inputs(wl: Workload, seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Draw the CPU input tensors of workload ``wl``.

    Returns a dict with ``subkeys, q_w, q_r, v`` (bf16 or fp32), ``alpha, beta``
    (fp32, [B,H,T]) and ``M0`` (fp32, [H,N,d_v]). The same subkey table serves
    both branches (the write and read projections of the pages are separate,
    the ABI accepts two tables; one table per head is drawn here).
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(wl.seed if seed is None else seed)
    B, H, T, n, dh, dv = wl.B, wl.H, wl.T, wl.n_sub, wl.d_h, wl.d_v
    f32 = torch.float32

    subkeys = torch.randn((H, 2, n, dh), generator=g, dtype=f32)
    if wl.n_centroids > 0:
        cent = torch.randn((H, wl.n_centroids, 2 * dh), generator=g, dtype=f32)
        comp = torch.randint(0, wl.n_centroids, (B, H, T), generator=g)
        hsel = torch.arange(H).view(1, H, 1).expand(B, H, T)
        mu = cent[hsel, comp].view(B, H, T, 2, dh)
        q_w = mu + wl.sigma * torch.randn((B, H, T, 2, dh), generator=g, dtype=f32)
        q_r = mu + wl.sigma * torch.randn((B, H, T, 2, dh), generator=g, dtype=f32)
        del mu
    else:
        q_w = torch.randn((B, H, T, 2, dh), generator=g, dtype=f32)
        q_r = torch.randn((B, H, T, 2, dh), generator=g, dtype=f32)
    v = torch.randn((B, H, T, dv), generator=g, dtype=f32)
    alpha = torch.sigmoid(torch.randn((B, H, T), generator=g, dtype=f32) * 0.5 + wl.alpha_mu)
    beta = torch.sigmoid(torch.randn((B, H, T), generator=g, dtype=f32))
    if wl.m0_std > 0:
        M0 = torch.randn((H, wl.N, dv), generator=g, dtype=f32) * wl.m0_std
    else:
        M0 = torch.zeros((H, wl.N, dv), dtype=f32)

    if wl.bf16_inputs:
        subkeys = subkeys.to(torch.bfloat16)
        q_w = q_w.to(torch.bfloat16)
        q_r = q_r.to(torch.bfloat16)
        v = v.to(torch.bfloat16)
    return {"subkeys": subkeys.contiguous(), "q_w": q_w.contiguous(), "q_r": q_r.contiguous(),
            "v": v.contiguous(), "alpha": alpha.contiguous(), "beta": beta.contiguous(),
            "M0": M0.contiguous()}


def d_model(wl: Workload) -> int:
    """Model width d of the layer around the path: d = H * d_v, the relation of
    the SDM notes' own configuration (§2.8: d = 1920 with H = 2, d_v = 960)."""
    return wl.H * wl.d_v


def make_glue_inputs(wl: Workload, d: Optional[int] = None, seed: Optional[int] = None
                     ) -> Dict[str, torch.Tensor]:
    """Inputs of the glue either side of the scan (own generator, seed + 1000, so
    the scan inputs above are unchanged). Draw order (fp32 draws):

    1. x ``[B, T, d]`` ~ N(0, 1)                       (layer input)
    2. W_a ``[H, d]``, 3. W_b ``[H, d]`` ~ N(0, 1/d)   (gate projections)
    4. b_dt ``[H]`` = -2.5 + 0.1 N(0, 1)               (mean alpha ~ 0.9)
    5. A ``[H]`` = exp(0.1 N(0, 1))                    (positive decay rates)
    6. g ``[B, H, T, d_v]`` ~ N(0, 1)                  (output-gate pre-activation)
    7. gamma ``[H, d_v]`` = 1 + 0.1 N(0, 1)            (RMS-Norm scale)

    x, W_a, W_b and g are rounded to bf16 where the workload's inputs are bf16.
    """
    d = d_model(wl) if d is None else d
    g = torch.Generator(device="cpu")
    g.manual_seed((wl.seed if seed is None else seed) + 1000)
    B, H, T, dv = wl.B, wl.H, wl.T, wl.d_v
    f32 = torch.float32
    x = torch.randn((B, T, d), generator=g, dtype=f32)
    W_a = torch.randn((H, d), generator=g, dtype=f32) / d ** 0.5
    W_b = torch.randn((H, d), generator=g, dtype=f32) / d ** 0.5
    b_dt = -2.5 + 0.1 * torch.randn((H,), generator=g, dtype=f32)
    A = torch.exp(0.1 * torch.randn((H,), generator=g, dtype=f32))
    gate = torch.randn((B, H, T, dv), generator=g, dtype=f32)
    gamma = 1.0 + 0.1 * torch.randn((H, dv), generator=g, dtype=f32)
    if wl.bf16_inputs:
        x, W_a, W_b, gate = (t.to(torch.bfloat16) for t in (x, W_a, W_b, gate))
    return {"x": x.contiguous(), "W_a": W_a.contiguous(), "W_b": W_b.contiguous(),
            "b_dt": b_dt.contiguous(), "A": A.contiguous(), "g": gate.contiguous(),
            "gamma": gamma.contiguous()}


def input_recipe(wl: Workload) -> Dict[str, object]:
    """Plain description of a workload's input recipe (for result records)."""
    d = dataclasses.asdict(wl)
    d["N"] = wl.N
    d["keys"] = (f"{wl.n_centroids}-centroid Gaussian mixture, sigma={wl.sigma}"
                 if wl.n_centroids else "iid N(0,1)")
    return d
