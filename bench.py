#!/usr/bin/env python3
"""Benchmark of the SDM hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
per-sequence table init from M0, product-key addressing of both branches, and
the sparse gated delta scan (planner + scan kernels). Inputs are resident in
HBM before the timed region; outputs are preallocated.

Prints ONE JSON line: throughput (tokens/s = B*T per step), the scan's roofline
entry (algorithmic slot-row bytes B*H*T*(2W+R)*d_v*4 per launch over the
launch's average duration from HIP events) and the CPU oracle timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SDM scan tokens/s and slot-row HBM GB/s at N=65536,W=R=64,d_v=128"
HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_traffic_{}.json")
# the sources the scan kernels are compiled from: the counter summary holds for them only
SCAN_SRCS = [os.path.join(ROOT, "sparse_memory_linear_amd", "csrc", f) for f in ("scan.hip", "sdm_buffer.h")]


def scan_source_sha256() -> str:
    """SHA-256 of the scan sources' code: each line with its // comment and
    trailing blanks removed, blank lines dropped (comment edits keep the hash)."""
    h = hashlib.sha256()
    for path in SCAN_SRCS:
        with open(path, encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="gdn_matched")
    p.add_argument("--form", default="eq4", choices=["eq4", "fig2"])
    p.add_argument("--table", default="f32", choices=["f32", "bf16"],
                   help="element type of the state table (bf16 halves every row access)")
    p.add_argument("--scoring", default="dot", choices=["dot", "idw"],
                   help="subkey score of the addressing: dot product, or FwPKM's inverse distance")
    p.add_argument("--cpu-seconds", type=float, default=20.0,
                   help="target CPU time of the oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--glue", action="store_true",
                   help="layer step: gates from the layer input, then addressing and scan, then the "
                        "per-head RMS-Norm and output gate")
    p.add_argument("--train", action="store_true",
                   help="training step: addressing, forward with pre-images, backward with undo")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the extra entries of the default line (shared-residual scan, long-context scan "
                        "and its slot-reuse statistics)")
    p.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                   help="run one plain device copy of BYTES bytes before the benchmark "
                        "(a known-size kernel that calibrates HBM byte counters)")
    return p.parse_args()


def host_cpu() -> str:
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True).stdout
        for line in out.splitlines():
            if line.startswith("Model name"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return platform.processor() or "unknown"


def host_facts() -> dict:
    """What the host reports: nproc (the CPUs this process may use), os.cpu_count()
    and the lscpu model name."""
    try:
        nproc = int(subprocess.run(["nproc"], capture_output=True, text=True).stdout.strip())
    except Exception:
        nproc = None
    lscpu = {}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True).stdout
        for line in out.splitlines():
            k, _, v = line.partition(":")
            if k.strip() in ("Model name", "CPU family", "Model", "Thread(s) per core", "Core(s) per socket",
                             "Socket(s)", "CPU max MHz", "L3 cache"):
                lscpu[k.strip()] = v.strip()
    except Exception:
        pass
    return {"nproc": nproc, "cpu_count": os.cpu_count(), "host_cpu": host_cpu(), "lscpu": lscpu}


def pct(xs, q: float) -> float:
    """q-th percentile (nearest rank) of a list of timings."""
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(q / 100.0 * (len(xs) - 1)))))]


def stats(xs) -> dict:
    return {"median": pct(xs, 50), "p10": pct(xs, 10), "p90": pct(xs, 90), "n": len(xs)}


def slot_reuse(idx, N: int, window: int = 32768) -> dict:
    """Slot-reuse statistics of one branch's slots idx [B, H, T, k] with FwPKM's
    definitions (its ablation table: per 32K-token window, then averaged):
    coverage = fraction of the N slots accessed; collision = fraction of the
    accesses that land on a slot accessed more than once; KLD = KL divergence of
    the access distribution from the uniform one (natural log)."""
    import numpy as np
    idx = idx.reshape(-1, idx.shape[-2], idx.shape[-1])  # [streams, T, k]
    cov, col, kld = [], [], []
    for st in range(idx.shape[0]):
        for t0 in range(0, idx.shape[1], window):
            c = np.bincount(idx[st, t0:t0 + window].reshape(-1).astype(np.int64), minlength=N)
            n = c.sum()
            p = c[c > 0] / n
            cov.append((c > 0).mean())
            col.append(c[c > 1].sum() / n)
            kld.append(float((p * np.log(p * N)).sum()))
    f = lambda v: {"mean": float(np.mean(v)), "min": float(np.min(v)), "max": float(np.max(v))}
    return {"window_tokens": window, "windows": len(cov), "coverage": f(cov), "collision": f(col), "kld": f(kld)}


def measured_traffic(workload: str = "gdn_matched"):
    """HBM bytes per scan launch from the committed counter summary of this
    workload, if it was taken on the current scan kernel source."""
    try:
        with open(TRAFFIC_FILE.format(workload)) as f:
            rec = json.load(f)
        if rec.get("scan_source_sha256") == scan_source_sha256():
            return rec.get("traffic_bytes_per_launch")
    except (OSError, ValueError):
        pass
    return None


def cpu_baseline(wl, x, target_s: float, scoring: str = "dot", table: str = "f32", gx=None,
                 single_s: float = 0.0):
    """The oracle as it is (addressing of both branches + scan) on a bounded
    sample of the same workload: the first B' sequences with all H heads, or
    the first T' tokens of one sequence when a whole one already exceeds the
    target; the sample is sized from a short calibration run to ~target_s."""
    import math
    import oracle

    nthreads = oracle.default_threads()

    def run(nb, Tp):
        sl = lambda t: t[:nb, :, :Tp].contiguous()
        t0 = time.perf_counter()
        al, be = sl(x["alpha"]), sl(x["beta"])
        if gx is not None:
            al, be = oracle.gates(gx["x"][:nb, :Tp].contiguous(), gx["W_a"], gx["W_b"], gx["b_dt"], gx["A"], nthreads)
        iw, ww, _, _ = oracle.address(sl(x["q_w"]), x["subkeys"], wl.W, nthreads, scoring)
        ir, wr, _, _ = oracle.address(sl(x["q_r"]), x["subkeys"], wl.R, nthreads, scoring)
        M_in = oracle.broadcast_state(x["M0"].numpy(), nb)
        if table == "bf16":
            import torch
            _, y = oracle.scan_bf16(iw, ww, ir, wr, al, be, sl(x["v"]),
                                    torch.from_numpy(M_in.copy()).to(torch.bfloat16), oracle.EQ4, nthreads)
        else:
            _, y = oracle.scan(iw, ww, ir, wr, al, be, sl(x["v"]), M_in, oracle.EQ4, nthreads)
        if gx is not None:
            oracle.output_gate(y, gx["gamma"], sl(gx["g"]), 1e-6, nthreads)
        return time.perf_counter() - t0

    # two calibration points separate the per-call fixed cost from the per-token cost
    T1, T2 = min(wl.T, 64), min(wl.T, 512)
    t1, t2 = run(1, T1), run(1, T2)
    per_tok = max((t2 - t1) / max(T2 - T1, 1), t2 / T2 * 0.1, 1e-6)
    want = max(target_s - max(t1 - T1 * per_tok, 0.0), 0.0) / per_tok
    if want <= wl.T:
        nb, Tp = 1, max(T2, int(want))
    else:
        nb, Tp = min(wl.B, max(1, math.ceil(want / wl.T))), wl.T
    ts = run(nb, Tp) if (nb, Tp) != (1, T2) else t2
    rec = {"value": nb * Tp / ts, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
           "sample": f"{nb} of {wl.B} sequences of {wl.name}, all {wl.H} heads, first {Tp} of "
                     f"{wl.T} tokens ({'gates + ' if gx is not None else ''}{scoring} addressing of both "
                     f"branches + EQ4 scan, {table} table{' + output gate' if gx is not None else ''}), "
                     f"{ts:.1f} s wall",
           "threads_note": "the pool takes the GPU box's CPU share for one GPU (16 threads), "
                           "whatever nproc reports",
           **host_facts()}
    if single_s > 0:
        # the same oracle on one thread, first T1 tokens of one sequence sized to ~single_s
        nthreads_saved = nthreads
        nthreads = 1
        t1s = run(1, T1)
        per1 = max(t1s / T1, 1e-6)
        T1p = int(min(wl.T, max(T1, single_s / per1)))
        t1p = run(1, T1p) if T1p != T1 else t1s
        nthreads = nthreads_saved
        rec["single_thread"] = {"value": T1p / t1p, "unit": "tokens/s", "cores": 1,
                                "sample": f"1 sequence, all {wl.H} heads, first {T1p} tokens, {t1p:.1f} s wall"}
    return rec


def cpu_baseline_train(wl, x, dy, target_s: float, scoring: str = "dot"):
    """The oracle's training step (addressing of both branches + its backward,
    which runs its forward first) on a bounded sample: the first T' tokens of
    the first sequence, all heads, T' sized from a calibration run."""
    import oracle

    nthreads = oracle.default_threads()

    def run(Tp):
        sl = lambda t: t[:1, :, :Tp].contiguous()
        t0 = time.perf_counter()
        iw, ww, _, _ = oracle.address(sl(x["q_w"]), x["subkeys"], wl.W, nthreads, scoring)
        ir, wr, _, _ = oracle.address(sl(x["q_r"]), x["subkeys"], wl.R, nthreads, scoring)
        oracle.scan_backward(iw, ww, ir, wr, sl(x["alpha"]), sl(x["beta"]), sl(x["v"]),
                             oracle.broadcast_state(x["M0"].numpy(), 1), dy[:1, :, :Tp],
                             None, oracle.EQ4, nthreads)
        return time.perf_counter() - t0

    T1, T2 = min(wl.T, 64), min(wl.T, 512)
    t1, t2 = run(T1), run(T2)
    per_tok = max((t2 - t1) / max(T2 - T1, 1), t2 / T2 * 0.1, 1e-6)
    Tp = int(min(wl.T, max(T2, (target_s - max(t1 - T1 * per_tok, 0.0)) / per_tok)))
    ts = run(Tp) if Tp != T2 else t2
    return {"value": Tp / ts, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"1 of {wl.B} sequences of {wl.name}, all {wl.H} heads, first {Tp} of {wl.T} "
                      f"tokens ({scoring} addressing of both branches + EQ4 forward and backward), {ts:.1f} s wall",
            **host_facts()}


def train_bench(a, wl, x, dev):
    """Training: one step = table init, addressing of both branches, the forward
    that stores pre-images, zeroing dL/dM of the final state, the backward that
    undoes the forward, and the initial state's gradient (sum over sequences)."""
    import torch
    import sparse_memory_linear_amd as sdm

    g = {k: v.to(dev) for k, v in x.items()}
    B, H, T, N, dv, W, R = wl.B, wl.H, wl.T, wl.N, wl.d_v, wl.W, wl.R
    gen = torch.Generator().manual_seed(1234)
    dy_host = torch.randn((B, H, T, dv), generator=gen)
    dy = dy_host.to(dev)
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
    addr_out = (torch.empty((B, H, T, W), dtype=torch.int32, device=dev), f32(B, H, T, W),
                torch.empty((B, H, T, R), dtype=torch.int32, device=dev), f32(B, H, T, R))
    M, dM, y, snap = f32(B, H, N, dv), f32(B, H, N, dv), f32(B, H, T, dv), f32(B, H, T, W, dv)
    grads = {"dv": f32(B, H, T, dv), "dalpha": f32(B, H, T), "dbeta": f32(B, H, T),
             "dwt_w": f32(B, H, T, W), "dwt_r": f32(B, H, T, R)}
    dM0 = f32(H, N, dv)
    ws_f = torch.empty((sdm.sdm_scan_workspace_bytes(B, H, T, W, R, dv),), dtype=torch.uint8, device=dev)
    ws_b = torch.empty((sdm.sdm_scan_backward_workspace_bytes(B, H, T, W, R, dv),), dtype=torch.uint8,
                       device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    NM = 7

    def step(marks=None):
        rec = (lambda i: marks[i].record()) if marks else (lambda i: None)
        rec(0)
        sdm.sdm_state_init(g["M0"], B, out=M)
        rec(1)
        iw, ww, ir, wr = sdm.sdm_address(g["q_w"], g["q_r"], g["subkeys"], g["subkeys"], W, R, out=addr_out,
                                         scoring=a.scoring)
        rec(2)
        args = (iw, ww, ir, wr, g["alpha"], g["beta"], g["v"])
        sdm.sdm_scan_forward_save(*args, M, a.form, y=y, snap=snap, workspace=ws_f)
        rec(3)
        dM.zero_()
        rec(4)
        sdm.sdm_scan_backward(*args, snap, dy, M, dM, a.form, out=grads, workspace=ws_b)
        rec(5)
        sdm.sdm_state_init_backward(dM, out=dM0)
        rec(6)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    marks = [[ev() for _ in range(NM)] for _ in range(a.steps)]
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(marks[i])
    torch.cuda.synchronize()
    ms_step = 1e3 * (time.perf_counter() - t0) / a.steps
    part = lambda i: sum(m[i].elapsed_time(m[i + 1]) for m in marks) / a.steps
    names = ["state_init", "address", "forward_save", "dM_zero", "backward", "state_init_backward"]
    br = {n: part(i) for i, n in enumerate(names)}
    th = B * H * T
    fwd_bytes = th * (3 * W + R) * dv * 4     # gather W, scatter W, store W pre-images, gather R
    bwd_bytes = th * (4 * W + 3 * R) * dv * 4  # G, pre-image in and G, M out per write; M, G in, G out per read
    bwd_gbps = bwd_bytes / (br["backward"] * 1e-3) / 1e9
    rec = {
        "metric": "SDM training tokens/s (addressing + forward with pre-images + backward with undo) "
                  "at N=65536,W=R=64,d_v=128",
        "value": B * T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "H": H, "T": T, "N": N, "W": W, "R": R, "d_v": dv,
                   "d_h": wl.d_h, "form": a.form, "scoring": a.scoring, "mode": "train",
                   "inputs": "bf16 q/v/subkeys, fp32 table/gates/gradients" if wl.bf16_inputs else "fp32"},
        "breakdown_ms": br,
        "forward_save_GBps": fwd_bytes / (br["forward_save"] * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "achieved": bwd_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": bwd_gbps / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "sdm_scan_backward (bwd_plan_kernel + scan_backward_kernel + bwd_partials_reduce)",
                     "algorithmic_bytes_per_launch": bwd_bytes},
    }
    if not a.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_train(wl, x, dy_host.numpy(), a.cpu_seconds, a.scoring)
    print(json.dumps(rec), flush=True)


def decode_bench(a, wl, x, dev):
    """Decoding: each step feeds one token of every sequence through addressing
    and the scan (a call with T = 1), the state staying resident between steps."""
    import torch
    import sparse_memory_linear_amd as sdm

    B, H, N, dv, W, R = wl.B, wl.H, wl.N, wl.d_v, wl.W, wl.R
    nsteps = a.warmup + a.steps
    if nsteps > wl.T:
        sys.exit(f"decode: warmup + steps must be at most {wl.T}")
    sub = x["subkeys"].to(dev)
    tok = lambda key, k: x[key][:, :, k:k + 1].contiguous().to(dev)
    per = [{key: tok(key, k) for key in ("q_w", "q_r", "alpha", "beta", "v")} for k in range(nsteps)]
    tdt = torch.bfloat16 if a.table == "bf16" else torch.float32
    M = sdm.sdm_state_init(x["M0"].to(dev), B, dtype=tdt)
    addr_out = (torch.empty((B, H, 1, W), dtype=torch.int32, device=dev),
                torch.empty((B, H, 1, W), dtype=torch.float32, device=dev),
                torch.empty((B, H, 1, R), dtype=torch.int32, device=dev),
                torch.empty((B, H, 1, R), dtype=torch.float32, device=dev))
    y = torch.empty((B, H, 1, dv), dtype=torch.float32, device=dev)
    ws = torch.empty((sdm.sdm_scan_workspace_bytes(B, H, 1, W, R, dv),), dtype=torch.uint8, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def step(k, marks=None):
        i = per[k]
        if marks:
            marks[0].record()
        iw, ww, ir, wr = sdm.sdm_address(i["q_w"], i["q_r"], sub, sub, W, R, out=addr_out, scoring=a.scoring)
        if marks:
            marks[1].record()
        sdm.sdm_scan_forward(iw, ww, ir, wr, i["alpha"], i["beta"], i["v"], M, a.form, y=y, workspace=ws)
        if marks:
            marks[2].record()

    for k in range(a.warmup):
        step(k)
    torch.cuda.synchronize()
    marks = [[ev() for _ in range(3)] for _ in range(a.steps)]
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(a.warmup + i, marks[i])
    torch.cuda.synchronize()
    ms_step = 1e3 * (time.perf_counter() - t0) / a.steps
    addr_ms = sum(m[0].elapsed_time(m[1]) for m in marks) / a.steps
    scan_ms = sum(m[1].elapsed_time(m[2]) for m in marks) / a.steps
    row_bytes = B * H * (2 * W + R) * dv * (2 if a.table == "bf16" else 4)
    gbps = row_bytes / (scan_ms * 1e-3) / 1e9
    rec = {
        "metric": "SDM decode tokens/s at N=65536,W=R=64,d_v=128 (one token per sequence per step)",
        "value": B / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "H": H, "T_per_step": 1, "N": N, "W": W, "R": R, "d_v": dv,
                   "d_h": wl.d_h, "form": a.form, "scoring": a.scoring, "table": a.table,
                   "inputs": f"bf16 q/v/subkeys, {a.table} table, fp32 gates",
                   "state_GiB": B * H * N * dv * (2 if a.table == "bf16" else 4) / 2**30},
        "breakdown_ms": {"address": addr_ms, "scan": scan_ms},
        "slot_row_GBps": gbps,
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": None,
                     "kernel": "sdm_scan_forward (direct short-call form)",
                     "algorithmic_bytes_per_launch": row_bytes},
    }
    if not a.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl, x, a.cpu_seconds, a.scoring, a.table)
    print(json.dumps(rec), flush=True)


def main():
    a = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus > 1 or world > 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(the per-(sequence, head) streams would shard with no exchange; "
              "see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_memory_linear_amd as sdm
    from sparse_memory_linear_amd import inputs

    dev = torch.device("cuda:0")
    if a.copy_probe > 0:
        src = torch.ones(a.copy_probe // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    wl = inputs.get(a.workload)
    x = inputs.make_inputs(wl)
    if wl.name == "decode":
        return decode_bench(a, wl, x, dev)
    if a.train:
        if a.table != "f32":
            sys.exit("training keeps an fp32 table (the backward restores fp32 pre-images)")
        return train_bench(a, wl, x, dev)
    g = {k: v.to(dev) for k, v in x.items()}
    B, H, T, N, dv, W, R = wl.B, wl.H, wl.T, wl.N, wl.d_v, wl.W, wl.R
    addr_out = (torch.empty((B, H, T, W), dtype=torch.int32, device=dev),
                torch.empty((B, H, T, W), dtype=torch.float32, device=dev),
                torch.empty((B, H, T, R), dtype=torch.int32, device=dev),
                torch.empty((B, H, T, R), dtype=torch.float32, device=dev))
    esz = 2 if a.table == "bf16" else 4
    M = torch.empty((B, H, N, dv), dtype=torch.bfloat16 if a.table == "bf16" else torch.float32, device=dev)
    y = torch.empty((B, H, T, dv), dtype=torch.float32, device=dev)
    ws = torch.empty((sdm.sdm_scan_workspace_bytes(B, H, T, W, R, dv),), dtype=torch.uint8, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    if a.glue:
        gx = {k: v.to(dev) for k, v in inputs.make_glue_inputs(wl).items()}
        gates_out = (torch.empty((B, H, T), dtype=torch.float32, device=dev),
                     torch.empty((B, H, T), dtype=torch.float32, device=dev))
        o = torch.empty((B, H, T, dv), dtype=torch.float32, device=dev)
        wsg = torch.empty((sdm.sdm_scan_gated_workspace_bytes(B, H, T, W, R, dv),), dtype=torch.uint8, device=dev)
    NM = 5 if a.glue else 4

    def step(marks=None):
        rec = (lambda i: marks[i].record()) if marks else (lambda i: None)
        rec(0)
        sdm.sdm_state_init(g["M0"], B, out=M)
        rec(1)
        if a.glue:
            al, be = sdm.sdm_gates(gx["x"], gx["W_a"], gx["W_b"], gx["b_dt"], gx["A"], out=gates_out)
            rec(4)
        else:
            al, be = g["alpha"], g["beta"]
        iw, ww, ir, wr = sdm.sdm_address(g["q_w"], g["q_r"], g["subkeys"], g["subkeys"], W, R, out=addr_out,
                                         scoring=a.scoring)
        rec(2)
        if a.glue:  # the scan with the output step (RMS-Norm + gate) fused into its last pass
            sdm.sdm_scan_forward_gated(iw, ww, ir, wr, al, be, g["v"], M, gx["gamma"], gx["g"], 1e-6, a.form,
                                       out=o, workspace=wsg)
        else:
            sdm.sdm_scan_forward(iw, ww, ir, wr, al, be, g["v"], M, a.form, y=y, workspace=ws)
        rec(3)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    marks = [[ev() for _ in range(NM)] for _ in range(a.steps)]
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(marks[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = 1e3 * wall / a.steps
    init_ms = sum(m[0].elapsed_time(m[1]) for m in marks) / a.steps
    addr_ms = sum(m[4 if a.glue else 1].elapsed_time(m[2]) for m in marks) / a.steps
    scan_each = [m[2].elapsed_time(m[3]) for m in marks]
    scan_ms = sum(scan_each) / a.steps
    breakdown = {"state_init": init_ms, "address": addr_ms, "scan": scan_ms}
    glue = None
    if a.glue:
        gates_ms = sum(m[1].elapsed_time(m[4]) for m in marks) / a.steps
        breakdown["gates"] = gates_ms
        breakdown["scan_gated"] = breakdown.pop("scan")
        dm = inputs.d_model(wl)
        xb = 2 if wl.bf16_inputs else 4
        gate_bytes = B * T * dm * xb + 2 * B * H * T * 4          # x in, alpha and beta out
        glue = {"d_model": dm,
                "gates_GBps": gate_bytes / (gates_ms * 1e-3) / 1e9,
                "gates_mfma_TFLOPs": 2 * B * T * dm * 2 * H / (gates_ms * 1e-3) / 1e12,
                "output_step": output_step_entry(sdm, g, gx, M, y, o, ws, wsg, addr_out, a.form)}

    row_bytes = B * H * T * (2 * W + R) * dv * esz
    scan_gbps = row_bytes / (scan_ms * 1e-3) / 1e9
    rec = {
        "metric": METRIC,
        "value": B * T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "H": H, "T": T, "N": N, "W": W, "R": R,
                   "d_v": dv, "d_h": wl.d_h, "form": a.form, "scoring": a.scoring, "table": a.table,
                   "inputs": (f"bf16 q/v/subkeys, {a.table} table, fp32 gates" if wl.bf16_inputs
                              else f"fp32 inputs, {a.table} table")},
        "breakdown_ms": breakdown,
        # the half-score contraction of both branches: 2 halves x n_sub x d_h MACs per token-branch
        "address_mfma_TFLOPs": 2 * B * H * T * 2 * (2 * wl.n_sub * wl.d_h) / (addr_ms * 1e-3) / 1e12,
        "scan_tokens_per_s": B * T / (scan_ms * 1e-3),
        "scan_ms_per_step": stats(scan_each),
        "slot_row_GBps": scan_gbps,
        "roofline": {"bound": "hbm", "achieved": scan_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": scan_gbps / HBM_PEAK_GBPS,
                     # the counters were taken on this configuration (dot-product addressing
                     # decides which rows the scan touches)
                     "traffic": measured_traffic()
                     if (a.table, a.form, a.scoring, wl.name) == ("f32", "eq4", "dot", "gdn_matched") else None,
                     "kernel": "sdm_scan_forward (plan_kernel + scan_kernel + ypart_reduce)",
                     "algorithmic_bytes_per_launch": row_bytes},
    }
    if glue:
        rec["glue"] = glue
        rec["config"]["mode"] = "layer (gates + addressing + scan with the output gate fused)"
    default_line = (wl.name, a.form, a.table, a.scoring, a.glue) == ("gdn_matched", "eq4", "f32", "dot", False)
    if default_line and not a.no_extras:
        # the shared-residual form on the same slots, then the long-context workload
        rec["fig2_scan"] = scan_entry(sdm, g, M, y, ws, addr_out, "fig2", row_bytes, reps=7)
        del g, M, y, ws, addr_out
        torch.cuda.empty_cache()
        rec["long_context_scan"] = long_context_entry(sdm, inputs, dev)
    if not a.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl, x, a.cpu_seconds, a.scoring, a.table,
                                           inputs.make_glue_inputs(wl) if a.glue else None,
                                           single_s=8.0 if default_line else 0.0)
    print(json.dumps(rec), flush=True)


def output_step_entry(sdm, g, gx, M, y, o, ws, wsg, addr_out, form: str, reps: int = 5) -> dict:
    """What the output step (RMS-Norm + gate) adds to the scan, fused into the
    scan's last pass and as a separate kernel after it: medians of reps calls on
    a fresh table each, HIP events on the current stream."""
    import torch
    iw, ww, ir, wr = addr_out
    B = M.shape[0]
    calls = {
        "scan": lambda: sdm.sdm_scan_forward(iw, ww, ir, wr, g["alpha"], g["beta"], g["v"], M, form, y=y,
                                             workspace=ws),
        "scan_gated": lambda: sdm.sdm_scan_forward_gated(iw, ww, ir, wr, g["alpha"], g["beta"], g["v"], M,
                                                         gx["gamma"], gx["g"], 1e-6, form, out=o, workspace=wsg),
        "scan_then_output_gate": lambda: (calls["scan"](), sdm.sdm_output_gate(y, gx["gamma"], gx["g"], 1e-6,
                                                                               out=o)),
    }
    med = {}
    for name, fn in calls.items():
        times = []
        for i in range(reps + 1):
            sdm.sdm_state_init(g["M0"], B, out=M)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            if i:
                times.append(e0.elapsed_time(e1))
        med[name] = stats(times)["median"]
    return {"ms": med, "fused_extra_ms": med["scan_gated"] - med["scan"],
            "separate_extra_ms": med["scan_then_output_gate"] - med["scan"]}


def scan_entry(sdm, g, M, y, ws, addr_out, form: str, row_bytes: int, reps: int) -> dict:
    """sdm_scan_forward on resident inputs: reps calls after one warm-up, each on a
    fresh table from M0 (untimed), timed with HIP events on the current stream."""
    import torch
    iw, ww, ir, wr = addr_out
    B = M.shape[0]
    times = []
    for i in range(reps + 1):
        sdm.sdm_state_init(g["M0"], B, out=M)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        sdm.sdm_scan_forward(iw, ww, ir, wr, g["alpha"], g["beta"], g["v"], M, form, y=y, workspace=ws)
        e1.record()
        e1.synchronize()
        if i:
            times.append(e0.elapsed_time(e1))
    st = stats(times)
    gbps = row_bytes / (st["median"] * 1e-3) / 1e9
    return {"form": form, "ms": st, "slot_row_GBps": gbps, "frac": gbps / HBM_PEAK_GBPS,
            "algorithmic_bytes_per_launch": row_bytes}


def long_context_entry(sdm, inputs, dev) -> dict:
    """The long-context workload (B=1, H=8, T=131072, N=65536, W=R=64, d_v=128,
    mixture keys, EQ4, fp32 table): addressing once, then the scan timed like the
    default line's, and the slot-reuse statistics of both branches' slots."""
    import torch
    wl = inputs.get("long_context")
    x = inputs.make_inputs(wl)
    g = {k: v.to(dev) for k, v in x.items()}
    del x
    B, H, T, N, dv, W, R = wl.B, wl.H, wl.T, wl.N, wl.d_v, wl.W, wl.R
    out = (torch.empty((B, H, T, W), dtype=torch.int32, device=dev),
           torch.empty((B, H, T, W), dtype=torch.float32, device=dev),
           torch.empty((B, H, T, R), dtype=torch.int32, device=dev),
           torch.empty((B, H, T, R), dtype=torch.float32, device=dev))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sdm.sdm_address(g["q_w"], g["q_r"], g["subkeys"], g["subkeys"], W, R, out=out)
    e0.record()
    sdm.sdm_address(g["q_w"], g["q_r"], g["subkeys"], g["subkeys"], W, R, out=out)
    e1.record()
    e1.synchronize()
    addr_ms = e0.elapsed_time(e1)
    M = torch.empty((B, H, N, dv), dtype=torch.float32, device=dev)
    y = torch.empty((B, H, T, dv), dtype=torch.float32, device=dev)
    ws = torch.empty((sdm.sdm_scan_workspace_bytes(B, H, T, W, R, dv),), dtype=torch.uint8, device=dev)
    row_bytes = B * H * T * (2 * W + R) * dv * 4
    ent = scan_entry(sdm, g, M, y, ws, out, "eq4", row_bytes, reps=5)
    ent.update({"workload": "long_context", "B": B, "H": H, "T": T, "N": N, "W": W, "R": R, "d_v": dv,
                "keys": f"{wl.n_centroids}-centroid Gaussian mixture, sigma={wl.sigma}",
                "scan_tokens_per_s": B * T / (ent["ms"]["median"] * 1e-3), "address_ms": addr_ms,
                "traffic": measured_traffic("long_context"),
                "slot_reuse": {"write": slot_reuse(out[0].cpu().numpy(), N),
                               "read": slot_reuse(out[2].cpu().numpy(), N)}})
    del g, M, y, ws, out
    torch.cuda.empty_cache()
    return ent


if __name__ == "__main__":
    main()
