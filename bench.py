#!/usr/bin/env python3
"""Benchmark of the large-head-dim attention path on one MI355X.

Metric: attention TFLOPS (forward, and forward+backward) at D=512, N=8192, bf16, as a fraction
of the dense bf16 MFMA peak. A step is one pass of the whole path over one batch of synthetic
inputs already resident in HBM: the forward kernel, then the backward launches (preprocess,
P/dS, dK, dV, dQ). Credited flops per legal (query, key) pair and query head: 4*D forward,
10*D backward (the recomputation inside the backward is not credited). By default the backward
runs with the library's P/dS workspace (one kernel forms and stores P and dS; dK = dS^T Q,
dV = P^T dO and dQ = dS K are products of them); --no-ds-workspace times the recomputing dK, dV
and dQ kernels instead (the P/dS launch is then empty).

Legs that follow the timed step, each in its own object of the JSON line (none of them changes
the step's timed region):
  configs        every other configuration of the benchmark set: the forward-only latency case
                 (B=1, H=2, N=512, D=320), the causal H=8 N=4096 D=512 step, the causal GQA
                 D=1024 fp16 step and the packed varlen causal step (forward, backward, per kernel)
  recompute_bwd  the O(N)-memory backward (no P/dS workspace) on the headline shape and on the
                 varlen set, beside the stored-P/dS path's time
  decode         the split-KV decode pass (HBM-bound)
  fp8_fwd        the FP8 forward on the step's inputs (quantizing pre-pass included)
  cpu_baseline   the float64 oracle on whole KV groups of the same inputs, on the host's cores
The side legs draw their inputs on the GPU with a seeded device generator (same distribution as
the CPU recipe, other values) so that large inputs need no host round trip.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
Prints one JSON line (rank 0).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOPS (fwd, fwd+bwd) at D=512 N=8192 bf16; % of MFMA peak"
# 256 CUs x 2.4 GHz x 4096 dense bf16/fp16 flop per clock per CU.
PEAK_TFLOPS = 2516.6
HBM_PEAK_GBS = 8000.0
# Dense fp8 (e4m3) MFMA: twice the bf16 rate.
FP8_PEAK_TFLOPS = 5033.2
# Algorithmic flops per legal pair and query head, by kernel (D multiplies these). Recomputing, dV
# does 4 D (S, P^T dO), dK and dQ 6 D (S, dP, one product); with the stored P and dS the P/dS
# kernel does 4 D (S, dP) and dK, dV, dQ are one product each, 2 D.
KERNEL_FLOPS_PER_PAIR_D = {"fwd": 4, "pds": 0, "dk": 6, "dv": 4, "dq": 6}
STORED_FLOPS_PER_PAIR_D = {"pds": 4, "dk": 2, "dv": 2, "dq": 2, "products": 6}
# (name, ffpa_bwd_stage index) of the timed launches after the forward, in ffpa_bwd's order; for
# small dense grids ffpa_bwd forms dK, dV and dQ in one launch (stage 5, "products").
BWD_STAGES = (("pre", 0), ("pds", 4), ("dk", 1), ("dv", 2), ("dq", 3))
BWD_STAGES_FUSED = (("pre", 0), ("pds", 4), ("products", 5))
COMPUTE_KERNELS = ("fwd", "pds", "dk", "dv", "dq", "products")
PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "traffic_dense_d512_n8192.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "head_dim_attention_amd", "csrc", f)
                  for f in ("ffpa_device.h", "ffpa_params.h", "ffpa_fwd.hip", "ffpa_bwd.hip", "ffpa_fp8.hip")]
# The other configurations reported beside the headline step (forward-only, causal, GQA, varlen).
CONFIG_LEGS = ("fwd_d320_n512", "causal_d512_n4096", "gqa_causal_d1024_n8192", "varlen_causal_d512")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def legal_pairs(nq: int, nkv: int, causal: bool) -> int:
    if not causal:
        return nq * nkv
    # bottom-right: query i sees keys 0..i + nkv - nq
    tot = 0
    for i in range(nq):
        tot += max(0, min(nkv, i + nkv - nq + 1))
    return tot


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dense_d512_n8192")
    ap.add_argument("--seed", type=int, default=2024)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--no-ds-workspace", action="store_true",
                    help="backward without the P/dS workspace (dV and dQ recompute)")
    ap.add_argument("--decode-workload", default="decode_gqa_d512_k65536",
                    help="workload of the split-KV decode leg ('none' skips it)")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 forward leg")
    ap.add_argument("--no-configs", action="store_true", help="skip the other configurations and the recompute leg")
    ap.add_argument("--only-legs", default="",
                    help="comma-separated config legs to run instead of the headline step (profiling)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration under rocprofv3)")
    return ap.parse_args(argv)


def load_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, if it still applies."""
    try:
        with open(PROFILE_SUMMARY) as f:
            s = json.load(f)
    except (OSError, ValueError):
        return None
    if s.get("kernel_source_hash") != kernel_source_hash():
        return None
    k = s.get("kernels", {}).get(kernel)
    if not k:
        return None
    return k.get("hbm_bytes_per_launch")


def _tf(flops: float, ms: float) -> float:
    return flops / (ms * 1e-3) / 1e12


def _check(F, st):
    if st:
        raise RuntimeError(F.ffpa_status_string(st))


class DenseStep:
    """The launches of one dense forward + backward step on resident inputs, through the C ABI:
    forward (split when the grid is small), then backward stages 0, 4, 1, 2, 3."""

    def __init__(self, F, qd, kd, vd, dod, causal: bool, store_ds: bool):
        import torch
        self.F, self.lib = F, F.load_library()
        self.qd, self.kd, self.vd, self.dod = qd, kd, vd, dod
        b, hq, nq, d = qd.shape
        hkv, nkv = kd.shape[1], kd.shape[2]
        self.dims = (b, hq, hkv, nq, nkv, d)
        self.causal, self.scale = causal, 1.0 / math.sqrt(d)
        dev = qd.device
        self.o = torch.empty_like(qd)
        self.lse = torch.empty((b, hq, nq), dtype=torch.float32, device=dev)
        self.delta = torch.empty_like(self.lse)
        self.dq, self.dk, self.dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        self.ws_bytes = F.ffpa_bwd_workspace_bytes(b, hq, nq, nkv) if store_ds else 0
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=dev) if self.ws_bytes > 0 else None
        # Grids too small to fill the GPU take the key-range split forward (workspace allocated
        # here, outside any timed region); the headline grid needs none.
        self.fws_bytes = F.ffpa_fwd_split_workspace_bytes(b, hq, hkv, nq, nkv, d)
        self.fws = torch.empty(self.fws_bytes, dtype=torch.uint8, device=dev) if self.fws_bytes > 0 else None
        self.dt = 0 if qd.dtype == torch.bfloat16 else 1
        self.stream = torch.cuda.current_stream(dev)
        self.pairs = legal_pairs(nq, nkv, causal) * b * hq
        self.configure()

    def configure(self):
        """Launch list and per-kernel flops for the current workspace (as ffpa_bwd runs them)."""
        b, hq, hkv, nq, nkv, d = self.dims
        self.fused = self.ws is not None and self.F.ffpa_bwd_fused_products(b, hq, hkv, nq, nkv, d)
        self.bwd_stages = BWD_STAGES_FUSED if self.fused else BWD_STAGES
        self.stages = ("fwd",) + tuple(n for n, _ in self.bwd_stages)
        self.flops_d = dict(KERNEL_FLOPS_PER_PAIR_D, products=0)
        if self.ws is not None:
            self.flops_d.update(STORED_FLOPS_PER_PAIR_D)
        self.launches = [self.fwd] + [(lambda i=i: self.bwd_stage(i)) for _, i in self.bwd_stages]

    def fwd(self):
        P, (b, hq, hkv, nq, nkv, d) = self.F._binding._ptr, self.dims
        sp = self.stream.cuda_stream
        if self.fws is None:
            st = self.lib.ffpa_fwd(P(self.qd), P(self.kd), P(self.vd), P(self.o), P(self.lse), b, hq, hkv, nq, nkv, d,
                                   self.dt, self.scale, int(self.causal), sp)
        else:
            st = self.lib.ffpa_fwd_split(P(self.qd), P(self.kd), P(self.vd), P(self.o), P(self.lse), b, hq, hkv, nq,
                                         nkv, d, self.dt, self.scale, int(self.causal), P(self.fws), self.fws_bytes, sp)
        _check(self.F, st)

    def bwd_stage(self, i):
        P, (b, hq, hkv, nq, nkv, d) = self.F._binding._ptr, self.dims
        st = self.lib.ffpa_bwd_stage(i, P(self.qd), P(self.kd), P(self.vd), P(self.o), P(self.dod), P(self.lse), None,
                                     P(self.delta), P(self.dq), P(self.dk), P(self.dv), b, hq, hkv, nq, nkv, d,
                                     self.dt, self.scale, int(self.causal), P(self.ws), self.ws_bytes,
                                     self.stream.cuda_stream)
        _check(self.F, st)

    def time(self, steps: int, warmup: int):
        """HIP events on the launch stream around every launch of every step; returns (mean ms per
        stage, host wall ms per step)."""
        import torch
        for _ in range(warmup):
            for fn in self.launches:
                fn()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(self.launches) + 1)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(steps):
            ev[s][0].record(self.stream)
            for i, fn in enumerate(self.launches):
                fn()
                ev[s][i + 1].record(self.stream)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / steps
        stage_ms = {name: sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)) / steps
                    for i, name in enumerate(self.stages)}
        return stage_ms, wall_ms

    def time_steps(self, steps: int, warmup: int):
        """Whole steps with HIP events on the launch stream only between steps (the launches of a
        step follow each other as ffpa_bwd issues them); returns (mean event ms per step, host
        wall ms per step)."""
        import torch
        for _ in range(warmup):
            for fn in self.launches:
                fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record(self.stream)
        for s in range(steps):
            for fn in self.launches:
                fn()
            ev[s + 1].record(self.stream)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / steps
        return sum(ev[s].elapsed_time(ev[s + 1]) for s in range(steps)) / steps, wall_ms

    def kernel_table(self, stage_ms):
        d = self.dims[5]
        kernels = {}
        for n in COMPUTE_KERNELS:
            if self.flops_d[n] == 0 or n not in stage_ms:
                continue
            fl = self.flops_d[n] * d * self.pairs
            kernels[n] = {"ms": round(stage_ms[n], 4), "algorithmic_tflops": round(_tf(fl, stage_ms[n]), 2),
                          "frac": round(_tf(fl, stage_ms[n]) / PEAK_TFLOPS, 4)}
        b, hq, _, nq, _, _ = self.dims
        pre_bytes = 2.0 * b * hq * nq * d * self.qd.element_size() + 4.0 * b * hq * nq
        gbs = pre_bytes / (stage_ms["pre"] * 1e-3) / 1e9
        kernels["pre"] = {"ms": round(stage_ms["pre"], 4), "algorithmic_gbs": round(gbs, 1),
                          "frac": round(gbs / HBM_PEAK_GBS, 4)}
        return kernels


def _timed(fn, steps: int, warmup: int, stream) -> float:
    """Mean HIP-event ms of fn() over `steps` calls on `stream` after `warmup` calls."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return sum(ev[i].elapsed_time(ev[i + 1]) for i in range(steps)) / steps


def dense_config_leg(F, W, w, seed: int, steps: int, warmup: int, store_ds: bool = True) -> dict:
    """Forward (+ backward) of a dense workload: times, credited TFLOPS and fractions of peak."""
    import torch
    dev = torch.device("cuda:0")
    q, k, v, do = W.workload_inputs(w, seed, device="cuda")
    if do is None:
        do = torch.zeros_like(q)
    step = DenseStep(F, q, k, v, do, w.causal, store_ds)
    b, hq, hkv, nq, nkv, d = step.dims
    fwd_flops = 4.0 * d * step.pairs
    out = {"workload": w.name, "batch": b, "heads": hq, "kv_heads": hkv, "seq_len_q": nq, "seq_len_kv": nkv,
           "head_dim": d, "causal": w.causal, "dtype": w.dtype, "credited_fwd_flops": fwd_flops}
    if not w.backward:
        n = max(steps, 200)
        ms = _timed(step.fwd, n, max(warmup, 10), step.stream)
        out.update({"fwd_ms": round(ms, 5), "fwd_tflops": round(_tf(fwd_flops, ms), 2),
                    "fwd_frac": round(_tf(fwd_flops, ms) / PEAK_TFLOPS, 4), "timed_calls": n,
                    "note": "latency-bound (grid of a few workgroups); warm caches"})
        del step
        torch.cuda.empty_cache()
        return out
    # The step as ffpa_bwd runs it (events only between steps), then once more with an event
    # around every launch for the per-kernel times (each record between launches adds a few
    # microseconds to the sum of the stage times).
    ms_step, _ = step.time_steps(steps, warmup)
    stage_ms, _ = step.time(steps, 0)
    ms_fwd = stage_ms["fwd"]
    out.update({"fwd_ms": round(ms_fwd, 4), "fwd_tflops": round(_tf(fwd_flops, ms_fwd), 2),
                "fwd_frac": round(_tf(fwd_flops, ms_fwd) / PEAK_TFLOPS, 4),
                "bwd_ms": round(sum(stage_ms.values()) - ms_fwd, 4), "fwdbwd_ms": round(ms_step, 4),
                "stage_event_sum_ms": round(sum(stage_ms.values()), 4),
                "fwdbwd_tflops": round(_tf(3.5 * fwd_flops, ms_step), 2),
                "fwdbwd_frac": round(_tf(3.5 * fwd_flops, ms_step) / PEAK_TFLOPS, 4),
                "bwd_path": ("stored P and dS" + (", dK + dV + dQ in one launch" if step.fused else "")
                             if step.ws is not None else "recompute (O(N) memory)"),
                "workspace_gib": round(step.ws_bytes / 2**30, 3),
                "forward_kernel": "key-range split + merge" if step.fws is not None else "one launch",
                "kernels": step.kernel_table(stage_ms)})
    if d > 512:
        # the FP8 forward above D = 512 (at D <= 512 the main step times it)
        f8 = fp8_leg(F, q, k, v, w.causal, step.pairs, max(steps, 10), warmup)
        if "ms" in f8:
            f8["vs_bf16_fwd"] = round(ms_fwd / f8["ms"], 3)
        out["fp8_fwd"] = f8
    del step
    torch.cuda.empty_cache()
    return out


def varlen_config_leg(F, W, w, seed: int, steps: int, warmup: int, store_ds_modes=(True, False)) -> dict:
    """Packed varlen forward and backward through ffpa_varlen_fwd / ffpa_varlen_bwd (workspaces
    allocated outside the timed region), for each backward path in store_ds_modes."""
    import torch
    dev = torch.device("cuda:0")
    lens = W.varlen_lengths(w.batch, seed)
    q, k, v, do, cu_q, cu_k = W.workload_inputs(w, seed, device="cuda")
    cq, ck = cu_q.to(dev), cu_k.to(dev)
    cu_host = cu_q.tolist()
    tq, hq, d = q.shape
    hkv = k.shape[1]
    mx = max(lens)
    lib = F.load_library()
    P = F._binding._ptr
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    dt = 0 if q.dtype == torch.bfloat16 else 1
    scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.empty((hq, tq), dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    pairs = hq * sum(n * (n + 1) // 2 for n in lens)
    fwd_flops = 4.0 * d * pairs

    def fwd():
        _check(F, lib.ffpa_varlen_fwd(P(q), P(k), P(v), P(o), P(lse), P(cq), P(ck), w.batch, mx, mx, tq, tq, hq, hkv,
                                      d, dt, scale, 1, sp))

    ms_fwd = _timed(fwd, steps, warmup, stream)
    out = {"workload": w.name, "sequences": w.batch, "lengths": lens, "total_tokens": tq, "heads": hq,
           "head_dim": d, "causal": True, "dtype": w.dtype, "credited_fwd_flops": fwd_flops,
           "fwd_ms": round(ms_fwd, 4), "fwd_tflops": round(_tf(fwd_flops, ms_fwd), 2),
           "fwd_frac": round(_tf(fwd_flops, ms_fwd) / PEAK_TFLOPS, 4)}
    import ctypes
    host = (ctypes.c_int32 * len(cu_host))(*cu_host)
    hp = ctypes.cast(host, ctypes.c_void_p)
    for store_ds in store_ds_modes:
        nws = F.ffpa_varlen_bwd_workspace_bytes_exact(hq, cu_host, cu_host, tq, tq, mx, mx) if store_ds else 0
        ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws > 0 else None

        def bwd():
            _check(F, lib.ffpa_varlen_bwd(P(q), P(k), P(v), P(o), P(do), P(lse), None, P(delta), P(dq), P(dk), P(dv),
                                          P(cq), P(ck), hp, hp, w.batch, mx, mx, tq, tq, hq, hkv, d, dt, scale, 1,
                                          P(ws), nws, sp))

        ms_bwd = _timed(bwd, steps, warmup, stream)
        key = "" if store_ds else "recompute_"
        tot = ms_fwd + ms_bwd
        out.update({f"{key}bwd_ms": round(ms_bwd, 4), f"{key}fwdbwd_ms": round(tot, 4),
                    f"{key}fwdbwd_tflops": round(_tf(3.5 * fwd_flops, tot), 2),
                    f"{key}fwdbwd_frac": round(_tf(3.5 * fwd_flops, tot) / PEAK_TFLOPS, 4),
                    f"{key}workspace_gib": round(nws / 2**30, 3)})
        del ws
        torch.cuda.empty_cache()
    out["workspace_bound_gib"] = round(F.ffpa_varlen_bwd_workspace_bytes(hq, tq, tq, mx, mx) / 2**30, 3)
    return out


def decode_leg(F, W, w, seed: int, steps: int, warmup: int) -> dict:
    """Time ffpa_decode_fwd (split-KV pass + combine pass) on a decode workload, inputs resident in
    HBM. The pass is HBM-bound: algorithmic bytes are K and V read once plus Q and O, LSE, and the
    partial results written and read back once by the combine."""
    import torch
    q, k, v, _ = W.workload_inputs(w, seed)
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    b, hq, nq, d = qd.shape
    hkv, nkv = kd.shape[1], kd.shape[2]
    o = torch.empty_like(qd)
    lse = torch.empty((b, hq, nq), dtype=torch.float32, device=dev)
    nws = F.ffpa_decode_workspace_bytes(b, hq, hkv, nq, nkv, d)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)
    lib = F.load_library()
    stream = torch.cuda.current_stream(dev)
    P = F._binding._ptr
    dt = 0 if w.dtype == "bf16" else 1

    def run():
        _check(F, lib.ffpa_decode_fwd(P(qd), P(kd), P(vd), P(o), P(lse), b, hq, hkv, nq, nkv, d, dt,
                                      1.0 / math.sqrt(d), int(w.causal), P(ws), nws, stream.cuda_stream))

    ms = _timed(run, steps, warmup, stream)
    el = qd.element_size()
    kv_bytes = 2.0 * b * hkv * nkv * d * el
    part_bytes = 2.0 * nws  # partial O and LSE written once, read once
    alg_bytes = kv_bytes + 2.0 * b * hq * nq * d * el + 4.0 * b * hq * nq + part_bytes
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    return {"workload": w.name, "batch": b, "heads": hq, "kv_heads": hkv, "seq_len_q": nq, "seq_len_kv": nkv,
            "head_dim": d, "causal": w.causal, "dtype": w.dtype, "ms": round(ms, 4),
            "nsplit": nws // (b * hq * nq * (d + 1) * 4),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": load_traffic("decode"),
                         "algorithmic_bytes": alg_bytes, "kv_bytes": kv_bytes}}


def fp8_leg(F, qd, kd, vd, causal: bool, pairs: int, steps: int, warmup: int) -> dict:
    """Time ffpa_fwd_fp8 (the quantizing pre-pass and the FP8 MFMA forward, one call) on the
    measured workload's Q, K, V, inputs resident in HBM; flops as the forward's, against the dense
    fp8 MFMA peak."""
    import torch
    b, hq, nq, d = qd.shape
    hkv, nkv = kd.shape[1], kd.shape[2]
    o = torch.empty_like(qd)
    lse = torch.empty((b, hq, nq), dtype=torch.float32, device=qd.device)
    nws = F.ffpa_fwd_fp8_workspace_bytes(b, hq, hkv, nq, nkv, d)
    if nws == 0:
        return {"skipped": f"no FP8 forward at D={d}"}
    ws = torch.empty(nws, dtype=torch.uint8, device=qd.device)
    lib = F.load_library()
    stream = torch.cuda.current_stream(qd.device)
    P = F._binding._ptr
    dt = 0 if qd.dtype == torch.bfloat16 else 1

    def run():
        _check(F, lib.ffpa_fwd_fp8(P(qd), P(kd), P(vd), P(o), P(lse), b, hq, hkv, nq, nkv, d, dt, 1.0 / math.sqrt(d),
                                   int(causal), P(ws), nws, stream.cuda_stream))

    ms = _timed(run, steps, warmup, stream)
    tf = _tf(4.0 * d * pairs, ms)
    return {"ms": round(ms, 4), "includes": "amax and quantization pre-pass + FP8 forward kernel",
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / FP8_PEAK_TFLOPS, 4), "traffic": load_traffic("fp8_fwd")},
            "vs_bf16_fwd": None}


def host_description() -> dict:
    """CPU model (/proc/cpuinfo), the CPUs this process may run on, and NumPy's BLAS build."""
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        import threadpoolctl
        infos = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        if infos:
            i = infos[0]
            blas = f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer', 'n/a')} threads, " \
                   f"{i.get('architecture', 'n/a')})"
    except Exception:  # noqa: BLE001 - description only
        pass
    return {"cpu_model": model, "affinity_cpus": len(os.sched_getaffinity(0)), "blas": blas}


def cpu_baseline(q, k, v, do, scale, causal, dq, dk, dv, o, lse, tol_o, budget_s=10.0):
    """Time the float64 oracle on whole KV groups of the same inputs (batch 0, KV heads 0, 1, ...)
    until about `budget_s` seconds of CPU work have run, with BLAS limited to the CPUs this
    process may use (len(os.sched_getaffinity(0)) threads).

    Returns (baseline dict, parity dict): the same runs check the GPU's O, LSE, dQ, dK, dV for those
    groups in full.
    """
    import numpy as np
    import threadpoolctl

    from oracle import ref

    hkv = k.shape[1]
    g = q.shape[1] // hkv
    nq, nkv, d = q.shape[2], k.shape[2], q.shape[3]
    cores = len(os.sched_getaffinity(0))
    s64 = float(np.float32(scale))

    def relerr(x, y):
        return float(np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-30))

    par = {"o_max_abs": 0.0, "lse_max_abs": 0.0, "dq_rel_l2": 0.0, "dk_rel_l2": 0.0, "dv_rel_l2": 0.0}
    elapsed, groups = 0.0, 0
    with threadpoolctl.threadpool_limits(limits=cores, user_api="blas"):
        used = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
                   or [1])
        while groups < hkv and (groups == 0 or elapsed < budget_s):
            kv = groups
            hs = slice(kv * g, (kv + 1) * g)
            qg, dog = q[0, hs].double().numpy(), do[0, hs].double().numpy()
            kg, vg = k[0, kv].double().numpy(), v[0, kv].double().numpy()
            t0 = time.perf_counter()
            dq_r, dk_r, dv_r, o_r, lse_r = ref.group_backward(qg, kg, vg, dog, s64, causal)[:5]
            elapsed += time.perf_counter() - t0
            groups += 1
            fin = np.isfinite(lse_r)
            lg = lse[0, hs].double().cpu().numpy()
            par["o_max_abs"] = max(par["o_max_abs"], float(np.max(np.abs(o[0, hs].double().cpu().numpy() - o_r))))
            if fin.any():
                par["lse_max_abs"] = max(par["lse_max_abs"], float(np.max(np.abs(lg[fin] - lse_r[fin]))))
            par["dq_rel_l2"] = max(par["dq_rel_l2"], relerr(dq[0, hs].double().cpu().numpy(), dq_r))
            par["dk_rel_l2"] = max(par["dk_rel_l2"], relerr(dk[0, kv].double().cpu().numpy(), dk_r))
            par["dv_rel_l2"] = max(par["dv_rel_l2"], relerr(dv[0, kv].double().cpu().numpy(), dv_r))
    flops = 14.0 * d * legal_pairs(nq, nkv, causal) * g * groups
    host = host_description()
    base = {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOPS", "cores": int(min(used, cores)),
            "kind": "oracle",
            "sample": f"float64 NumPy oracle forward+backward of {groups} of {hkv} KV groups "
                      f"({groups * g} of {q.shape[1]} query heads, batch 0) of the same inputs: "
                      f"{elapsed:.2f} s, credited {flops:.3e} flops",
            "seconds": round(elapsed, 3), "cpu": host["cpu_model"], "affinity_cpus": host["affinity_cpus"],
            "blas_threads": int(used), "blas": host["blas"]}
    par["sample"] = f"KV groups 0..{groups - 1} of batch 0, all rows"
    par["pass"] = bool(par["o_max_abs"] <= tol_o and par["lse_max_abs"] <= 1e-3 and
                       max(par["dq_rel_l2"], par["dk_rel_l2"], par["dv_rel_l2"]) <= 2e-2)
    return base, par


def calibration_copy(mib: int, dev) -> None:
    """One device-to-device copy of `mib` MiB: its FETCH_SIZE / WRITE_SIZE readings under a
    counter run give the scale from those counters to bytes."""
    if mib <= 0:
        return
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def run_legs(F, W, names, seed: int, steps: int, warmup: int) -> dict:
    legs = {}
    for name in names:
        w = W.get(name)
        print(f"bench: timing configuration {name}", file=sys.stderr, flush=True)
        if w.varlen:
            legs[name] = varlen_config_leg(F, W, w, seed, steps, warmup)
        else:
            legs[name] = dense_config_leg(F, W, w, seed, steps, warmup)
    return legs


def main(argv=None) -> int:
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: times a single GPU only; --gpus {args.gpus} is not supported "
              "(heads are independent, so more GPUs would each run a share of the heads)", file=sys.stderr)
        return 2

    import head_dim_attention_amd as F
    import workloads as W

    if args.only_legs:
        names = [n for n in args.only_legs.split(",") if n]
        for n in names:
            if n not in W.WORKLOADS:
                print(f"bench.py: unknown workload {n}", file=sys.stderr)
                return 2
    else:
        w = W.get(args.workload)
        if w.varlen or not w.backward:
            print(f"bench.py: the step needs a dense forward+backward workload; {w.name} is timed as a "
                  "configuration leg (--only-legs)", file=sys.stderr)
            return 2

    import torch

    F.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.only_legs:
        legs = run_legs(F, W, names, args.seed, max(args.steps, 5), args.warmup)
        calibration_copy(args.calib_copy_mib, dev)
        print(json.dumps({"configs": legs}), flush=True)
        return 0

    q, k, v, do = W.workload_inputs(w, args.seed)
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    step = DenseStep(F, qd, kd, vd, dod, w.causal, not args.no_ds_workspace)
    b, hq, hkv, nq, nkv, d = step.dims
    causal = w.causal

    for fn in step.launches:  # one untimed pass before the warmup message
        fn()
    print(f"bench: warmup ({args.warmup} steps), timing {args.steps} steps of {w.name}", file=sys.stderr, flush=True)
    # The timed region: W warmup steps, then K whole steps between device syncs, with HIP events
    # only between steps. Then K more steps with an event around every launch, for the per-kernel
    # times and the roofline kernel.
    step_ms, wall_ms = step.time_steps(args.steps, args.warmup)
    stage_ms, _ = step.time(args.steps, 0)

    pairs = step.pairs
    fwd_flops = 4.0 * d * pairs
    fb_flops = 14.0 * d * pairs
    value = _tf(fb_flops, wall_ms)
    fwd_tflops = _tf(fwd_flops, stage_ms["fwd"])

    # Dominant kernel: the longest of the compute kernels.
    dom = max((n for n in COMPUTE_KERNELS if step.flops_d[n] > 0 and n in stage_ms), key=lambda n: stage_ms[n])
    achieved = _tf(step.flops_d[dom] * d * pairs, stage_ms[dom])

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": f"synthetic: iid N(0,1) x{w.input_scale} from torch seed {args.seed}, resident in HBM",
        "config": {"workload": w.name, "batch": b, "heads": hq, "kv_heads": hkv, "seq_len_q": nq, "seq_len_kv": nkv,
                   "head_dim": d, "causal": causal, "parallelism": "none (1 GPU)"},
        "fwd_tflops": round(fwd_tflops, 2),
        "fwd_frac_of_peak": round(fwd_tflops / PEAK_TFLOPS, 4),
        "fwdbwd_frac_of_peak": round(value / PEAK_TFLOPS, 4),
        "peak_tflops": PEAK_TFLOPS,
        "event_ms_per_step": round(step_ms, 4),
        "stage_event_sum_ms": round(sum(stage_ms.values()), 4),
        "bwd_path": (f"stored P and dS ({step.ws_bytes / 2**30:.2f} GiB workspace): dK = dS^T Q, dV = P^T dO, "
                     "dQ = dS K" if step.ws is not None else "dK, dV and dQ recompute S, P (dP, dS)"),
        "kernels": step.kernel_table(stage_ms),
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4), "traffic": load_traffic(dom)},
    }

    if not args.no_fp8:
        print("bench: timing the FP8 forward on the same inputs", file=sys.stderr, flush=True)
        f8 = fp8_leg(F, qd, kd, vd, causal, pairs, max(args.steps, 10), args.warmup)
        if "ms" in f8:
            f8["vs_bf16_fwd"] = round(stage_ms["fwd"] / f8["ms"], 3)
        out["fp8_fwd"] = f8

    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on whole KV groups", file=sys.stderr, flush=True)
        base, par = cpu_baseline(q, k, v, do, 1.0 / math.sqrt(d), causal, step.dq, step.dk, step.dv, step.o,
                                 step.lse, 2e-2 if w.dtype == "bf16" else 4e-3)
        out["cpu_baseline"] = base
        out["parity"] = par
    else:
        out["cpu_baseline"] = None

    if not args.no_configs:
        # The O(N)-memory backward of the same shape, beside the stored-P/dS one.
        ws_keep = step.ws
        step.ws, step.ws_bytes = None, 0
        step.configure()
        print("bench: timing the recomputing backward on the same inputs", file=sys.stderr, flush=True)
        rec_step, _ = step.time_steps(max(args.steps // 2, 5), 1)
        rs_ms, _ = step.time(max(args.steps // 2, 5), 0)
        # backward times: sums of the per-launch pass; forward+backward: the whole-step pass
        bwd_rec = sum(rs_ms.values()) - rs_ms["fwd"]
        rec = {"workload": w.name, "bwd_ms": round(bwd_rec, 4), "fwdbwd_ms": round(rec_step, 4),
               "fwdbwd_tflops": round(_tf(fb_flops, rec_step), 2),
               "fwdbwd_frac": round(_tf(fb_flops, rec_step) / PEAK_TFLOPS, 4),
               "stored_ds_bwd_ms": round(sum(stage_ms.values()) - stage_ms["fwd"], 4),
               "stored_ds_workspace_gib": round((ws_keep.numel() if ws_keep is not None else 0) / 2**30, 3),
               "kernels": step.kernel_table(rs_ms)}
        del ws_keep, step
        del qd, kd, vd, dod
        torch.cuda.empty_cache()
        out["configs"] = run_legs(F, W, CONFIG_LEGS, args.seed, max(args.steps // 2, 5), args.warmup)
        vl = out["configs"].get("varlen_causal_d512", {})
        out["recompute_bwd"] = {w.name: rec}
        if "recompute_bwd_ms" in vl:
            out["recompute_bwd"]["varlen_causal_d512"] = {
                "bwd_ms": vl["recompute_bwd_ms"], "fwdbwd_tflops": vl["recompute_fwdbwd_tflops"],
                "fwdbwd_frac": vl["recompute_fwdbwd_frac"], "stored_ds_bwd_ms": vl["bwd_ms"],
                "stored_ds_workspace_gib": vl["workspace_gib"]}

    if args.decode_workload != "none":
        print(f"bench: timing the split-KV decode pass on {args.decode_workload}", file=sys.stderr, flush=True)
        out["decode"] = decode_leg(F, W, W.get(args.decode_workload), args.seed, max(args.steps, 10), args.warmup)

    calibration_copy(args.calib_copy_mib, dev)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
