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

Two side legs follow the step, each reported in its own object of the JSON line: the split-KV
decode pass on a decode workload ("decode", HBM-bound) and the FP8 forward on the step's inputs
("fp8_fwd", quantizing pre-pass included, against the fp8 MFMA peak).

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
STORED_FLOPS_PER_PAIR_D = {"pds": 4, "dk": 2, "dv": 2, "dq": 2}
# (name, ffpa_bwd_stage index) of the timed launches after the forward, in ffpa_bwd's order.
BWD_STAGES = (("pre", 0), ("pds", 4), ("dk", 1), ("dv", 2), ("dq", 3))
STAGES = ("fwd",) + tuple(n for n, _ in BWD_STAGES)
COMPUTE_KERNELS = ("fwd", "pds", "dk", "dv", "dq")
PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "traffic_dense_d512_n8192.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "head_dim_attention_amd", "csrc", f)
                  for f in ("ffpa_device.h", "ffpa_params.h", "ffpa_fwd.hip", "ffpa_bwd.hip", "ffpa_fp8.hip")]


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
        st = lib.ffpa_decode_fwd(P(qd), P(kd), P(vd), P(o), P(lse), b, hq, hkv, nq, nkv, d, dt,
                                 1.0 / math.sqrt(d), int(w.causal), P(ws), nws, stream.cuda_stream)
        if st:
            raise RuntimeError(F.ffpa_status_string(st))

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        run()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = sum(ev[i].elapsed_time(ev[i + 1]) for i in range(steps)) / steps
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
        st = lib.ffpa_fwd_fp8(P(qd), P(kd), P(vd), P(o), P(lse), b, hq, hkv, nq, nkv, d, dt, 1.0 / math.sqrt(d),
                              int(causal), P(ws), nws, stream.cuda_stream)
        if st:
            raise RuntimeError(F.ffpa_status_string(st))

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        run()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = sum(ev[i].elapsed_time(ev[i + 1]) for i in range(steps)) / steps
    tf = 4.0 * d * pairs / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 4), "includes": "amax and quantization pre-pass + FP8 forward kernel",
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / FP8_PEAK_TFLOPS, 4), "traffic": load_traffic("fp8_fwd")},
            "vs_bf16_fwd": None}


def cpu_baseline(q, k, v, do, scale, causal, dq, dk, dv, o, lse, tol_o, budget_s=10.0):
    """Time the float64 oracle on whole KV groups of the same inputs (batch 0, KV heads 0, 1, ...)
    until about `budget_s` seconds of CPU work have run.

    Returns (baseline dict, parity dict): the same runs check the GPU's O, LSE, dQ, dK, dV for those
    groups in full.
    """
    import numpy as np
    import threadpoolctl

    from oracle import ref

    hkv = k.shape[1]
    g = q.shape[1] // hkv
    nq, nkv, d = q.shape[2], k.shape[2], q.shape[3]
    threads = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    s64 = float(np.float32(scale))

    def relerr(x, y):
        return float(np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-30))

    par = {"o_max_abs": 0.0, "lse_max_abs": 0.0, "dq_rel_l2": 0.0, "dk_rel_l2": 0.0, "dv_rel_l2": 0.0}
    elapsed, groups = 0.0, 0
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
    base = {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOPS", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 NumPy oracle forward+backward of {groups} of {hkv} KV groups "
                      f"({groups * g} of {q.shape[1]} query heads, batch 0) of the same inputs: "
                      f"{elapsed:.2f} s, credited {flops:.3e} flops",
            "seconds": round(elapsed, 3), "cpu": platform.processor() or platform.machine()}
    par["sample"] = f"KV groups 0..{groups - 1} of batch 0, all rows"
    par["pass"] = bool(par["o_max_abs"] <= tol_o and par["lse_max_abs"] <= 1e-3 and
                       max(par["dq_rel_l2"], par["dk_rel_l2"], par["dv_rel_l2"]) <= 2e-2)
    return base, par


def main(argv=None) -> int:
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: times a single GPU only; --gpus {args.gpus} is not supported "
              "(heads are independent, so more GPUs would each run a share of the heads)", file=sys.stderr)
        return 2

    import torch

    import head_dim_attention_amd as F
    import workloads as W

    F.load_library()
    w = W.get(args.workload)
    if w.varlen or not w.backward:
        print(f"bench.py: {w.name} is not a dense forward+backward workload; choose one that is", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v, do = W.workload_inputs(w, args.seed)
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    b, hq, nq, d = qd.shape
    hkv, nkv = kd.shape[1], kd.shape[2]
    scale = 1.0 / math.sqrt(d)
    causal = w.causal

    o = torch.empty_like(qd)
    lse = torch.empty((b, hq, nq), dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    lib = F.load_library()
    ws_bytes = 0 if args.no_ds_workspace else F.ffpa_bwd_workspace_bytes(b, hq, nq, nkv)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes > 0 else None
    flops_d = dict(KERNEL_FLOPS_PER_PAIR_D)
    if ws is not None:
        flops_d.update(STORED_FLOPS_PER_PAIR_D)
        if d > 512:  # the dK kernel recomputes and stores P and dS itself; the P/dS launch is empty
            flops_d.update({"pds": 0, "dk": 6})
    dt = 0 if w.dtype == "bf16" else 1
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    P = F._binding._ptr

    # Grids too small to fill the GPU take the key-range split forward (its workspace allocated
    # here, outside the timed region); the headline grid needs none.
    fws_bytes = F.ffpa_fwd_split_workspace_bytes(b, hq, hkv, nq, nkv, d)
    fws = torch.empty(fws_bytes, dtype=torch.uint8, device=dev) if fws_bytes > 0 else None

    def fwd():
        if fws is None:
            st = lib.ffpa_fwd(P(qd), P(kd), P(vd), P(o), P(lse), b, hq, hkv, nq, nkv, d, dt, scale, int(causal), sp)
        else:
            st = lib.ffpa_fwd_split(P(qd), P(kd), P(vd), P(o), P(lse), b, hq, hkv, nq, nkv, d, dt, scale, int(causal),
                                    P(fws), fws_bytes, sp)
        if st:
            raise RuntimeError(F.ffpa_status_string(st))

    def bwd_stage(i):
        st = lib.ffpa_bwd_stage(i, P(qd), P(kd), P(vd), P(o), P(dod), P(lse), P(delta), P(dq), P(dk), P(dv),
                                b, hq, hkv, nq, nkv, d, dt, scale, int(causal), P(ws), ws_bytes, sp)
        if st:
            raise RuntimeError(F.ffpa_status_string(st))

    launches = [fwd] + [(lambda i=i: bwd_stage(i)) for _, i in BWD_STAGES]

    for _ in range(args.warmup):
        for fn in launches:
            fn()
    torch.cuda.synchronize()
    print(f"bench: warmup done ({args.warmup} steps), timing {args.steps} steps of {w.name}", file=sys.stderr,
          flush=True)

    # Events on the stream the kernels are launched on, between every launch of every step.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(launches) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record(stream)
        for i, fn in enumerate(launches):
            fn()
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    stage_ms = {name: sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)) / args.steps
                for i, name in enumerate(STAGES)}
    step_ms = sum(stage_ms.values())

    pairs = legal_pairs(nq, nkv, causal) * b * hq
    fwd_flops = 4.0 * d * pairs
    fb_flops = 14.0 * d * pairs
    value = fb_flops / (wall_ms * 1e-3) / 1e12
    fwd_tflops = fwd_flops / (stage_ms["fwd"] * 1e-3) / 1e12

    # Dominant kernel: the longest of the compute kernels.
    dom = max((n for n in COMPUTE_KERNELS if flops_d[n] > 0), key=lambda n: stage_ms[n])
    dom_flops = flops_d[dom] * d * pairs
    achieved = dom_flops / (stage_ms[dom] * 1e-3) / 1e12
    traffic = load_traffic(dom)
    kernels = {}
    for n in COMPUTE_KERNELS:
        if flops_d[n] == 0:
            continue
        fl = flops_d[n] * d * pairs
        kernels[n] = {"ms": round(stage_ms[n], 4), "algorithmic_tflops": round(fl / (stage_ms[n] * 1e-3) / 1e12, 2),
                      "frac": round(fl / (stage_ms[n] * 1e-3) / 1e12 / PEAK_TFLOPS, 4)}
    pre_bytes = 2.0 * b * hq * nq * d * qd.element_size() + 4.0 * b * hq * nq
    kernels["pre"] = {"ms": round(stage_ms["pre"], 4), "algorithmic_gbs": round(pre_bytes / (stage_ms["pre"] * 1e-3) / 1e9, 1),
                      "frac": round(pre_bytes / (stage_ms["pre"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

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
        "bwd_path": (f"stored P and dS ({ws_bytes / 2**30:.2f} GiB workspace): dK = dS^T Q, dV = P^T dO, dQ = dS K"
                     if ws is not None else "dK, dV and dQ recompute S, P (dP, dS)"),
        "kernels": kernels,
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4), "traffic": traffic},
    }

    if args.decode_workload != "none":
        print(f"bench: timing the split-KV decode pass on {args.decode_workload}", file=sys.stderr, flush=True)
        out["decode"] = decode_leg(F, W, W.get(args.decode_workload), args.seed, max(args.steps, 10), args.warmup)

    if not args.no_fp8:
        print("bench: timing the FP8 forward on the same inputs", file=sys.stderr, flush=True)
        f8 = fp8_leg(F, qd, kd, vd, causal, pairs, max(args.steps, 10), args.warmup)
        if "ms" in f8:
            f8["vs_bf16_fwd"] = round(stage_ms["fwd"] / f8["ms"], 3)
        out["fp8_fwd"] = f8

    if args.calib_copy_mib > 0:
        nbytes = args.calib_copy_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on one KV group", file=sys.stderr, flush=True)
        base, par = cpu_baseline(q, k, v, do, scale, causal, dq, dk, dv, o, lse, 2e-2 if w.dtype == "bf16" else 4e-3)
        out["cpu_baseline"] = base
        out["parity"] = par
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
