"""bench.py's output contract on the GPU: one JSON line with the metric, the whole-step value, the
dominant kernel's roofline object, the decode and FP8 legs with their own rooflines, the other
configurations and the recomputing backward (a short
run: two timed steps, no CPU baseline)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line():
    print("bench.py --steps 2 --warmup 1 --no-cpu-baseline", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1",
                        "--no-cpu-baseline"], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1 and d["value"] > 0 and d["dtype"] == "bf16"
    assert d["config"]["workload"] == "dense_d512_n8192"
    # the step is timed with events only between steps; the per-launch pass is reported beside it,
    # and both lie within a few percent of the host wall time of a step
    assert d["event_ms_per_step"] > 0 and d["stage_event_sum_ms"] > 0
    assert abs(d["event_ms_per_step"] - d["ms_per_step"]) < 0.05 * d["ms_per_step"]
    assert set(d["kernels"]) >= {"fwd", "pds", "dk", "dv", "dq"}
    roof = d["roofline"]
    assert set(roof) >= {"bound", "achieved", "peak", "unit", "frac", "traffic"}
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and 0 < roof["frac"] < 1
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    dec = d["decode"]["roofline"]
    assert dec["bound"] == "hbm" and dec["unit"] == "GB/s" and 0 < dec["frac"] < 1
    f8 = d["fp8_fwd"]["roofline"]
    assert f8["bound"] == "mfma" and 0 < f8["frac"] < 1 and f8["peak"] > roof["peak"]
    # every other configuration of the benchmark set, and the recomputing backward beside the stored one
    cfg = d["configs"]
    assert set(cfg) == {"fwd_d320_n512", "causal_d512_n4096", "gqa_causal_d1024_n8192", "varlen_causal_d512"}
    assert cfg["fwd_d320_n512"]["fwd_ms"] > 0 and "bwd_ms" not in cfg["fwd_d320_n512"]
    for name in ("causal_d512_n4096", "gqa_causal_d1024_n8192", "varlen_causal_d512"):
        c = cfg[name]
        assert 0 < c["fwd_frac"] < 1 and 0 < c["fwdbwd_frac"] < 1, name
        assert c["fwdbwd_ms"] > c["fwd_ms"] > 0, name
        if name != "varlen_causal_d512":
            assert c["stage_event_sum_ms"] > c["fwd_ms"] and c["bwd_ms"] > 0, name
    assert cfg["gqa_causal_d1024_n8192"]["kernels"]["dk"]["ms"] > 0
    assert cfg["varlen_causal_d512"]["workspace_gib"] <= cfg["varlen_causal_d512"]["workspace_bound_gib"]
    rec = d["recompute_bwd"]
    assert rec["dense_d512_n8192"]["bwd_ms"] > 0 and rec["varlen_causal_d512"]["bwd_ms"] > 0
