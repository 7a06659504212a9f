"""Build libffpa.so (the gfx950 HIP kernels plus the C ABI) in-tree with hipcc.

Usage: python -m head_dim_attention_amd.build [--jobs N] [--verbose]
Every call recompiles from source; objects go to head_dim_attention_amd/_build/ and the shared
library to head_dim_attention_amd/libffpa.so.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libffpa.so")
ARCH = "gfx950"

# Packed-fp32 VALU forms are disabled for all device code: the compiler is kept from emitting
# v_pk_{add,mul,fma}_f32.
# MFMA accumulators are kept in VGPRs (-amdgpu-mfma-vgpr-form): the kernels read every score block
# with VALU instructions, and the stationary MFMA operands then go to AGPRs instead.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
    "-I", os.path.join(ROOT, "include"),
]


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libffpa.so)")


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l
                    and "argument unused during compilation" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(jobs: int | None = None, verbose: bool = False, out: str = LIB, extra_flags=()) -> str:
    """Compile every source under csrc/ and link `out` (default: the in-package libffpa.so)."""
    cc = hipcc()
    bdir = BUILD if out == LIB else out + ".objs"
    os.makedirs(bdir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(bdir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    flags = [*HIP_FLAGS, *extra_flags]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_run, [cc, *flags, "-c", s, "-o", o], verbose) for s, o in zip(srcs, objs)]
        for f in futs:
            f.result()
    tmp = out + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, out)
    return out


_RES_KEYS = (("VGPRs", "vgpr"), ("AGPRs", "agpr"), ("VGPRs Spill", "spill"), ("ScratchSize [bytes/lane]", "scratch"),
             ("LDS Size [bytes/block]", "lds"), ("Occupancy [waves/SIMD]", "occupancy"))


def resource_report(jobs: int | None = None) -> str:
    """Per-kernel register, spill, LDS and occupancy figures from the compiler's resource remarks
    (-Rpass-analysis=kernel-resource-usage) for every source, as a markdown table."""
    cc = hipcc()
    srcs = sources()
    tmpdir = BUILD + ".res"
    os.makedirs(tmpdir, exist_ok=True)

    def one(src):
        cmd = [cc, *HIP_FLAGS, "--cuda-device-only", "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o",
               os.path.join(tmpdir, os.path.basename(src) + ".o")]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"command failed: {' '.join(cmd)}\n{r.stderr}")
        rows, cur = [], None
        for line in r.stderr.splitlines():
            m = re.search(r"remark:\s+Function Name: (\S+)", line)
            if m:
                cur = {"name": m.group(1)}
                rows.append(cur)
                continue
            for key, col in _RES_KEYS:
                m = re.search(r"remark:\s+" + re.escape(key) + r": (\d+)", line)
                if m and cur is not None:
                    cur[col] = int(m.group(1))
        return os.path.basename(src), rows

    with cf.ThreadPoolExecutor(max_workers=jobs or len(srcs)) as ex:
        results = list(ex.map(one, srcs))
    demangle = shutil.which("c++filt") or shutil.which("llvm-cxxfilt")
    names = [row["name"] for _, rows in results for row in rows]
    pretty = {}
    if demangle:
        lines = subprocess.run([demangle], input="\n".join(names), capture_output=True, text=True).stdout.splitlines()
        if len(lines) == len(names):
            pretty = dict(zip(names, lines))
    # The bf16 and fp16 instances of a kernel share one row when their figures agree.
    merged = {}
    for src, rows in results:
        for row in rows:
            if "kernel" not in row["name"]:
                continue
            nm = re.sub(r"\(.*\)$", "", pretty.get(row["name"], row["name"])).replace("void ", "")
            nm = nm.replace("ffpa::", "")
            figs = tuple(row.get(c, "") for _, c in _RES_KEYS)
            key = (src, re.sub(r"\b(BF16|FP16)\b", "T", nm), figs)
            merged.setdefault(key, []).append("bf16" if "BF16" in nm else "fp16" if "FP16" in nm else "")
    out = ["| source | kernel | types | VGPRs | AGPRs | VGPR spill | scratch B/lane | LDS bytes | waves/SIMD |",
           "|---|---|---|---|---|---|---|---|---|"]
    for (src, nm, figs), types in merged.items():
        out.append(f"| {src} | `{nm}` | {'/'.join(t for t in types if t)} | " + " | ".join(str(f) for f in figs) + " |")
    return "\n".join(out) + "\n"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--out", default=LIB, help="output library path (variants for comparison)")
    ap.add_argument("--extra-flag", action="append", default=[], help="extra hipcc flag (repeatable)")
    ap.add_argument("--report-resources", action="store_true",
                    help="print each kernel's registers, spills, LDS and occupancy (no library is built)")
    a = ap.parse_args(argv)
    if a.report_resources:
        print(resource_report(a.jobs), end="")
        return 0
    print(build(a.jobs, a.verbose, os.path.abspath(a.out), a.extra_flag))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
