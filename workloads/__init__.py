"""Seeded synthetic inputs shared by the oracle checks, the GPU parity tests and the benchmark.

This module only draws random numbers and describes shapes; it holds none of the attention
arithmetic. Every tensor is drawn on the CPU from ``torch.Generator().manual_seed(seed)`` as
float32 standard normals in the order Q, K, V, dO, then scaled (where a workload asks for it) and
rounded to the storage dtype (bf16 or fp16). Callers copy the same tensors to the GPU and upcast
them to float64 for the oracle, so both sides see identical bits.

The five named workloads follow the shapes the ffpa-attn user guide uses for large head dims
(the Triton and CuTe-DSL backend pages show B=1, H=32, N=8192, D=512 bf16 in their examples;
varlen packs sequences as [T, H, D] with int32 cu_seqlens per the CuTe-DSL "Varlen (packed THD)
API" section).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

__all__ = ["Workload", "WORKLOADS", "dense_inputs", "varlen_inputs", "varlen_lengths", "get"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int          # dense batch, or number of sequences for varlen
    hq: int
    hkv: int
    n: int              # Nkv (and Nq unless nq is set) for dense workloads; unused for varlen
    d: int
    dtype: str          # "bf16" | "fp16"
    causal: bool
    backward: bool
    varlen: bool = False
    input_scale: float = 1.0
    nq: int = 0         # Nq when it differs from n (decode: a few queries against a long cache)

    @property
    def n_q(self) -> int:
        return self.nq if self.nq > 0 else self.n

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float16


WORKLOADS = {
    "fwd_d320_n512": Workload("fwd_d320_n512", 1, 2, 2, 512, 320, "bf16", False, False),
    "causal_d512_n4096": Workload("causal_d512_n4096", 1, 8, 8, 4096, 512, "bf16", True, True),
    "dense_d512_n8192": Workload("dense_d512_n8192", 1, 32, 32, 8192, 512, "bf16", False, True),
    "gqa_causal_d1024_n8192": Workload("gqa_causal_d1024_n8192", 1, 32, 8, 8192, 1024, "fp16", True, True,
                                       input_scale=0.5),
    "varlen_causal_d512": Workload("varlen_causal_d512", 8, 32, 32, 0, 512, "bf16", True, True, varlen=True),
    # Split-KV decode: one new query per head against a 64K-key cache, 4 query heads per KV head.
    "decode_gqa_d512_k65536": Workload("decode_gqa_d512_k65536", 1, 32, 8, 65536, 512, "bf16", True, False, nq=1),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def _gen(seed: int, device: str = "cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _draw(g: torch.Generator, shape, dtype: torch.dtype, scale: float) -> torch.Tensor:
    x = torch.randn(*shape, generator=g, dtype=torch.float32, device=g.device)
    if scale != 1.0:
        x = x * scale
    return x.to(dtype)


def dense_inputs(b: int, hq: int, hkv: int, nq: int, nkv: int, d: int, dtype: torch.dtype, seed: int,
                 input_scale: float = 1.0, with_grad: bool = True, device: str = "cpu"):
    """Return (q, k, v, do) tensors: q/do [b,hq,nq,d], k/v [b,hkv,nkv,d]. ``device`` other than the
    CPU draws the same distribution with that device's generator (different values; for timing
    large inputs without a host round trip)."""
    g = _gen(seed, device)
    q = _draw(g, (b, hq, nq, d), dtype, input_scale)
    k = _draw(g, (b, hkv, nkv, d), dtype, input_scale)
    v = _draw(g, (b, hkv, nkv, d), dtype, input_scale)
    do = _draw(g, (b, hq, nq, d), dtype, input_scale) if with_grad else None
    return q, k, v, do


def varlen_lengths(nseq: int, seed: int, lo_units: int = 8, hi_units: int = 128, unit: int = 64) -> list[int]:
    """Sequence lengths drawn uniformly from the multiples of ``unit`` in [lo_units*unit, hi_units*unit]."""
    g = _gen(seed)
    units = torch.randint(lo_units, hi_units + 1, (nseq,), generator=g)
    return [int(u) * unit for u in units]


def cu_from_lengths(lengths) -> torch.Tensor:
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def varlen_inputs(lengths_q, lengths_k, hq: int, hkv: int, d: int, dtype: torch.dtype, seed: int,
                  input_scale: float = 1.0, with_grad: bool = True, device: str = "cpu"):
    """Return (q, k, v, do, cu_q, cu_k): packed [T, H, D] tensors and int32 cumulative lengths (CPU;
    ``device`` as in dense_inputs for the packed tensors)."""
    cu_q = cu_from_lengths(lengths_q)
    cu_k = cu_from_lengths(lengths_k)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    g = _gen(seed + 1, device)
    q = _draw(g, (tq, hq, d), dtype, input_scale)
    k = _draw(g, (tk, hkv, d), dtype, input_scale)
    v = _draw(g, (tk, hkv, d), dtype, input_scale)
    do = _draw(g, (tq, hq, d), dtype, input_scale) if with_grad else None
    return q, k, v, do, cu_q, cu_k


def workload_inputs(w: Workload, seed: int, varlen_lengths_override: Optional[list] = None, device: str = "cpu"):
    """Inputs for a named workload. Varlen lengths come from ``varlen_lengths(w.batch, seed)`` (always
    the CPU generator, so they do not depend on ``device``)."""
    if w.varlen:
        lens = varlen_lengths_override if varlen_lengths_override is not None else varlen_lengths(w.batch, seed)
        return varlen_inputs(lens, lens, w.hq, w.hkv, w.d, w.torch_dtype, seed, w.input_scale, w.backward, device)
    return dense_inputs(w.batch, w.hq, w.hkv, w.n_q, w.n, w.d, w.torch_dtype, seed, w.input_scale, w.backward,
                        device)
