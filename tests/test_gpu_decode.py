"""GPU parity of the split-KV decode forward (ffpa_decode_fwd) against the float64 oracle.

The decode path computes the same O and LSE as the forward ("Triton Backend", "Feature support":
decode as a two-stage split-KV path), so the oracle's forward is its reference. Cases cover one
to seven queries, GQA groups whose (query head, query) rows fill one or several 32-row blocks,
every head-dim configuration of the decode kernel (D <= 512 double-buffered, D > 512 single),
causal rows without a legal key (Nq > Nkv), ragged key tails and key counts that give one range or
many.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import ref
from tests.gpu_helpers import check_o_lse, rel_l2, to64

pytestmark = pytest.mark.gpu

BF, FP = torch.bfloat16, torch.float16

# (B, Hq, Hkv, Nq, Nkv, D, dtype, causal)
DECODE_CASES = [
    (1, 8, 2, 1, 1000, 512, BF, False),
    (2, 4, 4, 3, 777, 320, FP, True),
    (1, 32, 4, 7, 2049, 512, BF, True),    # 56 rows per KV head: two row blocks
    (1, 4, 1, 5, 300, 1024, FP, False),    # MQA, D > 512
    (1, 2, 2, 2, 40, 768, BF, True),       # two key tiles: a single range
    (1, 16, 1, 7, 513, 448, BF, True),     # 112 rows: four row blocks
    (1, 2, 2, 7, 3, 512, BF, True),        # causal Nq > Nkv: rows without a legal key
    (3, 6, 3, 1, 4099, 640, FP, True),
]


def _ids(c):
    b, hq, hkv, nq, nkv, d, dt, causal = c
    return f"b{b}h{hq}x{hkv}q{nq}k{nkv}d{d}{'bf16' if dt == BF else 'fp16'}{'c' if causal else ''}"


@pytest.fixture(scope="module")
def lib():
    import head_dim_attention_amd as F
    F.load_library()
    return F


@pytest.mark.parametrize("case", DECODE_CASES, ids=_ids)
def test_decode_matches_oracle(lib, case):
    b, hq, hkv, nq, nkv, d, dt, causal = case
    q, k, v, _ = W.dense_inputs(b, hq, hkv, nq, nkv, d, dt, seed=99 + nq + nkv, with_grad=False)
    scale = 1.0 / math.sqrt(d)
    print(f"case {_ids(case)}", flush=True)
    o, lse = lib.ffpa_decode_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = ref.attn_fwd(q, k, v, scale=np.float64(np.float32(scale)), causal=causal)
    check_o_lse(o, lse, o_ref, lse_ref, dt, _ids(case))


def test_decode_matches_forward_and_is_deterministic(lib):
    """Same result as ffpa_fwd up to fp32 addition order; repeated calls are bit-identical."""
    q, k, v, _ = W.dense_inputs(1, 16, 4, 4, 3000, 512, BF, seed=5, with_grad=False)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    o1, l1 = lib.ffpa_decode_fwd(qc, kc, vc, causal=True)
    o2, l2 = lib.ffpa_decode_fwd(qc, kc, vc, causal=True)
    of, lf = lib.ffpa_fwd(qc, kc, vc, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert rel_l2(to64(o1), to64(of)) < 1e-2
    assert float((l1 - lf).abs().max()) < 1e-4


def test_decode_full_size_sampled_rows(lib):
    """The measured decode workload (1 x 32 query heads, 8 KV heads, one query, 64K keys, D=512):
    all rows against the oracle, which is cheap for one query per head."""
    w = W.get("decode_gqa_d512_k65536")
    q, k, v, _ = W.workload_inputs(w, seed=2024)
    scale = 1.0 / math.sqrt(w.d)
    o, lse = lib.ffpa_decode_fwd(q.cuda(), k.cuda(), v.cuda(), causal=w.causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = ref.attn_fwd(q, k, v, scale=np.float64(np.float32(scale)), causal=w.causal)
    check_o_lse(o, lse, o_ref, lse_ref, BF, w.name)


def test_decode_autograd_route(lib):
    """ffpa_attn_func takes the decode path for Nq < 8; its backward is the usual one."""
    q, k, v, do = W.dense_inputs(1, 8, 2, 3, 500, 512, BF, seed=6)
    qc, kc, vc = (x.cuda().requires_grad_(True) for x in (q, k, v))
    o = lib.ffpa_attn_func(qc, kc, vc, is_causal=True)
    o.backward(do.cuda())
    od, _ = lib.ffpa_decode_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), od)
    g_ref = ref.attn_bwd(q, k, v, do, scale=np.float64(np.float32(1.0 / math.sqrt(512))), causal=True)
    for g, r in zip((qc.grad, kc.grad, vc.grad), g_ref):
        assert rel_l2(to64(g), r) < 2e-2


def test_decode_workspace_checks(lib):
    from head_dim_attention_amd import _binding as B
    L = B.load_library()
    q = torch.zeros(1, 4, 2, 512, dtype=BF, device="cuda")
    k = torch.zeros(1, 2, 700, 512, dtype=BF, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(1, 4, 2, dtype=torch.float32, device="cuda")
    need = B.ffpa_decode_workspace_bytes(1, 4, 2, 2, 700, 512)
    assert need > 0 and need % (4 * 513) == 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    P = B._ptr
    args = (P(q), P(k), P(k), P(o), P(lse), 1, 4, 2, 2, 700, 512, 0, ctypes.c_float(0.04), 1)
    S = ctypes.c_void_p(0)
    assert L.ffpa_decode_fwd(*args, ctypes.c_void_p(0), need, S) == 1     # no workspace
    assert L.ffpa_decode_fwd(*args, P(ws), need - 1, S) == 1             # too small
    assert L.ffpa_decode_fwd(*args, P(ws), need, S) == 0
    torch.cuda.synchronize()
