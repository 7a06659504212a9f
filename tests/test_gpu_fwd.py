"""GPU parity of the forward kernel against the float64 oracle (through the C ABI binding)."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import ref
from tests.gpu_helpers import check_o_lse, rel_l2, to64

pytestmark = pytest.mark.gpu

BF, FP = torch.bfloat16, torch.float16

# (B, Hq, Hkv, Nq, Nkv, D, dtype, causal): several tiles, ragged tails, every tile configuration
# (D <= 512 with two head-dim halves; D > 512 with four quarters, padded and exact), cross-attention
# both ways (causal Nq > Nkv has rows with no legal key), GQA/MQA, single query and single key.
DENSE_CASES = [
    (1, 2, 2, 64, 64, 320, BF, False),
    (1, 2, 2, 17, 17, 320, BF, True),
    (2, 4, 2, 65, 200, 352, BF, True),
    (1, 2, 1, 200, 65, 512, FP, True),
    (1, 3, 3, 129, 129, 512, BF, False),
    (1, 4, 1, 130, 130, 544, BF, False),
    (1, 2, 2, 1, 300, 1024, FP, False),
    (1, 2, 2, 257, 257, 1024, BF, True),
    (1, 8, 2, 100, 333, 768, FP, False),
    (1, 2, 2, 96, 1, 416, BF, False),
    (1, 2, 2, 70, 40, 896, FP, True),
]


def _ids(c):
    b, hq, hkv, nq, nkv, d, dt, causal = c
    return f"b{b}h{hq}x{hkv}q{nq}k{nkv}d{d}{'bf16' if dt == BF else 'fp16'}{'c' if causal else ''}"


@pytest.fixture(scope="module")
def lib():
    import head_dim_attention_amd as F
    F.load_library()
    return F


@pytest.mark.parametrize("case", DENSE_CASES, ids=_ids)
def test_fwd_dense(lib, case):
    b, hq, hkv, nq, nkv, d, dt, causal = case
    q, k, v, _ = W.dense_inputs(b, hq, hkv, nq, nkv, d, dt, seed=1234 + nq + d, with_grad=False)
    scale = 1.0 / math.sqrt(d)
    print(f"case {_ids(case)}", flush=True)
    o, lse = lib.ffpa_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = ref.attn_fwd(q, k, v, scale=np.float64(np.float32(scale)), causal=causal)
    check_o_lse(o, lse, o_ref, lse_ref, dt, _ids(case))


def test_fwd_causal_row0_exact(lib):
    """Causal, Nq == Nkv: query 0 sees only key 0, so O_0 is V_0 exactly."""
    q, k, v, _ = W.dense_inputs(1, 4, 2, 80, 80, 512, BF, seed=7, with_grad=False)
    o, lse = lib.ffpa_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True)
    torch.cuda.synchronize()
    vr = v.repeat_interleave(2, dim=1)
    assert torch.equal(o[:, :, 0].cpu(), vr[:, :, 0])


def test_fwd_empty_rows_exact(lib):
    """Causal with Nq > Nkv: the first Nq - Nkv rows have no legal key: O = 0 and LSE = -inf exactly."""
    q, k, v, _ = W.dense_inputs(1, 2, 2, 100, 30, 320, FP, seed=8, with_grad=False)
    o, lse = lib.ffpa_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True)
    torch.cuda.synchronize()
    assert torch.all(o[:, :, :70] == 0)
    assert torch.all(torch.isneginf(lse[:, :, :70]))
    assert torch.all(torch.isfinite(lse[:, :, 70:]))


def test_fwd_zero_query_prefix_means(lib):
    """Q = 0: uniform weights over the legal keys; causal gives prefix means (bottom-right offset)."""
    _, k, v, _ = W.dense_inputs(1, 2, 2, 1, 90, 384, BF, seed=9, with_grad=False)
    q = torch.zeros(1, 2, 60, 384, dtype=BF)
    o, lse = lib.ffpa_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True)
    torch.cuda.synchronize()
    vd = v.double()
    for i in (0, 1, 29, 59):
        last = i + 90 - 60
        exp = vd[0, :, :last + 1].mean(dim=1)
        assert torch.max(torch.abs(o[0, :, i].cpu().double() - exp)) < 2e-2
        assert torch.allclose(lse[0, :, i].cpu().double(), torch.full((2,), math.log(last + 1), dtype=torch.float64),
                              atol=1e-3)


SPLIT_CASES = [
    # (B, Hq, Hkv, Nq, Nkv, D, dtype, causal): grids below two workgroups per compute unit, which
    # the binding sends through ffpa_fwd_split
    (1, 8, 8, 2048, 2048, 512, BF, True),
    (1, 4, 2, 1000, 1500, 384, FP, False),
    (2, 2, 1, 700, 520, 320, BF, True),     # causal Nq > Nkv: rows without a legal key
    (1, 2, 2, 300, 4096, 768, FP, True),    # D > 512 form
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: f"b{c[0]}h{c[1]}x{c[2]}q{c[3]}k{c[4]}d{c[5]}{'c' if c[7] else ''}")
def test_fwd_split(lib, case):
    """Key-range split forward: parity with the oracle, agreement with the unsplit forward up to
    fp32 summation order (O within 1e-2 relative L2, LSE within 1e-4, -inf rows identical) and
    run-to-run bit equality."""
    from head_dim_attention_amd import _binding as B
    b, hq, hkv, nq, nkv, d, dt, causal = case
    assert B.ffpa_fwd_split_workspace_bytes(b, hq, hkv, nq, nkv, d) > 0
    q, k, v, _ = W.dense_inputs(b, hq, hkv, nq, nkv, d, dt, seed=300 + d + nq, with_grad=False)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    scale = 1.0 / math.sqrt(d)
    print(f"split case {case}", flush=True)
    o, lse = lib.ffpa_fwd(qc, kc, vc, causal=causal, scale=scale)
    o3, l3 = lib.ffpa_fwd(qc, kc, vc, causal=causal, scale=scale)
    o2, l2 = lib.ffpa_fwd(qc, kc, vc, causal=causal, scale=scale, split=False)
    torch.cuda.synchronize()
    assert torch.equal(o, o3) and torch.equal(lse, l3)
    assert torch.equal(torch.isneginf(lse), torch.isneginf(l2))
    fin = torch.isfinite(l2)
    assert float((lse[fin] - l2[fin]).abs().max()) < 1e-4
    assert rel_l2(to64(o), to64(o2)) < 1e-2
    o_ref, lse_ref = ref.attn_fwd(q, k, v, scale=np.float64(np.float32(scale)), causal=causal)
    check_o_lse(o, lse, o_ref, lse_ref, dt, f"split {case}")


def test_fwd_gqa_equals_repeated(lib):
    q, k, v, _ = W.dense_inputs(1, 8, 2, 150, 150, 512, BF, seed=10, with_grad=False)
    o1, l1 = lib.ffpa_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True)
    o2, l2 = lib.ffpa_fwd(q.cuda(), k.repeat_interleave(4, 1).cuda(), v.repeat_interleave(4, 1).cuda(), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_deterministic(lib):
    q, k, v, _ = W.dense_inputs(1, 4, 4, 300, 300, 640, FP, seed=11, with_grad=False)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    o1, l1 = lib.ffpa_fwd(qc, kc, vc, causal=False)
    o2, l2 = lib.ffpa_fwd(qc, kc, vc, causal=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fwd_large_scores_rescale_path(lib):
    """Scores whose row max grows by far more than 2^8 across tiles exercise the rescaling loop."""
    q, k, v, _ = W.dense_inputs(1, 2, 2, 64, 256, 320, BF, seed=12, with_grad=False)
    ramp = torch.linspace(0.2, 6.0, 256).view(1, 1, 256, 1)
    k = (k.float() * ramp).to(BF)
    q = (q.float() * 3.0).to(BF)
    o, lse = lib.ffpa_fwd(q.cuda(), k.cuda(), v.cuda(), causal=False)
    torch.cuda.synchronize()
    scale = 1.0 / math.sqrt(320)
    o_ref, lse_ref = ref.attn_fwd(q, k, v, scale=np.float64(np.float32(scale)), causal=False)
    check_o_lse(o, lse, o_ref, lse_ref, BF, "rescale")


VARLEN_CASES = [
    # (lengths_q, lengths_k, Hq, Hkv, D, dtype, causal)
    ([17, 64, 200, 1], [17, 64, 200, 1], 4, 4, 512, BF, True),
    ([0, 33, 130, 64], [5, 0, 64, 130], 4, 2, 320, FP, True),
    ([50, 7, 129], [80, 200, 3], 2, 1, 1024, BF, False),
    ([64, 64], [64, 64], 2, 2, 704, FP, True),
    # head counts that are multiples of 8 take the per-XCD head interleave of the varlen grid
    ([0, 45, 300, 129, 64], [10, 45, 280, 0, 64], 8, 2, 512, BF, True),
    ([33, 150, 7], [33, 150, 7], 16, 8, 384, FP, False),
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=lambda c: f"q{c[0]}k{c[1]}h{c[2]}x{c[3]}d{c[4]}{'c' if c[6] else ''}")
def test_fwd_varlen(lib, case):
    lq, lk, hq, hkv, d, dt, causal = case
    q, k, v, _, cu_q, cu_k = W.varlen_inputs(lq, lk, hq, hkv, d, dt, seed=99 + d, with_grad=False)
    scale = 1.0 / math.sqrt(d)
    o, lse = lib.ffpa_varlen_fwd(q.cuda(), k.cuda(), v.cuda(), cu_q.cuda(), cu_k.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = ref.varlen_fwd(q, k, v, cu_q.numpy(), cu_k.numpy(), scale=np.float64(np.float32(scale)),
                                    causal=causal)
    check_o_lse(o, lse, o_ref, lse_ref, dt, f"varlen {lq} {lk}")


def test_fwd_workload_d320_n512(lib):
    """The small forward-only workload (B=1, H=2, N=512, D=320, bf16, non-causal) at full size."""
    w = W.get("fwd_d320_n512")
    q, k, v, _ = W.workload_inputs(w, seed=2024)
    scale = 1.0 / math.sqrt(w.d)
    o, lse = lib.ffpa_fwd(q.cuda(), k.cuda(), v.cuda(), causal=w.causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = ref.attn_fwd(q, k, v, scale=np.float64(np.float32(scale)), causal=w.causal)
    check_o_lse(o, lse, o_ref, lse_ref, w.torch_dtype, w.name)
