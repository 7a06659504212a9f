"""GPU parity of the four-stage backward (preprocess, dV, dK, dQ) against the float64 oracle.

Every parity case runs both paths: with the P/dS workspace (dK stores P and dS; dV = P^T dO and
dQ = dS K are products) and without it (dV and dQ recompute S, P, dP and dS).
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import ref
from tests.gpu_helpers import check_grads, to64

pytestmark = pytest.mark.gpu

BF, FP = torch.bfloat16, torch.float16

# (B, Hq, Hkv, Nq, Nkv, D, dtype, causal)
DENSE_CASES = [
    (1, 2, 2, 64, 64, 320, BF, False),
    (1, 2, 2, 33, 33, 320, FP, True),
    (2, 4, 2, 65, 200, 352, BF, True),
    (1, 2, 1, 200, 65, 512, FP, True),
    (1, 3, 3, 129, 129, 512, BF, False),
    (1, 4, 1, 130, 130, 544, BF, True),
    (1, 2, 2, 1, 300, 1024, FP, False),
    (1, 2, 2, 257, 257, 1024, BF, True),
    (1, 8, 2, 100, 333, 768, FP, False),
    (1, 2, 2, 96, 1, 416, BF, False),
    (1, 4, 2, 70, 40, 896, FP, True),
]


def _ids(c):
    b, hq, hkv, nq, nkv, d, dt, causal = c
    return f"b{b}h{hq}x{hkv}q{nq}k{nkv}d{d}{'bf16' if dt == BF else 'fp16'}{'c' if causal else ''}"


@pytest.fixture(scope="module")
def lib():
    import head_dim_attention_amd as F
    F.load_library()
    return F


def _run_dense(lib, q, k, v, do, causal, scale, store_ds=True):
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = lib.ffpa_fwd(qc, kc, vc, causal=causal, scale=scale)
    dq, dk, dv = lib.ffpa_bwd(qc, kc, vc, o, doc, lse, causal=causal, scale=scale, store_ds=store_ds)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


PATHS = pytest.mark.parametrize("store_ds", [True, False], ids=["ds", "recompute"])


@PATHS
@pytest.mark.parametrize("case", DENSE_CASES, ids=_ids)
def test_bwd_dense(lib, case, store_ds):
    b, hq, hkv, nq, nkv, d, dt, causal = case
    q, k, v, do = W.dense_inputs(b, hq, hkv, nq, nkv, d, dt, seed=4321 + nq + d)
    scale = 1.0 / math.sqrt(d)
    print(f"case {_ids(case)} store_ds={store_ds}", flush=True)
    _, _, dq, dk, dv = _run_dense(lib, q, k, v, do, causal, scale, store_ds)
    g_ref = ref.attn_bwd(q, k, v, do, scale=np.float64(np.float32(scale)), causal=causal)
    check_grads((dq, dk, dv), g_ref, _ids(case))


@pytest.mark.parametrize("d", [512, 640])
def test_bwd_ds_path_matches_recompute(lib, d):
    """The two paths agree up to the order of fp32 additions and the rounding of P and dS."""
    q, k, v, do = W.dense_inputs(1, 4, 2, 161, 203, d, BF, seed=26)
    for causal in (False, True):
        _, _, dq1, dk1, dv1 = _run_dense(lib, q, k, v, do, causal, None, True)
        _, _, dq2, dk2, dv2 = _run_dense(lib, q, k, v, do, causal, None, False)
        for a, b in ((dq1, dq2), (dk1, dk2), (dv1, dv2)):
            x, y = to64(a), to64(b)
            assert np.linalg.norm(x - y) / np.linalg.norm(y) < 5e-3


@pytest.mark.parametrize("d", [320, 512, 768])
def test_bwd_stages_equal_bwd(lib, d):
    """ffpa_bwd_stage in the order 0, 4, 1, 2, 3 gives exactly ffpa_bwd's results, with and without
    the workspace; stage 4 without a workspace launches nothing."""
    q, k, v, do = W.dense_inputs(1, 4, 2, 100, 140, d, BF, seed=27)
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = lib.ffpa_fwd(qc, kc, vc, causal=True)
    for store_ds in (True, False):
        ref_g = lib.ffpa_bwd(qc, kc, vc, o, doc, lse, causal=True, store_ds=store_ds)
        nws = lib.ffpa_bwd_workspace_bytes(1, 4, 100, 140) if store_ds else 0
        ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
        delta = torch.empty_like(lse)
        dq, dk, dv = torch.empty_like(qc), torch.empty_like(kc), torch.empty_like(vc)
        for stage in (0, 4, 1, 2, 3):
            lib.ffpa_bwd_stage(stage, qc, kc, vc, o, doc, lse, delta, dq, dk, dv, causal=True, workspace=ws)
        torch.cuda.synchronize()
        for x, y in zip((dq, dk, dv), ref_g):
            assert torch.equal(x, y)


@PATHS
def test_bwd_empty_rows_zero_grad(lib, store_ds):
    """Causal with Nq > Nkv: rows without a legal key get dQ = 0 exactly and add nothing to dK/dV."""
    q, k, v, do = W.dense_inputs(1, 2, 2, 100, 30, 320, FP, seed=21)
    _, _, dq, dk, dv = _run_dense(lib, q, k, v, do, True, None, store_ds)
    assert torch.all(dq[:, :, :70] == 0)
    do2 = do.clone()
    do2[:, :, :70] = 100.0
    _, _, dq2, dk2, dv2 = _run_dense(lib, q, k, v, do2, True, None, store_ds)
    assert torch.equal(dk, dk2) and torch.equal(dv, dv2)
    assert torch.all(dq2[:, :, :70] == 0)


@PATHS
def test_bwd_deterministic(lib, store_ds):
    q, k, v, do = W.dense_inputs(1, 4, 2, 200, 200, 512, BF, seed=22)
    r1 = _run_dense(lib, q, k, v, do, True, None, store_ds)
    r2 = _run_dense(lib, q, k, v, do, True, None, store_ds)
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


def test_bwd_gqa_matches_group_sum(lib):
    """GQA dK/dV equal the group sums of MHA gradients on repeated K/V (to fp32 accumulation)."""
    q, k, v, do = W.dense_inputs(1, 8, 2, 96, 96, 512, BF, seed=23)
    _, _, dq1, dk1, dv1 = _run_dense(lib, q, k, v, do, True, None)
    _, _, dq2, dk2, dv2 = _run_dense(lib, q, k.repeat_interleave(4, 1), v.repeat_interleave(4, 1), do, True, None)
    assert torch.equal(dq1, dq2)
    g = lambda x: to64(x).reshape(1, 2, 4, 96, 512).sum(axis=2)
    for a, b in ((dk1, dk2), (dv1, dv2)):
        x, y = to64(a), g(b)
        assert np.linalg.norm(x - y) / np.linalg.norm(y) < 1e-2


def test_bwd_autograd_wrapper(lib):
    q, k, v, do = W.dense_inputs(1, 2, 1, 80, 80, 448, BF, seed=24)
    qc, kc, vc = (x.cuda().requires_grad_(True) for x in (q, k, v))
    o = lib.ffpa_attn_func(qc, kc, vc, is_causal=True)
    o.backward(do.cuda())
    _, _, dq, dk, dv = _run_dense(lib, q, k, v, do, True, None)
    assert torch.equal(qc.grad, dq) and torch.equal(kc.grad, dk) and torch.equal(vc.grad, dv)


VARLEN_CASES = [
    ([17, 64, 200, 1], [17, 64, 200, 1], 4, 4, 512, BF, True),
    ([0, 33, 130, 64], [5, 0, 64, 130], 4, 2, 320, FP, True),
    ([50, 7, 129], [80, 200, 3], 2, 1, 1024, BF, False),
    ([64, 64], [64, 64], 2, 2, 704, FP, True),
    # head counts that are multiples of 8 take the per-XCD head interleave of the varlen grid
    ([0, 45, 300, 129, 64], [10, 45, 280, 0, 64], 8, 2, 512, BF, True),
    ([33, 150, 7], [33, 150, 7], 16, 8, 384, FP, False),
]


@PATHS
@pytest.mark.parametrize("case", VARLEN_CASES, ids=lambda c: f"q{c[0]}k{c[1]}h{c[2]}x{c[3]}d{c[4]}{'c' if c[6] else ''}")
def test_bwd_varlen(lib, case, store_ds):
    lq, lk, hq, hkv, d, dt, causal = case
    q, k, v, do, cu_q, cu_k = W.varlen_inputs(lq, lk, hq, hkv, d, dt, seed=77 + d)
    scale = 1.0 / math.sqrt(d)
    qc, kc, vc, doc, cq, ck = q.cuda(), k.cuda(), v.cuda(), do.cuda(), cu_q.cuda(), cu_k.cuda()
    o, lse = lib.ffpa_varlen_fwd(qc, kc, vc, cq, ck, causal=causal, scale=scale)
    dq, dk, dv = lib.ffpa_varlen_bwd(qc, kc, vc, o, doc, lse, cq, ck, causal=causal, scale=scale, store_ds=store_ds)
    torch.cuda.synchronize()
    g_ref = ref.varlen_bwd(q, k, v, do, cu_q.numpy(), cu_k.numpy(), scale=np.float64(np.float32(scale)),
                           causal=causal)
    check_grads((dq, dk, dv), g_ref, f"varlen {lq} {lk}")


@PATHS
def test_bwd_varlen_equals_dense(lib, store_ds):
    """A packed batch gives the same gradients as separate dense calls per sequence."""
    lens = [40, 97, 64]
    q, k, v, do, cu_q, cu_k = W.varlen_inputs(lens, lens, 2, 2, 512, BF, seed=25)
    qc, kc, vc, doc, cq = q.cuda(), k.cuda(), v.cuda(), do.cuda(), cu_q.cuda()
    o, lse = lib.ffpa_varlen_fwd(qc, kc, vc, cq, causal=True)
    dq, dk, dv = lib.ffpa_varlen_bwd(qc, kc, vc, o, doc, lse, cq, causal=True, store_ds=store_ds)
    torch.cuda.synchronize()
    for s, n in enumerate(lens):
        a, b = int(cu_q[s]), int(cu_q[s + 1])
        sl = lambda x: x[a:b].transpose(0, 1).unsqueeze(0).contiguous()
        od, lsed = lib.ffpa_fwd(sl(qc), sl(kc), sl(vc), causal=True, split=False)  # varlen has no split
        g = lib.ffpa_bwd(sl(qc), sl(kc), sl(vc), od, sl(doc), lsed, causal=True, store_ds=store_ds)
        torch.cuda.synchronize()
        assert torch.equal(od, sl(o)) and torch.equal(lsed[0], lse[:, a:b])
        for x, y in zip((dq, dk, dv), g):
            assert torch.equal(sl(x), y)


# ----------------------------------------------------------------------------------------------
# The returned LSE is differentiable: loss = sum(dO * O) + sum(g * LSE).
# ----------------------------------------------------------------------------------------------
DLSE_CASES = [
    (1, 4, 2, 100, 60, 512, BF, True),     # causal Nq > Nkv: 40 empty rows per head
    (1, 2, 2, 130, 130, 384, FP, False),
    (1, 4, 1, 96, 200, 768, BF, True),
]


@PATHS
@pytest.mark.parametrize("case", DLSE_CASES, ids=_ids)
def test_bwd_dlse(lib, case, store_ds):
    b, hq, hkv, nq, nkv, d, dt, causal = case
    q, k, v, do = W.dense_inputs(b, hq, hkv, nq, nkv, d, dt, seed=601 + d)
    g = torch.randn((b, hq, nq), generator=torch.Generator().manual_seed(602 + d), dtype=torch.float32)
    scale = 1.0 / math.sqrt(d)
    print(f"case {_ids(case)} dlse store_ds={store_ds}", flush=True)
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = lib.ffpa_fwd(qc, kc, vc, causal=causal, scale=scale)
    dq, dk, dv = lib.ffpa_bwd(qc, kc, vc, o, doc, lse, causal=causal, scale=scale, store_ds=store_ds, dlse=g.cuda())
    torch.cuda.synchronize()
    g_ref = ref.attn_bwd(q, k, v, do, scale=np.float64(np.float32(scale)), causal=causal, dlse=g.double().numpy())
    check_grads((dq, dk, dv), g_ref, _ids(case) + " dlse")
    if causal and nq > nkv:
        assert torch.all(dq[:, :, :nq - nkv] == 0)


def test_bwd_dlse_only(lib):
    """dO = 0 leaves only the LSE term: dV is exactly zero and dQ/dK match the oracle."""
    q, k, v, do = W.dense_inputs(1, 2, 2, 80, 80, 512, BF, seed=603)
    g = torch.randn((1, 2, 80), generator=torch.Generator().manual_seed(604))
    do = torch.zeros_like(do)
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = lib.ffpa_fwd(qc, kc, vc, causal=True)
    dq, dk, dv = lib.ffpa_bwd(qc, kc, vc, o, doc, lse, causal=True, dlse=g.cuda())
    torch.cuda.synchronize()
    assert torch.all(dv == 0)
    g_ref = ref.attn_bwd(q, k, v, do, scale=np.float64(np.float32(1 / math.sqrt(512))), causal=True,
                         dlse=g.double().numpy())
    for x, r in ((dq, g_ref[0]), (dk, g_ref[1])):
        assert np.linalg.norm(to64(x) - r) / np.linalg.norm(r) <= 2e-2


def test_autograd_return_lse_is_differentiable(lib):
    """ffpa_attn_func(return_lse=True): a loss that uses the LSE gets the LSE's gradient."""
    q, k, v, do = W.dense_inputs(1, 4, 2, 90, 120, 512, BF, seed=605)
    g = torch.randn((1, 4, 90), generator=torch.Generator().manual_seed(606))
    qc, kc, vc = (x.cuda().requires_grad_(True) for x in (q, k, v))
    o, lse = lib.ffpa_attn_func(qc, kc, vc, is_causal=True, return_lse=True)
    ((o.float() * do.cuda().float()).sum() + (lse * g.cuda()).sum()).backward()
    g_ref = ref.attn_bwd(q, k, v, do, scale=np.float64(np.float32(1 / math.sqrt(512))), causal=True,
                         dlse=g.double().numpy())
    check_grads((qc.grad, kc.grad, vc.grad), g_ref, "autograd lse")
    # LSE alone: the output O is unused (its gradient is None inside the wrapper)
    qc.grad = kc.grad = vc.grad = None
    _, lse2 = lib.ffpa_attn_func(qc, kc, vc, is_causal=True, return_lse=True)
    (lse2 * g.cuda()).sum().backward()
    g_ref2 = ref.attn_bwd(q, k, v, np.zeros(do.shape), scale=np.float64(np.float32(1 / math.sqrt(512))),
                          causal=True, dlse=g.double().numpy())
    assert torch.all(vc.grad == 0)
    for x, r in ((qc.grad, g_ref2[0]), (kc.grad, g_ref2[1])):
        assert np.linalg.norm(to64(x) - r) / np.linalg.norm(r) <= 2e-2


@PATHS
def test_bwd_varlen_dlse(lib, store_ds):
    lq, lk = [0, 33, 130, 64], [5, 0, 64, 130]
    q, k, v, do, cu_q, cu_k = W.varlen_inputs(lq, lk, 4, 2, 512, BF, seed=607)
    g = torch.randn((4, sum(lq)), generator=torch.Generator().manual_seed(608))
    qc, kc, vc, doc, cq, ck = q.cuda(), k.cuda(), v.cuda(), do.cuda(), cu_q.cuda(), cu_k.cuda()
    o, lse = lib.ffpa_varlen_fwd(qc, kc, vc, cq, ck, causal=True)
    dq, dk, dv = lib.ffpa_varlen_bwd(qc, kc, vc, o, doc, lse, cq, ck, causal=True, store_ds=store_ds, dlse=g.cuda())
    torch.cuda.synchronize()
    g_ref = ref.varlen_bwd(q, k, v, do, cu_q.numpy(), cu_k.numpy(), scale=np.float64(np.float32(1 / math.sqrt(512))),
                           causal=True, dlse=g.double().numpy())
    check_grads((dq, dk, dv), g_ref, "varlen dlse")


def test_varlen_autograd_return_lse(lib):
    lens = [40, 97, 64]
    q, k, v, do, cu_q, cu_k = W.varlen_inputs(lens, lens, 2, 2, 512, BF, seed=609)
    g = torch.randn((2, sum(lens)), generator=torch.Generator().manual_seed(610))
    qc, kc, vc = (x.cuda().requires_grad_(True) for x in (q, k, v))
    o, lse = lib.ffpa_attn_varlen_func(qc, kc, vc, cu_q.cuda(), causal=True, return_lse=True)
    ((o.float() * do.cuda().float()).sum() + (lse * g.cuda()).sum()).backward()
    g_ref = ref.varlen_bwd(q, k, v, do, cu_q.numpy(), cu_q.numpy(), scale=np.float64(np.float32(1 / math.sqrt(512))),
                           causal=True, dlse=g.double().numpy())
    check_grads((qc.grad, kc.grad, vc.grad), g_ref, "varlen autograd lse")


def test_varlen_exact_workspace_equals_bound(lib):
    """The exact-size P/dS workspace (host copies of cu_seqlens) gives bit-identical gradients to
    the bound-sized one."""
    lq, lk = [0, 45, 300, 129, 64], [10, 45, 280, 0, 64]
    q, k, v, do, cu_q, cu_k = W.varlen_inputs(lq, lk, 8, 2, 512, BF, seed=611)
    qc, kc, vc, doc, cq, ck = q.cuda(), k.cuda(), v.cuda(), do.cuda(), cu_q.cuda(), cu_k.cuda()
    o, lse = lib.ffpa_varlen_fwd(qc, kc, vc, cq, ck, causal=True)
    mq, mk = max(lq), max(lk)
    exact = lib.ffpa_varlen_bwd(qc, kc, vc, o, doc, lse, cq, ck, mq, mk, causal=True, store_ds=True)
    bound = lib.ffpa_varlen_bwd(qc, kc, vc, o, doc, lse, cq, ck, mq, mk, causal=True, store_ds=True, validate=False)
    torch.cuda.synchronize()
    from head_dim_attention_amd import _binding as B
    assert B.ffpa_varlen_bwd_workspace_bytes_exact(8, cu_q.tolist(), cu_k.tolist(), sum(lq), sum(lk), mq, mk) < \
        B.ffpa_varlen_bwd_workspace_bytes(8, sum(lq), sum(lk), mq, mk)
    for x, y in zip(exact, bound):
        assert torch.equal(x, y)


# (batch, hq, hkv, nq, nkv, d, causal): slice counts (batch x KV heads x head-dim chunks) of 2 and
# 4 take the round-robin order of the one-launch products, 8 the per-XCD order, with more key
# tiles than query tiles, fewer, or as many.
@pytest.mark.parametrize("b,hq,hkv,nq,nkv,d,causal", [
    (1, 4, 2, 300, 260, 512, True), (1, 4, 2, 300, 260, 768, False), (1, 4, 2, 300, 260, 384, True),
    (1, 16, 8, 300, 420, 512, True), (2, 8, 4, 420, 260, 384, True), (1, 8, 8, 200, 200, 320, False)])
def test_bwd_fused_products_equal_stages(lib, b, hq, hkv, nq, nkv, d, causal):
    """Stage 5 (dK, dV and dQ in one launch, which ffpa_bwd uses for small dense grids) equals
    stages 1, 2 and 3 bit for bit."""
    print(f"fused products b={b} hq={hq} hkv={hkv} nq={nq} nkv={nkv} d={d} causal={causal}", flush=True)
    q, k, v, do = W.dense_inputs(b, hq, hkv, nq, nkv, d, BF, seed=29 + d + hq)
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    assert lib.ffpa_bwd_fused_products(b, hq, hkv, nq, nkv, d)
    o, lse = lib.ffpa_fwd(qc, kc, vc, causal=causal)
    ws = torch.empty(lib.ffpa_bwd_workspace_bytes(b, hq, nq, nkv), dtype=torch.uint8, device="cuda")
    delta = torch.empty_like(lse)
    outs = []
    for stages in ((0, 4, 1, 2, 3), (0, 4, 5)):
        dq, dk, dv = torch.empty_like(qc), torch.empty_like(kc), torch.empty_like(vc)
        for stage in stages:
            lib.ffpa_bwd_stage(stage, qc, kc, vc, o, doc, lse, delta, dq, dk, dv, causal=causal, workspace=ws)
        outs.append((dq, dk, dv))
    torch.cuda.synchronize()
    for x, y in zip(*outs):
        assert torch.equal(x, y)
    g = lib.ffpa_bwd(qc, kc, vc, o, doc, lse, causal=causal, store_ds=True)
    for x, y in zip(outs[1], g):
        assert torch.equal(x, y)
