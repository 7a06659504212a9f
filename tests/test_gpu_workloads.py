"""Full-size workloads, run exactly as the benchmark launches them, checked against the oracle on
whole sampled heads / KV groups / sequences (the oracle recomputes those in full)."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import ref
from tests.gpu_helpers import GRAD_RTOL, LSE_TOL, O_TOL, rel_l2, to64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def lib():
    import head_dim_attention_amd as F
    F.load_library()
    return F


def _check_group(tag, dt, o, lse, dq, dk, dv, o_r, lse_r, dq_r, dk_r, dv_r):
    fin = np.isfinite(lse_r)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_r)), f"{tag}: -inf LSE positions"
    eo = float(np.max(np.abs(o - o_r)))
    el = float(np.max(np.abs(lse[fin] - lse_r[fin]))) if fin.any() else 0.0
    eg = [rel_l2(x, r) for x, r in ((dq, dq_r), (dk, dk_r), (dv, dv_r))]
    print(f"{tag}: O max-abs {eo:.2e} (rel-L2 {rel_l2(o, o_r):.2e}), LSE {el:.2e}, "
          f"dQ/dK/dV rel-L2 {eg[0]:.2e}/{eg[1]:.2e}/{eg[2]:.2e}", flush=True)
    assert eo <= O_TOL[dt] and el <= LSE_TOL and max(eg) <= GRAD_RTOL, tag


@pytest.mark.parametrize("name,groups", [
    ("causal_d512_n4096", (0, 5)),
    ("dense_d512_n8192", (0, 31)),
    ("gqa_causal_d1024_n8192", (0, 3, 7)),
])
def test_dense_workload(lib, name, groups):
    w = W.get(name)
    q, k, v, do = W.workload_inputs(w, seed=2024)
    scale = 1.0 / math.sqrt(w.d)
    print(f"workload {name}: running on the GPU", flush=True)
    qc, kc, vc, doc = (x.cuda() for x in (q, k, v, do))
    o, lse = lib.ffpa_fwd(qc, kc, vc, causal=w.causal, scale=scale)
    dq, dk, dv = lib.ffpa_bwd(qc, kc, vc, o, doc, lse, causal=w.causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
    g = w.hq // w.hkv
    s64 = float(np.float32(scale))
    for kv in groups:
        hs = slice(kv * g, (kv + 1) * g)
        dq_r, dk_r, dv_r, o_r, lse_r = ref.group_backward(q[0, hs].double().numpy(), k[0, kv].double().numpy(),
                                                          v[0, kv].double().numpy(), do[0, hs].double().numpy(),
                                                          s64, w.causal)[:5]
        _check_group(f"{name} kv-group {kv}", w.torch_dtype, to64(o[0, hs]), lse[0, hs].double().cpu().numpy(),
                     to64(dq[0, hs]), to64(dk[0, kv]), to64(dv[0, kv]), o_r, lse_r, dq_r, dk_r, dv_r)


def test_varlen_workload(lib):
    w = W.get("varlen_causal_d512")
    lens = W.varlen_lengths(w.batch, 2024)
    q, k, v, do, cu_q, cu_k = W.workload_inputs(w, seed=2024)
    print(f"varlen lengths {lens}, T = {sum(lens)}", flush=True)
    scale = 1.0 / math.sqrt(w.d)
    qc, kc, vc, doc, cq = q.cuda(), k.cuda(), v.cuda(), do.cuda(), cu_q.cuda()
    o, lse = lib.ffpa_varlen_fwd(qc, kc, vc, cq, None, max(lens), max(lens), causal=True, scale=scale)
    dq, dk, dv = lib.ffpa_varlen_bwd(qc, kc, vc, o, doc, lse, cq, None, max(lens), max(lens), causal=True, scale=scale)
    torch.cuda.synchronize()
    assert lse.shape == (w.hq, sum(lens)) and lse.dtype == torch.float32
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    s64 = float(np.float32(scale))
    # every sequence, on its first and last head (heads 0 and 31 sit on different XCDs)
    for s in range(w.batch):
        a, b = int(cu_q[s]), int(cu_q[s + 1])
        for h in (0, w.hq - 1):
            dq_r, dk_r, dv_r, o_r, lse_r = ref.group_backward(q[a:b, h:h + 1].transpose(0, 1).double().numpy(),
                                                              k[a:b, h].double().numpy(), v[a:b, h].double().numpy(),
                                                              do[a:b, h:h + 1].transpose(0, 1).double().numpy(), s64,
                                                              True)[:5]
            _check_group(f"varlen seq {s} (L={b - a}) head {h}", w.torch_dtype, to64(o[a:b, h])[None],
                         lse[h:h + 1, a:b].double().cpu().numpy(), to64(dq[a:b, h])[None], to64(dk[a:b, h]),
                         to64(dv[a:b, h]), o_r, lse_r, dq_r, dk_r, dv_r)


@pytest.mark.parametrize("name", ["dense_d512_n8192", "gqa_causal_d1024_n8192", "causal_d512_n4096"])
def test_dense_workload_every_group_equal(lib, name):
    """Whole-tensor check of the head and XCD mapping at full size: with every KV group given the
    same inputs, every group's O, LSE, dQ, dK and dV must be bit-identical (the kernels are
    deterministic and a group's arithmetic does not depend on where it runs)."""
    w = W.get(name)
    q, k, v, do = W.workload_inputs(w, seed=2025)
    g = w.hq // w.hkv
    rep = lambda x, n: x[:, :n].repeat(1, x.shape[1] // n, 1, 1).contiguous()
    q, do = rep(q, g), rep(do, g)
    k, v = rep(k, 1), rep(v, 1)
    print(f"workload {name}: identical KV groups", flush=True)
    qc, kc, vc, doc = (x.cuda() for x in (q, k, v, do))
    o, lse = lib.ffpa_fwd(qc, kc, vc, causal=w.causal)
    dq, dk, dv = lib.ffpa_bwd(qc, kc, vc, o, doc, lse, causal=w.causal)
    torch.cuda.synchronize()
    for grp in range(1, w.hkv):
        hs, h0 = slice(grp * g, (grp + 1) * g), slice(0, g)
        assert torch.equal(o[:, hs], o[:, h0]) and torch.equal(lse[:, hs], lse[:, h0]), f"group {grp} forward"
        assert torch.equal(dq[:, hs], dq[:, h0]), f"group {grp} dq"
        assert torch.equal(dk[:, grp], dk[:, 0]) and torch.equal(dv[:, grp], dv[:, 0]), f"group {grp} dk/dv"


def test_small_causal_workload_run_to_run(lib):
    """The small causal grid takes the key-range split forward and the one-launch products (their
    item orders balance the load at run time, but every output element is still formed by one
    workgroup in a fixed order): two runs give bit-identical O, LSE, dQ, dK and dV."""
    w = W.get("causal_d512_n4096")
    q, k, v, do = W.workload_inputs(w, seed=2026)
    print("workload causal_d512_n4096: two runs", flush=True)
    qc, kc, vc, doc = (x.cuda() for x in (q, k, v, do))
    runs = []
    for _ in range(2):
        o, lse = lib.ffpa_fwd(qc, kc, vc, causal=True)
        runs.append((o, lse, *lib.ffpa_bwd(qc, kc, vc, o, doc, lse, causal=True)))
    torch.cuda.synchronize()
    for a, b in zip(*runs):
        assert torch.equal(a, b)


def test_varlen_workload_every_head_equal(lib):
    """The same check for the packed workload: all 32 heads given the same inputs must give
    bit-identical results on every head."""
    w = W.get("varlen_causal_d512")
    lens = W.varlen_lengths(w.batch, 2025)
    q, k, v, do, cu_q, _ = W.workload_inputs(w, seed=2025)
    q, k, v, do = (x[:, :1].repeat(1, x.shape[1], 1).contiguous() for x in (q, k, v, do))
    qc, kc, vc, doc, cq = q.cuda(), k.cuda(), v.cuda(), do.cuda(), cu_q.cuda()
    print(f"varlen identical heads, lengths {lens}", flush=True)
    o, lse = lib.ffpa_varlen_fwd(qc, kc, vc, cq, None, max(lens), max(lens), causal=True)
    dq, dk, dv = lib.ffpa_varlen_bwd(qc, kc, vc, o, doc, lse, cq, None, max(lens), max(lens), causal=True)
    torch.cuda.synchronize()
    for h in range(1, w.hq):
        for x in (o, dq, dk, dv):
            assert torch.equal(x[:, h], x[:, 0]), f"head {h}"
        assert torch.equal(lse[h], lse[0]), f"head {h} lse"
