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
    ("gqa_causal_d1024_n8192", (3,)),
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
    # the longest and the shortest sequence, one head each
    for s in (int(np.argmax(lens)), int(np.argmin(lens))):
        a, b = int(cu_q[s]), int(cu_q[s + 1])
        h = (7 * s + 3) % w.hq
        dq_r, dk_r, dv_r, o_r, lse_r = ref.group_backward(q[a:b, h:h + 1].transpose(0, 1).double().numpy(),
                                                          k[a:b, h].double().numpy(), v[a:b, h].double().numpy(),
                                                          do[a:b, h:h + 1].transpose(0, 1).double().numpy(), s64,
                                                          True)[:5]
        _check_group(f"varlen seq {s} (L={b - a}) head {h}", w.torch_dtype, to64(o[a:b, h])[None],
                     lse[h:h + 1, a:b].double().cpu().numpy(), to64(dq[a:b, h])[None], to64(dk[a:b, h]),
                     to64(dv[a:b, h]), o_r, lse_r, dq_r, dk_r, dv_r)
