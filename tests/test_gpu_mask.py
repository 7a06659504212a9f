"""GPU parity of attn_mask ("Triton Backend", "Feature support": boolean and additive masks that
broadcast in any dimension, with the bias gradient reduced back to the mask's shape) against the
float64 oracle.

Forward through ffpa_fwd_masked, backward through ffpa_bwd_masked (the P/dS workspace path: the
P/dS kernel for D <= 512, the recomputing dK kernel that stores P and dS for D > 512, then the
bias-gradient reduction). A boolean mask with the causal pattern must reproduce causal=True bit for
bit (the kept scores get + 0.0).
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import ref
from tests.gpu_helpers import GRAD_RTOL, check_grads, check_o_lse, rel_l2, to64

pytestmark = pytest.mark.gpu

BF, FP = torch.bfloat16, torch.float16


@pytest.fixture(scope="module")
def lib():
    import head_dim_attention_amd as F
    F.load_library()
    return F


def _bias(shape, dt, seed, kind):
    g = torch.Generator().manual_seed(seed)
    if kind == "bool":
        m = torch.rand(shape, generator=g) > 0.25
        return m
    return (torch.randn(shape, generator=g) * 2.0).to(dt)


def _ref_bias(m):
    if m.dtype == torch.bool:
        return ref.mask_to_bias(m)
    return m.double().numpy()


# (B, Hq, Hkv, Nq, Nkv, D, dtype, causal, mask shape, kind)
CASES = [
    (2, 4, 2, 100, 130, 512, BF, False, "BHQK", "add"),
    (1, 4, 4, 70, 90, 320, FP, True, "1HQK", "add"),
    (2, 2, 1, 65, 77, 512, BF, False, "B11K", "bool"),
    (1, 2, 2, 96, 96, 1024, BF, True, "QK", "add"),
    (2, 4, 2, 40, 50, 768, FP, False, "BHQ1", "add"),
    (1, 3, 3, 33, 200, 448, BF, True, "11QK", "bool"),
    (2, 2, 2, 64, 64, 512, BF, False, "B1QK", "add"),
    (1, 2, 1, 50, 70, 512, BF, True, "1H1K", "add"),
    (1, 2, 2, 70, 91, 384, BF, True, "BHQ1", "add"),
    (2, 2, 1, 45, 203, 512, FP, False, "BHQK", "bool"),
]


def _shape(spec, b, hq, nq, nkv):
    dims = {"B": b, "H": hq, "Q": nq, "K": nkv, "1": 1}
    return tuple(dims[c] for c in spec)


def _ids(c):
    return f"b{c[0]}h{c[1]}x{c[2]}q{c[3]}k{c[4]}d{c[5]}{'c' if c[7] else ''}-{c[8]}-{c[9]}"


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_mask_fwd_bwd(lib, case):
    b, hq, hkv, nq, nkv, d, dt, causal, spec, kind = case
    q, k, v, do = W.dense_inputs(b, hq, hkv, nq, nkv, d, dt, seed=500 + nq + d)
    m = _bias(_shape(spec, b, hq, nq, nkv), dt, 600 + nkv, "bool" if kind == "bool" else "add")
    scale = 1.0 / math.sqrt(d)
    s64 = np.float64(np.float32(scale))
    print(f"case {_ids(case)}", flush=True)
    qc, kc, vc, doc, mc = q.cuda(), k.cuda(), v.cuda(), do.cuda(), m.cuda()
    o, lse = lib.ffpa_fwd(qc, kc, vc, causal=causal, scale=scale, attn_mask=mc)
    g = lib.ffpa_bwd(qc, kc, vc, o, doc, lse, causal=causal, scale=scale, attn_mask=mc, mask_grad=kind == "add")
    torch.cuda.synchronize()
    rb = _ref_bias(m)
    o_ref, lse_ref = ref.attn_fwd(q, k, v, scale=s64, causal=causal, bias=rb)
    check_o_lse(o, lse, o_ref, lse_ref, dt, _ids(case))
    g_ref = ref.attn_bwd(q, k, v, do, scale=s64, causal=causal, bias=rb)
    check_grads(g[:3], g_ref[:3], _ids(case))
    if kind == "add":
        assert g[3].shape == m.shape and g[3].dtype == dt
        # Relative to the summed magnitudes |dS| (a bias broadcast over keys has an exactly zero
        # gradient, since rows of dS sum to zero, and the GPU sum is only small).
        full = ref.attn_bwd(q, k, v, do, scale=s64, causal=causal,
                            bias=np.broadcast_to(rb, (b, hq, nq, nkv)).copy())[3]
        scale_ref = np.linalg.norm(ref.reduce_to_shape(np.abs(full), m.shape))
        e = np.linalg.norm(to64(g[3]) - g_ref[3]) / scale_ref
        print(f"dmask error {e:.3e} (relative to the summed |dS|)")
        assert e <= GRAD_RTOL


@pytest.mark.parametrize("d", [512, 640])
def test_bool_mask_equals_causal(lib, d):
    b, hq, hkv, nq, nkv = 1, 4, 2, 90, 120
    q, k, v, do = W.dense_inputs(b, hq, hkv, nq, nkv, d, BF, seed=77)
    keep = torch.arange(nkv)[None, :] <= torch.arange(nq)[:, None] + (nkv - nq)
    qc, kc, vc, doc, mc = q.cuda(), k.cuda(), v.cuda(), do.cuda(), keep.cuda()
    o1, l1 = lib.ffpa_fwd(qc, kc, vc, causal=True, split=False)  # the masked forward has no key-range split
    o2, l2 = lib.ffpa_fwd(qc, kc, vc, causal=False, attn_mask=mc)
    g1 = lib.ffpa_bwd(qc, kc, vc, o1, doc, l1, causal=True)
    g2 = lib.ffpa_bwd(qc, kc, vc, o2, doc, l2, causal=False, attn_mask=mc)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for x, y in zip(g1, g2):
        assert torch.equal(x, y)


def test_fully_masked_rows(lib):
    """Rows whose mask drops every key: O = 0, LSE = -inf, zero dq, no contribution to dk/dv."""
    q, k, v, do = W.dense_inputs(1, 2, 2, 40, 64, 512, BF, seed=78)
    keep = torch.ones(40, 64, dtype=torch.bool)
    keep[5:9] = False
    qc, kc, vc, doc, mc = q.cuda(), k.cuda(), v.cuda(), do.cuda(), keep.cuda()
    o, lse = lib.ffpa_fwd(qc, kc, vc, attn_mask=mc)
    dq, dk, dv = lib.ffpa_bwd(qc, kc, vc, o, doc, lse, attn_mask=mc)
    torch.cuda.synchronize()
    assert torch.all(o[:, :, 5:9] == 0) and torch.all(lse[:, :, 5:9] == -math.inf)
    assert torch.all(dq[:, :, 5:9] == 0)
    do2 = doc.clone()
    do2[:, :, 5:9] = 50.0
    dq2, dk2, dv2 = lib.ffpa_bwd(qc, kc, vc, o, do2, lse, attn_mask=mc)
    torch.cuda.synchronize()
    assert torch.equal(dk, dk2) and torch.equal(dv, dv2)


def test_autograd_mask_grad(lib):
    q, k, v, do = W.dense_inputs(1, 4, 2, 64, 80, 512, BF, seed=79)
    bias = (torch.randn(1, 4, 64, 80, generator=torch.Generator().manual_seed(3)) * 1.5).to(BF)
    qc, kc, vc = (x.cuda().requires_grad_(True) for x in (q, k, v))
    bc = bias.cuda().requires_grad_(True)
    o = lib.ffpa_attn_func(qc, kc, vc, attn_mask=bc, is_causal=True)
    o.backward(do.cuda())
    torch.cuda.synchronize()
    s64 = np.float64(np.float32(1 / math.sqrt(512)))
    g_ref = ref.attn_bwd(q, k, v, do, scale=s64, causal=True, bias=bias.double().numpy())
    check_grads((qc.grad, kc.grad, vc.grad), g_ref[:3], "autograd mask")
    assert rel_l2(to64(bc.grad), g_ref[3]) <= GRAD_RTOL


@pytest.mark.slow
@pytest.mark.parametrize("d,kind", [(512, "add"), (448, "bool")])
def test_mask_full_size(lib, d, kind):
    """The masked forward and backward at the benchmark's sequence length (N = 8192: 256 key tiles
    per row through the two-group schedule, the mask fetched a tile ahead) with one [1, 1, N, N]
    mask shared by all heads; whole heads 0 and 3 against the oracle."""
    b, h, n = 1, 4, 8192
    q, k, v, do = W.dense_inputs(b, h, h, n, n, d, BF, seed=900 + d)
    m = _bias((1, 1, n, n), BF, 901, kind)
    scale = 1.0 / math.sqrt(d)
    s64 = np.float64(np.float32(scale))
    print(f"full-size masked d{d} {kind}: running on the GPU", flush=True)
    qc, kc, vc, doc, mc = q.cuda(), k.cuda(), v.cuda(), do.cuda(), m.cuda()
    o, lse = lib.ffpa_fwd(qc, kc, vc, scale=scale, attn_mask=mc)
    dq, dk, dv = lib.ffpa_bwd(qc, kc, vc, o, doc, lse, scale=scale, attn_mask=mc)[:3]
    torch.cuda.synchronize()
    rb = _ref_bias(m)
    for hd in (0, 3):
        sl = slice(hd, hd + 1)
        tag = f"full-size masked d{d} {kind} head {hd}"
        o_ref, lse_ref = ref.attn_fwd(q[:, sl], k[:, sl], v[:, sl], scale=s64, causal=False, bias=rb)
        check_o_lse(o[:, sl], lse[:, sl], o_ref, lse_ref, BF, tag)
        g_ref = ref.attn_bwd(q[:, sl], k[:, sl], v[:, sl], do[:, sl], scale=s64, causal=False, bias=rb)
        check_grads((dq[:, sl], dk[:, sl], dv[:, sl]), g_ref[:3], tag)


@pytest.mark.parametrize("d", [512, 768])
def test_mask_dlse(lib, d):
    """The LSE's gradient through the masked backward (and into the bias gradient)."""
    q, k, v, do = W.dense_inputs(1, 4, 2, 70, 90, d, BF, seed=620 + d)
    m = _bias((1, 4, 70, 90), BF, 621, "add")
    g = torch.randn((1, 4, 70), generator=torch.Generator().manual_seed(622))
    scale = 1.0 / math.sqrt(d)
    qc, kc, vc, doc, mc = q.cuda(), k.cuda(), v.cuda(), do.cuda(), m.cuda()
    o, lse = lib.ffpa_fwd(qc, kc, vc, causal=True, scale=scale, attn_mask=mc)
    dq, dk, dv, dm = lib.ffpa_bwd(qc, kc, vc, o, doc, lse, causal=True, scale=scale, attn_mask=mc, mask_grad=True,
                                  dlse=g.cuda())
    torch.cuda.synchronize()
    r = ref.attn_bwd(q, k, v, do, scale=np.float64(np.float32(scale)), causal=True, bias=_ref_bias(m),
                     dlse=g.double().numpy())
    check_grads((dq, dk, dv), r[:3], f"mask dlse d{d}")
    assert rel_l2(to64(dm), r[3]) <= GRAD_RTOL
