"""GPU tests of the strided (zero-copy) forward: [B, N, H, D] tensors and fused-QKV slices are
read in place ("Backends Overview", backend table notes: NHD zero-copy consumes [B, N, H, D] or
fused-QKV chunk views without materializing a packed copy).

The strided path runs the same kernels with different addressing, so its results must equal the
packed path's bit for bit; one case per layout is also checked against the oracle.
"""
import functools
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import ref
from tests.gpu_helpers import check_o_lse

pytestmark = pytest.mark.gpu

BF, FP = torch.bfloat16, torch.float16


@pytest.fixture(scope="module")
def lib():
    import head_dim_attention_amd as F
    F.load_library()
    return F


def _nhd(x):
    """A [B, N, H, D] copy of a [B, H, N, D] tensor, returned as its [B, H, N, D] view."""
    return x.transpose(1, 2).contiguous().transpose(1, 2)


# (B, Hq, Hkv, Nq, Nkv, D, dtype, causal)
CASES = [
    (2, 4, 2, 100, 130, 512, BF, True),
    (1, 2, 2, 65, 65, 320, FP, False),
    (1, 4, 1, 70, 90, 1024, BF, True),
    (1, 3, 3, 1, 700, 768, FP, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"b{c[0]}h{c[1]}x{c[2]}q{c[3]}k{c[4]}d{c[5]}")
def test_nhd_views_equal_packed(lib, case):
    b, hq, hkv, nq, nkv, d, dt, causal = case
    q, k, v, _ = W.dense_inputs(b, hq, hkv, nq, nkv, d, dt, seed=31 + d, with_grad=False)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    qn, kn, vn = _nhd(qc), _nhd(kc), _nhd(vc)
    assert not (qn.is_contiguous() and kn.is_contiguous()), "at least one input is a strided view"
    # (strided views take no key-range split, so the packed call is made without one)
    for fwd in (functools.partial(lib.ffpa_fwd, split=False), lib.ffpa_decode_fwd):
        o1, l1 = fwd(qc, kc, vc, causal=causal)
        o2, l2 = fwd(qn, kn, vn, causal=causal)
        torch.cuda.synchronize()
        assert o2.stride() == qn.stride(), "O keeps the [B, N, H, D] layout of q"
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
    scale = 1.0 / math.sqrt(d)
    o_ref, lse_ref = ref.attn_fwd(q, k, v, scale=np.float64(np.float32(scale)), causal=causal)
    o2, l2 = lib.ffpa_fwd(qn, kn, vn, causal=causal)
    torch.cuda.synchronize()
    check_o_lse(o2, l2, o_ref, lse_ref, dt, "nhd")


@pytest.mark.parametrize("nq", [96, 3])
def test_fused_qkv_slices(lib, nq):
    """q, k, v as slices of one [B, N, 3, H, D] tensor (N = Nq = Nkv for the packed projection)."""
    b, h, n, d = 2, 4, nq, 512
    g = torch.Generator().manual_seed(41 + nq)
    qkv = torch.randn(b, n, 3, h, d, generator=g).to(BF).cuda()
    q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))
    assert q.stride() == (n * 3 * h * d, d, 3 * h * d, 1)
    # (strided views take no key-range split, so the packed call is made without one)
    for fwd in (functools.partial(lib.ffpa_fwd, split=False), lib.ffpa_decode_fwd):
        o1, l1 = fwd(q.contiguous(), k.contiguous(), v.contiguous(), causal=True)
        o2, l2 = fwd(q, k, v, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o_ref, lse_ref = ref.attn_fwd(q.cpu(), k.cpu(), v.cpu(), scale=np.float64(np.float32(1 / math.sqrt(d))),
                                  causal=True)
    check_o_lse(o2, l2, o_ref, lse_ref, BF, "fused qkv")
