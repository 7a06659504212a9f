"""ffpa_decode_fwd_noalloc (the decode entry point that allocates nothing: its partial results go
to the library's fixed device scratch) against ffpa_decode_fwd with a caller workspace, through
the C ABI: two calls in a row, the second with smaller sizes, each bit-equal to the workspace
entry point (same kernels, same split) and within the parity tolerances of the oracle."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import ref
from tests.gpu_helpers import check_o_lse

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    import head_dim_attention_amd as F
    F.load_library()
    return F


def _call_noalloc(F, q, k, v, o, lse, causal, scale):
    b, hq, nq, d = q.shape
    hkv, nkv = k.shape[1], k.shape[2]
    P = F._binding._ptr
    dt = 0 if q.dtype == torch.bfloat16 else 1
    st = F.load_library().ffpa_decode_fwd_noalloc(P(q), P(k), P(v), P(o), P(lse), b, hq, hkv, nq, nkv, d, dt, scale,
                                                  int(causal), torch.cuda.current_stream().cuda_stream)
    assert st == F.FFPA_OK, F.ffpa_status_string(st)


# (B, Hq, Hkv, Nq, Nkv, D, dtype, causal): the first is the decode benchmark's shape, the second smaller
CALLS = [
    (1, 32, 8, 1, 65536, 512, torch.bfloat16, True),
    (2, 4, 2, 3, 1000, 320, torch.float16, False),
]


def test_noalloc_matches_workspace_entry_two_calls(lib):
    outs = []
    for i, (b, hq, hkv, nq, nkv, d, dt, causal) in enumerate(CALLS):
        print(f"noalloc call {i}: b{b} h{hq}x{hkv} q{nq} k{nkv} d{d} {dt}", flush=True)
        need = lib.ffpa_decode_workspace_bytes(b, hq, hkv, nq, nkv, d)
        assert 0 < need <= lib.NOALLOC_SCRATCH_BYTES
        q, k, v, _ = W.dense_inputs(b, hq, hkv, nq, nkv, d, dt, seed=900 + i, with_grad=False)
        qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
        scale = 1.0 / math.sqrt(d)
        o = torch.empty_like(qc)
        lse = torch.empty((b, hq, nq), dtype=torch.float32, device="cuda")
        _call_noalloc(lib, qc, kc, vc, o, lse, causal, scale)
        ref_o, ref_lse = lib.ffpa_decode_fwd(qc, kc, vc, causal=causal, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_lse), f"call {i} differs from ffpa_decode_fwd"
        o_r, lse_r = ref.attn_fwd(q, k, v, scale=np.float64(np.float32(scale)), causal=causal)
        check_o_lse(o, lse, o_r, lse_r, dt, f"noalloc call {i}")
        outs.append((o.clone(), lse.clone()))
    # A third call repeats the first after the smaller one left its contents in the scratch: the
    # result does not depend on what the scratch held before.
    b, hq, hkv, nq, nkv, d, dt, causal = CALLS[0]
    q, k, v, _ = W.dense_inputs(b, hq, hkv, nq, nkv, d, dt, seed=900, with_grad=False)
    o = torch.empty((b, hq, nq, d), dtype=dt, device="cuda")
    lse = torch.empty((b, hq, nq), dtype=torch.float32, device="cuda")
    _call_noalloc(lib, q.cuda(), k.cuda(), v.cuda(), o, lse, causal, 1.0 / math.sqrt(d))
    torch.cuda.synchronize()
    assert torch.equal(o, outs[0][0]) and torch.equal(lse, outs[0][1])


def test_noalloc_too_large_is_rejected(lib):
    """Sizes beyond the fixed scratch return FFPA_ERR_TOO_LARGE (ValueError in the binding) and
    launch nothing."""
    q = torch.zeros((64, 32, 7, 1024), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((64, 8, 4096, 1024), dtype=torch.bfloat16, device="cuda")
    assert lib.ffpa_decode_workspace_bytes(64, 32, 8, 7, 4096, 1024) > lib.NOALLOC_SCRATCH_BYTES
    with pytest.raises(ValueError, match="TOO_LARGE"):
        lib.ffpa_decode_fwd_noalloc(q, k, k, causal=True)
