"""GPU tests of the FP8 forward (ffpa_fwd_fp8) against the oracle's FP8 emulation.

The quantized tensors must match the emulation exactly: per-head amax, K8 and V8^T bytes (the GPU
converts with v_cvt_pk_fp8_f32, the oracle with PyTorch's float8_e4m3fn cast, from the same fp32
products). O then differs from the emulation only through the e4m3 rounding of P, which the GPU
takes against a running row max and the emulation against the final one: every element of O stays
within the bound fp8_o_bound derives from that (computed from the oracle's P, l and V8), LSE
(unquantized) within 1e-3, and O within 0.1 relative L2 of exact attention (a sanity check of the
whole quantized path: typical values are 3-5e-2).
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import ref
from tests.gpu_helpers import rel_l2, to64

pytestmark = pytest.mark.gpu

BF, FP = torch.bfloat16, torch.float16


@pytest.fixture(scope="module")
def lib():
    import head_dim_attention_amd as F
    F.load_library()
    return F


# (B, Hq, Hkv, Nq, Nkv, D, dtype, causal)
CASES = [
    (1, 2, 2, 128, 128, 512, BF, False),
    (2, 4, 2, 100, 150, 320, FP, True),
    (1, 4, 1, 70, 333, 448, BF, False),
    (1, 2, 2, 1, 200, 512, FP, True),
    (1, 3, 3, 257, 200, 384, BF, True),
    (1, 2, 1, 64, 40, 512, BF, False),     # one key tile
    (1, 2, 2, 100, 30, 448, FP, True),     # causal Nq > Nkv: rows without a legal key
    (1, 4, 2, 300, 1000, 512, BF, True),   # many tiles, ragged tails
    # D > 512: S over two head-dim halves, O in quarters
    (1, 2, 2, 128, 128, 768, BF, False),
    (1, 4, 2, 100, 150, 1024, FP, True),
    (1, 2, 1, 70, 333, 544, BF, False),    # head dim padded to 640
    (1, 2, 2, 1, 200, 768, FP, True),
    (1, 3, 3, 65, 64, 896, BF, True),      # one key tile, one query past a 64-query tile
    (1, 2, 2, 100, 30, 640, FP, True),     # causal Nq > Nkv: rows without a legal key
    (1, 4, 2, 300, 700, 1024, BF, True),   # many tiles, ragged tails
]


def _ids(c):
    return f"b{c[0]}h{c[1]}x{c[2]}q{c[3]}k{c[4]}d{c[5]}{'bf16' if c[6] == BF else 'fp16'}{'c' if c[7] else ''}"


def fp8_o_bound(parts, o_r, group, dt):
    """Elementwise bound on |O_gpu - O_emulation|. Both sides round every P_ij * 448 (times
    exp(m_final - m_running) >= 1 on the GPU) to e4m3, so each is within max(2^-4 P_ij, 2^-10 / 448)
    of P_ij (half a step: relative for normals, absolute below 2^-6) and the two differ by at most
    2^-3 P_ij + 2^-9 / 448 per legal key; O moves by that times |V8_jd| / l_i. On top: the output's
    rounding (half an ulp of bf16 / fp16) and a 1e-4 relative slack for the fp32 scores, exp2 and l."""
    p, l_, v = parts["p"], parts["l"], parts["v"]
    vabs = np.repeat(np.abs(v), group, axis=1)                      # [B, Hq, Nkv, D]
    dp = 2.0 ** -3 * p + (p > 0) * (2.0 ** -9 / 448.0)
    safe = np.where(l_ > 0, l_, 1.0)[..., None]
    half_ulp = 2.0 ** -9 if dt == BF else 2.0 ** -12
    return (dp @ vabs) / safe + (half_ulp + 1e-4) * np.abs(o_r) + 1e-6


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_fp8_forward(lib, case):
    from head_dim_attention_amd import _binding as B
    b, hq, hkv, nq, nkv, d, dt, causal = case
    q, k, v, _ = W.dense_inputs(b, hq, hkv, nq, nkv, d, dt, seed=900 + d + nq, with_grad=False)
    scale = 1.0 / math.sqrt(d)
    print(f"case {_ids(case)}", flush=True)
    nws = B.ffpa_fwd_fp8_workspace_bytes(b, hq, hkv, nq, nkv, d)
    ws = torch.zeros(nws, dtype=torch.uint8, device="cuda")
    o, lse = lib.ffpa_fwd_fp8(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, workspace=ws)
    torch.cuda.synchronize()
    # quantized operands: exact
    aq, ak, av, k8, v8t = B.fp8_workspace_views(ws, b, hq, hkv, nkv, d)
    k8r, akr = ref.fp8_quantize(k)
    v8r, avr = ref.fp8_quantize(v)
    _, aqr = ref.fp8_quantize(q)
    assert np.array_equal(aq.cpu().double().numpy(), aqr) and np.array_equal(ak.cpu().double().numpy(), akr)
    assert np.array_equal(av.cpu().double().numpy(), avr)
    as_val = lambda t: t.cpu().view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(as_val(k8), k8r)
    np_ = v8t.shape[-1]
    assert np.array_equal(as_val(v8t)[..., :nkv], np.swapaxes(v8r, 2, 3))
    assert np.all(v8t[..., nkv:].cpu().numpy() == 0)
    # results
    s64 = float(np.float32(scale))
    o_r, lse_r, parts = ref.attn_fwd_fp8(q, k, v, scale=s64, causal=causal, parts=True)
    og, lg = to64(o), lse.double().cpu().numpy()
    fin = np.isfinite(lse_r)
    assert np.array_equal(np.isneginf(lg), np.isneginf(lse_r))
    err_l = float(np.max(np.abs(lg[fin] - lse_r[fin]))) if fin.any() else 0.0
    bound = fp8_o_bound(parts, o_r, hq // hkv, dt)
    ratio = float(np.max(np.abs(og - o_r) / bound))
    o_ex, _ = ref.attn_fwd(q, k, v, scale=s64, causal=causal)
    e_ex = rel_l2(og, o_ex)
    e_em = rel_l2(og, o_r)
    print(f"O |err| / bound max {ratio:.3f}, rel-L2 vs emulation {e_em:.3e}, vs exact {e_ex:.3e}; "
          f"LSE {err_l:.3e}")
    assert ratio <= 1.0 and err_l <= 1e-3 and e_ex <= 0.1


def test_fp8_full_size_sampled_head(lib):
    """The measured shape (B=1, H=32, N=8192, D=512, bf16, as bench.py times it): every head's amax
    exactly, and one whole head's O against the emulation within the same bound, LSE within 1e-3."""
    from head_dim_attention_amd import _binding as B
    w = W.get("dense_d512_n8192")
    q, k, v, _ = W.workload_inputs(w, seed=2024)
    b, hq, nq, d = q.shape
    hkv, nkv = k.shape[1], k.shape[2]
    nws = B.ffpa_fwd_fp8_workspace_bytes(b, hq, hkv, nq, nkv, d)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(d)
    print("fp8 full size", flush=True)
    o, lse = lib.ffpa_fwd_fp8(q.cuda(), k.cuda(), v.cuda(), causal=False, scale=scale, workspace=ws)
    torch.cuda.synchronize()
    aq, ak, av, _, _ = B.fp8_workspace_views(ws, b, hq, hkv, nkv, d)
    for x, a in ((q, aq), (k, ak), (v, av)):
        assert np.array_equal(a.cpu().double().numpy(), ref.fp8_quantize(x)[1])
    h = 7
    qs, ks, vs = q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1]
    o_r, lse_r, parts = ref.attn_fwd_fp8(qs, ks, vs, scale=float(np.float32(scale)), causal=False, parts=True)
    og = to64(o[:, h:h + 1])
    ratio = float(np.max(np.abs(og - o_r) / fp8_o_bound(parts, o_r, 1, BF)))
    err_l = float(np.max(np.abs(lse[:, h:h + 1].double().cpu().numpy() - lse_r)))
    print(f"full size head {h}: O |err| / bound max {ratio:.3f}, LSE {err_l:.3e}")
    assert ratio <= 1.0 and err_l <= 1e-3


def test_fp8_full_size_d1024_sampled_heads(lib):
    """The grouped causal D = 1024 shape (B=1, Hq=32, Hkv=8, N=8192, fp16): every head's amax
    exactly, and two whole heads (different KV groups) against the emulation within the bound,
    LSE within 1e-3."""
    from head_dim_attention_amd import _binding as B
    w = W.get("gqa_causal_d1024_n8192")
    q, k, v, _ = W.workload_inputs(w, seed=2025)
    b, hq, nq, d = q.shape
    hkv, nkv = k.shape[1], k.shape[2]
    g = hq // hkv
    nws = B.ffpa_fwd_fp8_workspace_bytes(b, hq, hkv, nq, nkv, d)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    scale = 1.0 / math.sqrt(d)
    print("fp8 full size d1024", flush=True)
    o, lse = lib.ffpa_fwd_fp8(q.cuda(), k.cuda(), v.cuda(), causal=True, scale=scale, workspace=ws)
    torch.cuda.synchronize()
    aq, ak, av, _, _ = B.fp8_workspace_views(ws, b, hq, hkv, nkv, d)
    for x, a in ((q, aq), (k, ak), (v, av)):
        assert np.array_equal(a.cpu().double().numpy(), ref.fp8_quantize(x)[1])
    for h in (3, 29):
        qs, ks, vs = q[:, h:h + 1], k[:, h // g:h // g + 1], v[:, h // g:h // g + 1]
        o_r, lse_r, parts = ref.attn_fwd_fp8(qs, ks, vs, scale=float(np.float32(scale)), causal=True, parts=True)
        og = to64(o[:, h:h + 1])
        ratio = float(np.max(np.abs(og - o_r) / fp8_o_bound(parts, o_r, 1, w.torch_dtype)))
        err_l = float(np.max(np.abs(lse[:, h:h + 1].double().cpu().numpy() - lse_r)))
        print(f"full size d1024 head {h}: O |err| / bound max {ratio:.3f}, LSE {err_l:.3e}", flush=True)
        assert ratio <= 1.0 and err_l <= 1e-3
