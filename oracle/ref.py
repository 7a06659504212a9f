"""CPU float64 oracle for large-head-dim scaled-dot-product attention (forward + backward).

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports this module: only the tests, the
``smoke()`` check and the benchmark's ``cpu_baseline`` leg call it. It shares no code, tables or
helpers with the HIP kernels.

What is computed, and where the ffpa-attn user guide fixes it:

* The method keeps the contract of PyTorch's scaled_dot_product_attention ("Backends Overview",
  section "Automatic SDPA fallback": the entry point is SDPA-aligned). So per query head h, with
  S = scale * Q_h K_g^T, the output is O = softmax(S) V_g and the log-sum-exp is the natural-log
  LSE_i = log sum_j exp(S_ij) over the legal keys j.
* Causal masking is tail-aligned, i.e. bottom-right: key j is legal for query i iff
  j <= i + (Nkv - Nq) ("Triton Backend", section "Feature support", Shapes; "CuTe-DSL Backend",
  section "Hard constraints", SM100 dedicated range; section "Varlen (packed THD) API": applied per
  sequence).
* GQA/MQA is a zero-stride broadcast of the KV heads: query head h reads KV head h // (Hq/Hkv), and
  the gradient of a broadcast is the sum over the query heads that share it ("CuTe-DSL Backend",
  "Hard constraints").
* Rows with no legal key produce O = 0, LSE = -inf and exactly zero gradient ("CuTe-DSL Backend",
  "Hard constraints").
* LSE is float32 [H_q, T_q] for packed varlen input ("CuTe-DSL Backend", "Varlen (packed THD)
  API"); dense LSE is [B, H_q, N_q] (a reading: the pages state only the varlen shape).
* The backward has the four stages preprocess, dV, dK, dQ ("CuTe-DSL Backend", "Blackwell status"):
  Delta = rowsum(dO * O), dV = P^T dO, dP = dO V^T, dS = P * (dP - Delta), dK = scale dS^T Q,
  dQ = scale dS K. These are the exact gradients of L = sum(dO * O); the oracle writes the
  definition out and leaves the split into kernels to the GPU side.
* The LSE is an output the caller may use ("CuTe-DSL Backend", "Varlen (packed THD) API":
  return_lse=True hands it back), so it can carry a gradient dLSE of its own. With
  L = sum(dO * O) + sum(dLSE * LSE), the chain rule adds, for every legal entry, dLSE_i times
  d LSE_i / d S_ij = P_ij to the gradient with respect to the scores: dS = P * (dP - Delta) +
  P * dLSE. Empty rows have a constant LSE (-inf), so their dLSE contributes nothing.
* attn_mask ("Triton Backend", "Feature support"): an additive bias broadcastable to
  [B, Hq, Nq, Nkv] is added to the scaled scores (SDPA semantics); a boolean mask is the bias
  0 where it keeps a key and -inf where it drops one. An entry whose score is -inf is not a legal
  key, so a row with no finite score is an empty row (O = 0, LSE = -inf, zero gradient, as for
  the causal mask). The bias gradient is dS (the gradient of L with respect to the scores)
  summed over the dimensions the bias broadcasts.

Everything is the plain definition in float64 NumPy: S is materialised per (batch, KV group).
Queries are independent rows, so they are processed in row blocks to bound memory; that changes
nothing but the order in which the dK/dV sums over query rows are added.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "legal_mask", "softmax_rows", "group_forward", "group_backward", "mask_to_bias", "reduce_to_shape",
    "attn_fwd", "attn_bwd", "varlen_fwd", "varlen_bwd", "preprocess_delta", "fwd_rows",
    "e4m3", "fp8_quantize", "attn_fwd_fp8",
]

# Query rows per block when S is materialised: 2048 rows x 8192 keys x 8 B = 128 MiB per array.
_ROW_BLOCK = 2048


def legal_mask(rows: np.ndarray, nq: int, nkv: int, causal: bool) -> np.ndarray:
    """Boolean [len(rows), nkv]: key j is legal for query i (tail-aligned causal when ``causal``)."""
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(nkv, dtype=np.int64)[None, :]
    if not causal:
        return np.ones((rows.shape[0], nkv), dtype=bool)
    return j <= rows[:, None] + (nkv - nq)


def softmax_rows(s: np.ndarray, legal: np.ndarray):
    """Row softmax over the legal entries of ``s``; returns (P, LSE).

    Rows without a legal entry get P = 0 and LSE = -inf.
    """
    has = legal.any(axis=1)
    s_masked = np.where(legal, s, -np.inf)
    m = np.where(has, np.max(np.where(legal, s, -np.inf), axis=1, initial=-np.inf), 0.0)
    e = np.where(legal, np.exp(s_masked - m[:, None]), 0.0)
    z = e.sum(axis=1)
    safe_z = np.where(has, z, 1.0)
    p = np.where(has[:, None], e / safe_z[:, None], 0.0)
    lse = np.where(has, m + np.log(safe_z), -np.inf)
    return p, lse


def _scores(q_b, kg, scale, rows, nq, nkv, causal, bias_b):
    """Scaled scores of a row block (plus the bias rows, if any) and their legal entries."""
    s = scale * (q_b @ kg.T)
    legal = legal_mask(rows, nq, nkv, causal)
    if bias_b is not None:
        s = s + bias_b
        legal = legal & (s > -np.inf)
    return s, legal


def group_forward(qg: np.ndarray, kg: np.ndarray, vg: np.ndarray, scale: float, causal: bool, bias_g=None):
    """One KV group. qg [G, Nq, D]; kg, vg [Nkv, D]; bias_g None or [G, Nq, Nkv].
    Returns O [G, Nq, D], LSE [G, Nq]."""
    g_, nq, d = qg.shape
    nkv = kg.shape[0]
    o = np.zeros((g_, nq, d), dtype=np.float64)
    lse = np.full((g_, nq), -np.inf, dtype=np.float64)
    if nq == 0 or nkv == 0:
        return o, lse
    for h in range(g_):
        for r0 in range(0, nq, _ROW_BLOCK):
            rows = np.arange(r0, min(nq, r0 + _ROW_BLOCK))
            s, legal = _scores(qg[h, rows], kg, scale, rows, nq, nkv, causal,
                               None if bias_g is None else bias_g[h, rows])
            p, l_ = softmax_rows(s, legal)
            o[h, rows] = p @ vg
            lse[h, rows] = l_
    return o, lse


def group_backward(qg, kg, vg, dog, scale: float, causal: bool, bias_g=None, dlse_g=None):
    """Gradients of L = sum(dO * O) (+ sum(dLSE * LSE) with dlse_g) for one KV group.

    qg, dog [G, Nq, D]; kg, vg [Nkv, D]; bias_g None or [G, Nq, Nkv]; dlse_g None or [G, Nq], the
    gradient of the loss with respect to the LSE. Returns dQ [G, Nq, D],
    dK [Nkv, D], dV [Nkv, D], the forward's O [G, Nq, D], LSE [G, Nq] and Delta [G, Nq], and dS
    [G, Nq, Nkv] (the gradient with respect to the scores; None without a bias), all float64.
    """
    g_, nq, d = qg.shape
    nkv = kg.shape[0]
    dq = np.zeros_like(qg, dtype=np.float64)
    dk = np.zeros((nkv, d), dtype=np.float64)
    dv = np.zeros((nkv, d), dtype=np.float64)
    o = np.zeros((g_, nq, d), dtype=np.float64)
    lse = np.full((g_, nq), -np.inf, dtype=np.float64)
    delta = np.zeros((g_, nq), dtype=np.float64)
    ds_all = None if bias_g is None else np.zeros((g_, nq, nkv), dtype=np.float64)
    if nq == 0 or nkv == 0:
        return dq, dk, dv, o, lse, delta, ds_all
    for h in range(g_):
        for r0 in range(0, nq, _ROW_BLOCK):
            rows = np.arange(r0, min(nq, r0 + _ROW_BLOCK))
            q_b = qg[h, rows]
            do_b = dog[h, rows]
            s, legal = _scores(q_b, kg, scale, rows, nq, nkv, causal,
                               None if bias_g is None else bias_g[h, rows])
            p, l_ = softmax_rows(s, legal)
            o_b = p @ vg
            # Stage 1 (preprocess): Delta_i = sum_d dO_id * O_id.
            dlt = np.sum(do_b * o_b, axis=1)
            # Stage 2 (dV): dV += P^T dO.
            dv += p.T @ do_b
            # dP = dO V^T ; dS = P * (dP - Delta).
            dp = do_b @ vg.T
            ds = p * (dp - dlt[:, None])
            if dlse_g is not None:
                # The LSE's own gradient: d LSE_i / d S_ij = P_ij on the legal entries.
                ds = ds + p * dlse_g[h, rows][:, None]
            # Stage 3 (dK): dK += scale dS^T Q.
            dk += scale * (ds.T @ q_b)
            # Stage 4 (dQ): dQ = scale dS K.
            dq[h, rows] = scale * (ds @ kg)
            o[h, rows] = o_b
            lse[h, rows] = l_
            delta[h, rows] = dlt
            if ds_all is not None:
                ds_all[h, rows] = ds
    return dq, dk, dv, o, lse, delta, ds_all


def _threads() -> int:
    n = os.environ.get("FFPA_ORACLE_THREADS")
    if n:
        return max(1, int(n))
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _map_groups(fn, items):
    workers = min(_threads(), max(1, len(items)))
    if workers == 1:
        return [fn(it) for it in items]
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))


def mask_to_bias(mask) -> np.ndarray:
    """A boolean attn_mask (True keeps the key) as the equivalent additive bias (0 / -inf)."""
    m = np.asarray(mask.detach().cpu().numpy() if hasattr(mask, "detach") else mask, dtype=bool)
    return np.where(m, 0.0, -np.inf)


def _full_bias(bias, b, hq, nq, nkv):
    return None if bias is None else np.broadcast_to(_f64(bias), (b, hq, nq, nkv))


def reduce_to_shape(full: np.ndarray, shape) -> np.ndarray:
    """Sum a [B, Hq, Nq, Nkv] array over the dimensions a bias of ``shape`` broadcasts."""
    shape = tuple(shape)
    lead = full.ndim - len(shape)
    out = full.sum(axis=tuple(range(lead))) if lead > 0 else full
    axes = tuple(i for i, n in enumerate(shape) if n == 1 and out.shape[i] != 1)
    return out.sum(axis=axes, keepdims=True) if axes else out


def attn_fwd(q, k, v, *, scale: float, causal: bool, bias=None):
    """Dense forward. q [B,Hq,Nq,D]; k, v [B,Hkv,Nkv,D]; bias None or broadcastable to
    [B,Hq,Nq,Nkv] (use mask_to_bias for a boolean mask). Returns (O [B,Hq,Nq,D], LSE [B,Hq,Nq])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    b, hq, nq, d = q.shape
    hkv = k.shape[1]
    assert hq % hkv == 0, "Hq must be a multiple of Hkv"
    gsz = hq // hkv
    nkv = k.shape[2]
    fb = _full_bias(bias, b, hq, nq, nkv)
    o = np.zeros((b, hq, nq, d))
    lse = np.zeros((b, hq, nq))
    items = [(bi, g) for bi in range(b) for g in range(hkv)]

    def run(it):
        bi, g = it
        sl = slice(g * gsz, (g + 1) * gsz)
        return group_forward(q[bi, sl], k[bi, g], v[bi, g], scale, causal, None if fb is None else fb[bi, sl])

    for (bi, g), (og, lg) in zip(items, _map_groups(run, items)):
        o[bi, g * gsz:(g + 1) * gsz] = og
        lse[bi, g * gsz:(g + 1) * gsz] = lg
    return o, lse


def attn_bwd(q, k, v, do, *, scale: float, causal: bool, bias=None, dlse=None):
    """Dense backward of L = sum(dO * O) (+ sum(dLSE * LSE) when ``dlse`` [B,Hq,Nq] is given).
    Returns (dQ, dK, dV) float64 with the input shapes, and with a bias also dBias with the bias's
    shape (dS summed over its broadcast dimensions)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    dl = None if dlse is None else _f64(dlse)
    b, hq, nq, d = q.shape
    hkv = k.shape[1]
    gsz = hq // hkv
    nkv = k.shape[2]
    fb = _full_bias(bias, b, hq, nq, nkv)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    ds = None if fb is None else np.zeros((b, hq, nq, nkv))
    items = [(bi, g) for bi in range(b) for g in range(hkv)]

    def run(it):
        bi, g = it
        sl = slice(g * gsz, (g + 1) * gsz)
        r = group_backward(q[bi, sl], k[bi, g], v[bi, g], do[bi, sl], scale, causal,
                           None if fb is None else fb[bi, sl], None if dl is None else dl[bi, sl])
        return r[:3] + (r[6],)

    for (bi, g), (dqg, dkg, dvg, dsg) in zip(items, _map_groups(run, items)):
        dq[bi, g * gsz:(g + 1) * gsz] = dqg
        dk[bi, g] = dkg
        dv[bi, g] = dvg
        if ds is not None:
            ds[bi, g * gsz:(g + 1) * gsz] = dsg
    if ds is None:
        return dq, dk, dv
    return dq, dk, dv, reduce_to_shape(ds, np.shape(bias))


def preprocess_delta(o, do) -> np.ndarray:
    """Backward stage 1: Delta = rowsum(dO * O) over the last axis."""
    return np.sum(_f64(do) * _f64(o), axis=-1)


def _seq_slices(cu):
    cu = [int(x) for x in _f64(cu).astype(np.int64)]
    return [(cu[s], cu[s + 1]) for s in range(len(cu) - 1)]


def varlen_fwd(q, k, v, cu_q, cu_k, *, scale: float, causal: bool):
    """Packed forward. q [Tq,Hq,D]; k, v [Tk,Hkv,D]; cu_* int [B+1].

    Returns (O [Tq,Hq,D], LSE [Hq,Tq]). Each sequence s attends within its own slice, with the
    causal mask aligned to the end of that slice.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    tq, hq, d = q.shape
    hkv = k.shape[1]
    gsz = hq // hkv
    o = np.zeros((tq, hq, d))
    lse = np.full((hq, tq), -np.inf)
    sq, sk = _seq_slices(cu_q), _seq_slices(cu_k)
    items = [(s, g) for s in range(len(sq)) for g in range(hkv)]

    def run(it):
        s, g = it
        (q0, q1), (k0, k1) = sq[s], sk[s]
        qg = np.transpose(q[q0:q1, g * gsz:(g + 1) * gsz], (1, 0, 2))
        return group_forward(qg, k[k0:k1, g], v[k0:k1, g], scale, causal)

    for (s, g), (og, lg) in zip(items, _map_groups(run, items)):
        q0, q1 = sq[s]
        o[q0:q1, g * gsz:(g + 1) * gsz] = np.transpose(og, (1, 0, 2))
        lse[g * gsz:(g + 1) * gsz, q0:q1] = lg
    return o, lse


def varlen_bwd(q, k, v, do, cu_q, cu_k, *, scale: float, causal: bool, dlse=None):
    """Packed backward (``dlse`` None or [Hq,Tq], the LSE's gradient, as in attn_bwd).
    Returns (dQ [Tq,Hq,D], dK [Tk,Hkv,D], dV [Tk,Hkv,D]) float64."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    dl = None if dlse is None else _f64(dlse)
    tq, hq, d = q.shape
    hkv = k.shape[1]
    gsz = hq // hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    sq, sk = _seq_slices(cu_q), _seq_slices(cu_k)
    items = [(s, g) for s in range(len(sq)) for g in range(hkv)]

    def run(it):
        s, g = it
        (q0, q1), (k0, k1) = sq[s], sk[s]
        sl = slice(g * gsz, (g + 1) * gsz)
        qg = np.transpose(q[q0:q1, sl], (1, 0, 2))
        dog = np.transpose(do[q0:q1, sl], (1, 0, 2))
        return group_backward(qg, k[k0:k1, g], v[k0:k1, g], dog, scale, causal, None,
                              None if dl is None else dl[sl, q0:q1])[:3]

    for (s, g), (dqg, dkg, dvg) in zip(items, _map_groups(run, items)):
        (q0, q1), (k0, k1) = sq[s], sk[s]
        dq[q0:q1, g * gsz:(g + 1) * gsz] = np.transpose(dqg, (1, 0, 2))
        dk[k0:k1, g] += dkg
        dv[k0:k1, g] += dvg
    return dq, dk, dv


def fwd_rows(q_head, k_head, v_head, rows, *, scale: float, causal: bool):
    """Forward for selected query rows of one head: q_head [Nq,D], k/v_head [Nkv,D].

    Rows are independent, so this is the same definition restricted to ``rows``; it lets a test
    check sampled outputs of a full-size launch one row at a time.
    """
    qh, kh, vh = _f64(q_head), _f64(k_head), _f64(v_head)
    nq, nkv = qh.shape[0], kh.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    s = scale * (qh[rows] @ kh.T)
    p, lse = softmax_rows(s, legal_mask(rows, nq, nkv, causal))
    return p @ vh, lse


# ------------------------------------------------------------------------------------------------
# FP8 forward ("Backends Overview", backend table and notes: FP8 attention quantizes fp16/bf16
# Q, K, V inside the kernel; forward only). The guide's FP8 page is not among the pages, so the
# scale granularity below is a reading: OCP e4m3, one scale per (batch, head) and tensor
# (448 / amax, applied in fp32), P = exp(S - row max) quantized as e4m3(P * 448), and
# O = (P8 V8) / l with l the unquantized row sum. The quantized tensors are exact (both sides take
# the rounding decision on the same fp32 value); P8 is taken against the final row max here and
# against a running max on the GPU, so O agrees to the e4m3 rounding of P only.
# ------------------------------------------------------------------------------------------------
def e4m3(x) -> np.ndarray:
    """float64 values of fp32 inputs rounded to OCP e4m3 (float8_e4m3fn), nearest even, saturating
    at 448 (PyTorch's cast)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def fp8_quantize(x: np.ndarray):
    """Per-(batch, head) e4m3 quantization of x [B, H, N, D]: returns (x8 [B,H,N,D] float64 e4m3
    values, amax [B,H] float64). x8 = e4m3(fp32(x) * fp32(448 / amax)) (0 for a zero head)."""
    x = _f64(x)
    amax = np.abs(x).max(axis=(2, 3))
    f = np.where(amax > 0, np.float32(448.0) / amax.astype(np.float32), np.float32(0.0)).astype(np.float32)
    x8 = e4m3(x.astype(np.float32) * f[:, :, None, None])
    return x8, amax


def attn_fwd_fp8(q, k, v, *, scale: float, causal: bool, parts: bool = False):
    """FP8 forward as read above. Returns (O [B,Hq,Nq,D], LSE [B,Hq,Nq]) float64; with
    ``parts`` also a dict of the unquantized P [B,Hq,Nq,Nkv] (against the final row max, 0 for
    illegal keys), its row sums l [B,Hq,Nq] and the dequantized V8 [B,Hkv,Nkv,D] (V8 * amax / 448),
    from which a caller can bound any other placement of the P rounding."""
    q8, aq = fp8_quantize(q)
    k8, ak = fp8_quantize(k)
    v8, av = fp8_quantize(v)
    b, hq, nq, d = q8.shape
    hkv, nkv = k8.shape[1], k8.shape[2]
    gsz = hq // hkv
    o = np.zeros((b, hq, nq, d))
    lse = np.full((b, hq, nq), -np.inf)
    p_all = np.zeros((b, hq, nq, nkv)) if parts else None
    l_all = np.zeros((b, hq, nq)) if parts else None
    legal = legal_mask(np.arange(nq), nq, nkv, causal)
    for bi in range(b):
        for h in range(hq):
            g = h // gsz
            s = scale * (q8[bi, h] @ k8[bi, g].T) * (aq[bi, h] / 448.0) * (ak[bi, g] / 448.0)
            s = np.where(legal, s, -np.inf)
            has = legal.any(axis=1)
            m = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
            p = np.where(legal, np.exp(s - m[:, None]), 0.0)
            l_ = p.sum(axis=1)
            p8 = e4m3(p * 448.0)
            safe = np.where(l_ > 0, l_, 1.0)
            o[bi, h] = np.where((l_ > 0)[:, None], (p8 @ v8[bi, g]) * (av[bi, g] / 448.0 / 448.0) / safe[:, None], 0.0)
            lse[bi, h] = np.where(l_ > 0, m + np.log(safe), -np.inf)
            if parts:
                p_all[bi, h], l_all[bi, h] = p, l_
    if parts:
        return o, lse, {"p": p_all, "l": l_all, "v": v8 * (av / 448.0)[:, :, None, None]}
    return o, lse
