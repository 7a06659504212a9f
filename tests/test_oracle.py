"""Pins for the CPU float64 oracle (no GPU needed).

Each check ties the oracle to something other than itself: hand-derived cases, closed forms,
invariants, brute force on tiny inputs, central finite differences, and PyTorch's own SDPA +
autograd as an independent library routine. Together they are chosen so that a dropped scale,
a wrong sign, a top-left instead of bottom-right causal offset, a wrong GQA head map or a
transposed operand fails at least one test.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------------------------
# Hand-derived cases (tests/golden/hand_cases.json; derivations in the file).
# ----------------------------------------------------------------------------------------------
def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_golden_hand_cases(case):
    scale = case["scale"]
    w = np.array(case["weights"][0], dtype=np.float64)
    k = np.stack([np.log(w) / scale, np.zeros_like(w)], axis=1)          # [Nkv, 2]
    q = np.array(case["q"], dtype=np.float64)                              # [Nq, 2]
    v = np.array(case["v"], dtype=np.float64)
    do = np.array(case["do"], dtype=np.float64)
    qd, kd, vd, dod = q[None, None], k[None, None], v[None, None], do[None, None]
    o, lse = ref.attn_fwd(qd, kd, vd, scale=scale, causal=case["causal"])
    np.testing.assert_allclose(o[0, 0], np.array(case["expect_o"], dtype=np.float64), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], np.log(np.array(case["expect_lse_exp"], dtype=np.float64)),
                               rtol=0, atol=1e-12)
    dq, dk, dv = ref.attn_bwd(qd, kd, vd, dod, scale=scale, causal=case["causal"])
    np.testing.assert_allclose(dv[0, 0], np.array(case["expect_dv"]), rtol=0, atol=1e-12)
    ds = np.array(case["expect_ds"], dtype=np.float64)                     # [Nq, Nkv], by hand
    # Closed forms from the derivation: dK_j = scale sum_i dS_ij q_i ; dQ_i = scale sum_j dS_ij k_j.
    exp_dk = np.array([[scale * sum(ds[i, j] * q[i, c] for i in range(q.shape[0])) for c in range(2)]
                       for j in range(k.shape[0])])
    exp_dq = np.array([[scale * sum(ds[i, j] * k[j, c] for j in range(k.shape[0])) for c in range(2)]
                       for i in range(q.shape[0])])
    np.testing.assert_allclose(dk[0, 0], exp_dk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq[0, 0], exp_dq, rtol=0, atol=1e-12)
    if case["name"] == "three_keys_scale_one":
        # dQ written with the logarithms of the weights, as in the derivation text.
        assert abs(dq[0, 0, 0, 0] - (-1.5 * math.log(2) + 1.25 * math.log(5))) < 1e-12


# ----------------------------------------------------------------------------------------------
# P-a: constant V rows give O = that row, for every row with a legal key.
# ----------------------------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_constant_v(causal):
    r = rng(1)
    q = r.standard_normal((2, 4, 9, 16))
    k = r.standard_normal((2, 2, 6, 16))
    c = r.standard_normal(16)
    v = np.broadcast_to(c, (2, 2, 6, 16)).copy()
    o, lse = ref.attn_fwd(q, k, v, scale=0.3, causal=causal)
    legal_rows = ref.legal_mask(np.arange(9), 9, 6, causal).any(axis=1)
    np.testing.assert_allclose(o[:, :, legal_rows], np.broadcast_to(c, o[:, :, legal_rows].shape), atol=1e-13)
    assert np.all(o[:, :, ~legal_rows] == 0.0)


# ----------------------------------------------------------------------------------------------
# P-b: softmax rows sum to one; P-d: LSE against brute-force log-sum-exp with math.fsum.
# ----------------------------------------------------------------------------------------------
def test_softmax_rows_sum_to_one():
    r = rng(2)
    s = r.standard_normal((7, 11)) * 3
    for causal, nq in [(False, 7), (True, 7), (True, 11)]:
        rows = np.arange(7)
        legal = ref.legal_mask(rows, nq, 11, causal)
        p, _ = ref.softmax_rows(s, legal)
        sums = p.sum(axis=1)
        np.testing.assert_allclose(sums[legal.any(axis=1)], 1.0, atol=1e-14)
        assert np.all(p[~legal] == 0.0)


def test_lse_brute_force():
    r = rng(3)
    q = r.standard_normal((1, 1, 5, 8))
    k = r.standard_normal((1, 1, 7, 8)) * 2.0
    v = r.standard_normal((1, 1, 7, 8))
    scale = 0.7
    for causal in (False, True):
        _, lse = ref.attn_fwd(q, k, v, scale=scale, causal=causal)
        for i in range(5):
            terms = []
            for j in range(7):
                if causal and j > i + (7 - 5):
                    continue
                sij = scale * math.fsum(float(q[0, 0, i, c]) * float(k[0, 0, j, c]) for c in range(8))
                terms.append(math.exp(sij))
            assert abs(lse[0, 0, i] - math.log(math.fsum(terms))) < 1e-12


# ----------------------------------------------------------------------------------------------
# P-c: causal with Nq == Nkv: row 0 sees only key 0, so O_0 = V_0 and LSE_0 = S_00.
# ----------------------------------------------------------------------------------------------
def test_causal_row0():
    r = rng(4)
    q = r.standard_normal((1, 3, 10, 12))
    k = r.standard_normal((1, 3, 10, 12))
    v = r.standard_normal((1, 3, 10, 12))
    o, lse = ref.attn_fwd(q, k, v, scale=0.25, causal=True)
    np.testing.assert_allclose(o[0, :, 0], v[0, :, 0], atol=1e-15)
    np.testing.assert_allclose(lse[0, :, 0], 0.25 * np.einsum("hd,hd->h", q[0, :, 0], k[0, :, 0]), atol=1e-14)


# ----------------------------------------------------------------------------------------------
# P-f: Q = 0 gives uniform weights over the legal keys: prefix means pin the bottom-right offset.
# ----------------------------------------------------------------------------------------------
@pytest.mark.parametrize("nq,nkv", [(6, 6), (4, 9), (9, 4)])
def test_zero_query_prefix_means(nq, nkv):
    r = rng(5)
    q = np.zeros((1, 2, nq, 8))
    k = r.standard_normal((1, 2, nkv, 8))
    v = r.standard_normal((1, 2, nkv, 8))
    o, lse = ref.attn_fwd(q, k, v, scale=1.0, causal=True)
    for i in range(nq):
        last = i + nkv - nq                  # last legal key (bottom-right alignment)
        if last < 0:
            assert np.all(o[0, :, i] == 0.0) and np.all(np.isneginf(lse[0, :, i]))
            continue
        np.testing.assert_allclose(o[0, :, i], v[0, :, :last + 1].mean(axis=1), atol=1e-14)
        np.testing.assert_allclose(lse[0, :, i], math.log(last + 1), atol=1e-14)
    o2, lse2 = ref.attn_fwd(q, k, v, scale=1.0, causal=False)
    np.testing.assert_allclose(o2[0], np.broadcast_to(v[0].mean(axis=1, keepdims=True), o2[0].shape), atol=1e-14)
    np.testing.assert_allclose(lse2, math.log(nkv), atol=1e-14)


# ----------------------------------------------------------------------------------------------
# P-g: a single key: O_i = V_0 and LSE_i = S_i0.
# ----------------------------------------------------------------------------------------------
def test_single_key():
    r = rng(6)
    q = r.standard_normal((1, 2, 5, 8))
    k = r.standard_normal((1, 2, 1, 8))
    v = r.standard_normal((1, 2, 1, 8))
    o, lse = ref.attn_fwd(q, k, v, scale=0.5, causal=False)
    np.testing.assert_allclose(o[0], np.broadcast_to(v[0], o[0].shape), atol=1e-15)
    np.testing.assert_allclose(lse[0], 0.5 * np.einsum("hnd,hd->hn", q[0], k[0, :, 0]), atol=1e-14)


# ----------------------------------------------------------------------------------------------
# P-e: gradients against central finite differences of L = sum(dO * O).
# ----------------------------------------------------------------------------------------------
def _fd_check(q, k, v, do, scale, causal, varlen=None, dlse=None):
    """Central differences of L = sum(dO * O), plus sum(dLSE * LSE) over the rows with a finite
    LSE when dlse is given (an empty row's LSE is the constant -inf)."""
    eps = 1e-6

    def loss(qq, kk, vv):
        if varlen is None:
            o, lse = ref.attn_fwd(qq, kk, vv, scale=scale, causal=causal)
        else:
            o, lse = ref.varlen_fwd(qq, kk, vv, varlen[0], varlen[1], scale=scale, causal=causal)
        total = float(np.sum(do * o))
        if dlse is not None:
            fin = np.isfinite(lse)
            total += float(np.sum(dlse[fin] * lse[fin]))
        return total

    if varlen is None:
        grads = ref.attn_bwd(q, k, v, do, scale=scale, causal=causal, dlse=dlse)
    else:
        grads = ref.varlen_bwd(q, k, v, do, varlen[0], varlen[1], scale=scale, causal=causal, dlse=dlse)
    for which, (x, g) in enumerate(zip((q, k, v), grads)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += eps
            lp = loss(*args)
            args[which][idx] -= 2 * eps
            lm = loss(*args)
            num[idx] = (lp - lm) / (2 * eps)
        err = np.linalg.norm(num - g) / max(np.linalg.norm(num), 1e-30)
        assert err < 1e-6, f"grad {'qkv'[which]} rel err {err}"


@pytest.mark.parametrize("causal", [False, True])
def test_fd_gqa(causal):
    r = rng(7)
    q = r.standard_normal((2, 4, 5, 8))
    k = r.standard_normal((2, 2, 7, 8))
    v = r.standard_normal((2, 2, 7, 8))
    do = r.standard_normal((2, 4, 5, 8))
    _fd_check(q, k, v, do, 0.4, causal)


def test_fd_cross_causal_with_empty_rows():
    r = rng(8)
    q = r.standard_normal((1, 2, 7, 6))
    k = r.standard_normal((1, 1, 5, 6))
    v = r.standard_normal((1, 1, 5, 6))
    do = r.standard_normal((1, 2, 7, 6))
    _fd_check(q, k, v, do, 0.5, True)
    dq, _, _ = ref.attn_bwd(q, k, v, do, scale=0.5, causal=True)
    assert np.all(dq[:, :, :2] == 0.0)     # rows 0 and 1 have no legal key (i + 5 - 7 < 0)


def test_fd_varlen():
    r = rng(9)
    cu_q = np.array([0, 3, 3, 8])
    cu_k = np.array([0, 4, 6, 6])
    q = r.standard_normal((8, 2, 6))
    k = r.standard_normal((6, 1, 6))
    v = r.standard_normal((6, 1, 6))
    do = r.standard_normal((8, 2, 6))
    for causal in (False, True):
        _fd_check(q, k, v, do, 0.6, causal, varlen=(cu_q, cu_k))


@pytest.mark.parametrize("causal", [False, True])
def test_fd_lse_gradient_dense(causal):
    """The returned LSE carries its own gradient: finite differences of sum(dO*O) + sum(g*LSE) on
    GQA with empty rows (causal, Nq > Nkv)."""
    r = rng(31)
    q = r.standard_normal((1, 4, 7, 6))
    k = r.standard_normal((1, 2, 5, 6))
    v = r.standard_normal((1, 2, 5, 6))
    do = r.standard_normal((1, 4, 7, 6))
    g = r.standard_normal((1, 4, 7))
    _fd_check(q, k, v, do, 0.45, causal, dlse=g)
    # With dO = 0 the loss is sum(g * LSE) alone: dV is exactly zero (LSE does not depend on V).
    _, _, dv = ref.attn_bwd(q, k, v, np.zeros_like(do), scale=0.45, causal=causal, dlse=g)
    assert np.all(dv == 0.0)


def test_fd_lse_gradient_varlen():
    r = rng(32)
    cu_q = np.array([0, 3, 3, 8])
    cu_k = np.array([0, 4, 6, 6])
    q = r.standard_normal((8, 2, 6))
    k = r.standard_normal((6, 1, 6))
    v = r.standard_normal((6, 1, 6))
    do = r.standard_normal((8, 2, 6))
    g = r.standard_normal((2, 8))
    for causal in (False, True):
        _fd_check(q, k, v, do, 0.6, causal, varlen=(cu_q, cu_k), dlse=g)


def test_lse_gradient_closed_form():
    """dLSE alone on one query: dQ = scale * g * sum_j P_j k_j - which with Q = 0 (uniform P) is
    scale * g * mean(k); dK_j = scale * g * P_j q = scale * g * q / Nkv."""
    r = rng(33)
    nkv, d, scale, g = 5, 4, 0.7, 1.3
    q = np.zeros((1, 1, 1, d))
    k = r.standard_normal((1, 1, nkv, d))
    v = r.standard_normal((1, 1, nkv, d))
    dq, dk, dv = ref.attn_bwd(q, k, v, np.zeros((1, 1, 1, d)), scale=scale, causal=False,
                              dlse=np.full((1, 1, 1), g))
    np.testing.assert_allclose(dq[0, 0, 0], scale * g * k[0, 0].mean(axis=0), atol=1e-14)
    np.testing.assert_allclose(dk[0, 0], np.zeros((nkv, d)), atol=1e-15)   # q = 0
    q2 = r.standard_normal((1, 1, 1, d))
    _, dk2, _ = ref.attn_bwd(q2, np.zeros_like(k), v, np.zeros((1, 1, 1, d)), scale=scale, causal=False,
                             dlse=np.full((1, 1, 1), g))
    np.testing.assert_allclose(dk2[0, 0], np.broadcast_to(scale * g * q2[0, 0, 0] / nkv, (nkv, d)), atol=1e-14)


def test_lse_gradient_against_torch_autograd():
    """PyTorch float64 autograd of sum(dO*O) + sum(g*logsumexp(S)) with an explicit bottom-right mask."""
    r = rng(34)
    nq, nkv, d, scale = 6, 9, 5, 0.5
    q = r.standard_normal((1, 2, nq, d))
    k = r.standard_normal((1, 2, nkv, d))
    v = r.standard_normal((1, 2, nkv, d))
    do = r.standard_normal((1, 2, nq, d))
    g = r.standard_normal((1, 2, nq))
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    legal = torch.tensor(ref.legal_mask(np.arange(nq), nq, nkv, True))
    s = scale * qt @ kt.transpose(-1, -2)
    s = s.masked_fill(~legal, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    o = torch.softmax(s, dim=-1) @ vt
    (torch.sum(torch.tensor(do) * o) + torch.sum(torch.tensor(g) * lse)).backward()
    got = ref.attn_bwd(q, k, v, do, scale=scale, causal=True, dlse=g)
    for x, t in zip(got, (qt, kt, vt)):
        np.testing.assert_allclose(x, t.grad.numpy(), rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------------------------------------
# P-h: invariants of the backward.
# ----------------------------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    r = rng(10)
    nq, nkv = 9, 6
    q = r.standard_normal((1, 4, nq, 8))
    k = r.standard_normal((1, 2, nkv, 8))
    v = r.standard_normal((1, 2, nkv, 8))
    do = r.standard_normal((1, 4, nq, 8))
    dq, dk, dv = ref.attn_bwd(q, k, v, do, scale=0.3, causal=causal)
    # sum_j dS_ij = 0 for each row, so the KV-axis sum of dK vanishes for every KV head.
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # sum_j P_ij = 1 for non-empty rows, so sum_j dV_j = sum over non-empty rows of the group's dO.
    rows_ok = ref.legal_mask(np.arange(nq), nq, nkv, causal).any(axis=1)
    expect = do[:, :, rows_ok].reshape(1, 2, 2, -1, 8).sum(axis=(2, 3))
    np.testing.assert_allclose(dv.sum(axis=2), expect, atol=1e-12)


# ----------------------------------------------------------------------------------------------
# P-i: GQA equals MHA on repeat_interleave'd K/V (grads are group sums); varlen equals dense.
# ----------------------------------------------------------------------------------------------
def test_gqa_equals_repeated_mha():
    r = rng(11)
    q = r.standard_normal((2, 6, 5, 8))
    k = r.standard_normal((2, 2, 7, 8))
    v = r.standard_normal((2, 2, 7, 8))
    do = r.standard_normal((2, 6, 5, 8))
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    for causal in (False, True):
        o1, l1 = ref.attn_fwd(q, k, v, scale=0.4, causal=causal)
        o2, l2 = ref.attn_fwd(q, kr, vr, scale=0.4, causal=causal)
        np.testing.assert_allclose(o1, o2, atol=1e-14)
        np.testing.assert_allclose(l1, l2, atol=1e-14)
        g1 = ref.attn_bwd(q, k, v, do, scale=0.4, causal=causal)
        g2 = ref.attn_bwd(q, kr, vr, do, scale=0.4, causal=causal)
        np.testing.assert_allclose(g1[0], g2[0], atol=1e-13)
        np.testing.assert_allclose(g1[1], g2[1].reshape(2, 2, 3, 7, 8).sum(axis=2), atol=1e-13)
        np.testing.assert_allclose(g1[2], g2[2].reshape(2, 2, 3, 7, 8).sum(axis=2), atol=1e-13)


def test_varlen_equals_dense_per_sequence():
    r = rng(12)
    lq, lk = [3, 0, 5, 4], [4, 2, 2, 6]
    cu_q, cu_k = np.cumsum([0] + lq), np.cumsum([0] + lk)
    q = r.standard_normal((sum(lq), 4, 8))
    k = r.standard_normal((sum(lk), 2, 8))
    v = r.standard_normal((sum(lk), 2, 8))
    do = r.standard_normal((sum(lq), 4, 8))
    for causal in (False, True):
        o, lse = ref.varlen_fwd(q, k, v, cu_q, cu_k, scale=0.5, causal=causal)
        dq, dk, dv = ref.varlen_bwd(q, k, v, do, cu_q, cu_k, scale=0.5, causal=causal)
        for s in range(4):
            qs = q[cu_q[s]:cu_q[s + 1]].transpose(1, 0, 2)[None]
            ks = k[cu_k[s]:cu_k[s + 1]].transpose(1, 0, 2)[None]
            vs = v[cu_k[s]:cu_k[s + 1]].transpose(1, 0, 2)[None]
            dos = do[cu_q[s]:cu_q[s + 1]].transpose(1, 0, 2)[None]
            od, ld = ref.attn_fwd(qs, ks, vs, scale=0.5, causal=causal)
            np.testing.assert_allclose(o[cu_q[s]:cu_q[s + 1]], od[0].transpose(1, 0, 2), atol=1e-14)
            np.testing.assert_allclose(lse[:, cu_q[s]:cu_q[s + 1]], ld[0], atol=1e-14)
            gd = ref.attn_bwd(qs, ks, vs, dos, scale=0.5, causal=causal)
            np.testing.assert_allclose(dq[cu_q[s]:cu_q[s + 1]], gd[0][0].transpose(1, 0, 2), atol=1e-13)
            np.testing.assert_allclose(dk[cu_k[s]:cu_k[s + 1]], gd[1][0].transpose(1, 0, 2), atol=1e-13)
            np.testing.assert_allclose(dv[cu_k[s]:cu_k[s + 1]], gd[2][0].transpose(1, 0, 2), atol=1e-13)


# ----------------------------------------------------------------------------------------------
# P-j: PyTorch float64 SDPA with an explicit boolean mask, plus torch autograd, as an independent
# library routine (never is_causal: PyTorch's causal flag is top-left aligned).
# ----------------------------------------------------------------------------------------------
@pytest.mark.parametrize("nq,nkv,causal", [(6, 6, False), (6, 6, True), (5, 9, True), (12, 7, False)])
def test_against_torch_sdpa(nq, nkv, causal):
    r = rng(13)
    d = 16
    q = r.standard_normal((2, 4, nq, d))
    k = r.standard_normal((2, 2, nkv, d))
    v = r.standard_normal((2, 2, nkv, d))
    do = r.standard_normal((2, 4, nq, d))
    scale = 1.0 / math.sqrt(d)
    o, lse = ref.attn_fwd(q, k, v, scale=scale, causal=causal)
    dq, dk, dv = ref.attn_bwd(q, k, v, do, scale=scale, causal=causal)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    mask = torch.tensor(ref.legal_mask(np.arange(nq), nq, nkv, causal) if causal else np.ones((nq, nkv), bool))
    ke = tk.repeat_interleave(2, dim=1)
    ve = tv.repeat_interleave(2, dim=1)
    to = torch.nn.functional.scaled_dot_product_attention(tq, ke, ve, attn_mask=mask, scale=scale)
    to.backward(torch.tensor(do))
    np.testing.assert_allclose(o, to.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)
    # LSE via torch.logsumexp of the masked scores.
    s = scale * torch.matmul(torch.tensor(q), torch.tensor(k).repeat_interleave(2, dim=1).transpose(-1, -2))
    s = s.masked_fill(~mask, float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12)


# ----------------------------------------------------------------------------------------------
# P-k: rows without a legal key are exactly O = 0, LSE = -inf and zero gradient; they also add
# nothing to dK/dV.
# ----------------------------------------------------------------------------------------------
def test_empty_rows_exact():
    r = rng(14)
    q = r.standard_normal((1, 2, 8, 8))
    k = r.standard_normal((1, 2, 3, 8))
    v = r.standard_normal((1, 2, 3, 8))
    do = r.standard_normal((1, 2, 8, 8))
    o, lse = ref.attn_fwd(q, k, v, scale=0.5, causal=True)
    assert np.all(o[:, :, :5] == 0.0) and np.all(np.isneginf(lse[:, :, :5]))
    dq, dk, dv = ref.attn_bwd(q, k, v, do, scale=0.5, causal=True)
    assert np.all(dq[:, :, :5] == 0.0)
    do2 = do.copy()
    do2[:, :, :5] = 1e6                    # gradient flowing into empty rows must not reach dK/dV
    _, dk2, dv2 = ref.attn_bwd(q, k, v, do2, scale=0.5, causal=True)
    np.testing.assert_array_equal(dk, dk2)
    np.testing.assert_array_equal(dv, dv2)
    # varlen: a sequence with no keys gives empty rows too.
    cu_q, cu_k = np.array([0, 2, 5]), np.array([0, 0, 3])
    qv = r.standard_normal((5, 2, 8))
    kv_ = r.standard_normal((3, 2, 8))
    vv = r.standard_normal((3, 2, 8))
    ov, lv = ref.varlen_fwd(qv, kv_, vv, cu_q, cu_k, scale=0.5, causal=False)
    assert np.all(ov[:2] == 0.0) and np.all(np.isneginf(lv[:, :2]))


def test_preprocess_delta():
    r = rng(15)
    o = r.standard_normal((2, 3, 4, 5))
    do = r.standard_normal((2, 3, 4, 5))
    delta = ref.preprocess_delta(o, do)
    for idx in np.ndindex(2, 3, 4):
        assert abs(delta[idx] - math.fsum(float(a) * float(b) for a, b in zip(o[idx], do[idx]))) < 1e-12


def test_fwd_rows_matches_full():
    r = rng(16)
    q = r.standard_normal((1, 1, 20, 8))
    k = r.standard_normal((1, 1, 13, 8))
    v = r.standard_normal((1, 1, 13, 8))
    for causal in (False, True):
        o, lse = ref.attn_fwd(q, k, v, scale=0.3, causal=causal)
        rows = np.array([0, 5, 7, 19])
        orow, lrow = ref.fwd_rows(q[0, 0], k[0, 0], v[0, 0], rows, scale=0.3, causal=causal)
        np.testing.assert_allclose(orow, o[0, 0, rows], atol=1e-14)
        np.testing.assert_allclose(lrow, lse[0, 0, rows], atol=1e-14)


# ----------------------------------------------------------------------------------------------
# P-m: attn_mask. An additive bias is added to the scaled scores and a boolean mask is the bias
# 0 / -inf ("Triton Backend", "Feature support": boolean and additive masks broadcast in any
# dimension, the bias gradient reduced to the mask's shape).
# ----------------------------------------------------------------------------------------------
def test_bias_row_constant_shifts_lse_only():
    """Adding c_i to every score of row i leaves P and O unchanged and adds c_i to LSE_i."""
    r = rng(21)
    q = r.standard_normal((1, 2, 5, 8))
    k = r.standard_normal((1, 1, 7, 8))
    v = r.standard_normal((1, 1, 7, 8))
    c = r.standard_normal((1, 2, 5, 1))
    for causal in (False, True):
        o0, l0 = ref.attn_fwd(q, k, v, scale=0.3, causal=causal)
        o1, l1 = ref.attn_fwd(q, k, v, scale=0.3, causal=causal, bias=c)
        np.testing.assert_allclose(o1, o0, atol=1e-13)
        np.testing.assert_allclose(l1, l0 + c[..., 0], atol=1e-13)


def test_mask_equals_causal_and_empty_rows():
    """A boolean mask with the bottom-right causal pattern gives exactly the causal results;
    a row the mask empties is O = 0, LSE = -inf with zero gradient."""
    r = rng(22)
    nq, nkv = 6, 4
    q = r.standard_normal((2, 2, nq, 8))
    k = r.standard_normal((2, 2, nkv, 8))
    v = r.standard_normal((2, 2, nkv, 8))
    do = r.standard_normal((2, 2, nq, 8))
    keep = np.arange(nkv)[None, :] <= np.arange(nq)[:, None] + (nkv - nq)
    bias = ref.mask_to_bias(keep)
    o0, l0 = ref.attn_fwd(q, k, v, scale=0.5, causal=True)
    o1, l1 = ref.attn_fwd(q, k, v, scale=0.5, causal=False, bias=bias)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    g0 = ref.attn_bwd(q, k, v, do, scale=0.5, causal=True)
    g1 = ref.attn_bwd(q, k, v, do, scale=0.5, causal=False, bias=bias)
    for a, b in zip(g0, g1[:3]):
        assert np.array_equal(a, b)
    assert np.all(l1[:, :, :2] == -np.inf) and np.all(o1[:, :, :2] == 0)
    assert np.all(g1[3][:2] == 0) and g1[3].shape == bias.shape


@pytest.mark.parametrize("shape", [(2, 4, 5, 6), (1, 4, 5, 6), (2, 1, 5, 6), (1, 1, 5, 6), (2, 4, 1, 6),
                                   (1, 4, 5, 1), (5, 6)])
def test_fd_bias_gradient(shape):
    """dBias against central finite differences of L = sum(dO * O), for full and broadcast
    biases (the gradient of a broadcast bias is the sum over the dimensions it broadcasts)."""
    r = rng(23)
    q = r.standard_normal((2, 4, 5, 8))
    k = r.standard_normal((2, 2, 6, 8))
    v = r.standard_normal((2, 2, 6, 8))
    do = r.standard_normal((2, 4, 5, 8))
    bias = r.standard_normal(shape)
    for causal in (False, True):
        g = ref.attn_bwd(q, k, v, do, scale=0.4, causal=causal, bias=bias)
        assert g[3].shape == bias.shape
        num = np.zeros_like(bias)
        eps = 1e-6
        for idx in np.ndindex(bias.shape):
            bp, bm = bias.copy(), bias.copy()
            bp[idx] += eps
            bm[idx] -= eps
            lp = float(np.sum(do * ref.attn_fwd(q, k, v, scale=0.4, causal=causal, bias=bp)[0]))
            lm = float(np.sum(do * ref.attn_fwd(q, k, v, scale=0.4, causal=causal, bias=bm)[0]))
            num[idx] = (lp - lm) / (2 * eps)
        # (a bias constant along the keys has a zero gradient: rows of dS sum to zero)
        assert np.linalg.norm(num - g[3]) <= 1e-6 * max(np.linalg.norm(num), 1.0)


def test_bias_gradient_rows_sum_to_zero():
    """Each row of the full bias gradient (dS) sums to zero: sum_j P_ij (dP_ij - Delta_i) = 0."""
    r = rng(24)
    q = r.standard_normal((1, 2, 6, 8))
    k = r.standard_normal((1, 2, 9, 8))
    v = r.standard_normal((1, 2, 9, 8))
    do = r.standard_normal((1, 2, 6, 8))
    bias = r.standard_normal((1, 2, 6, 9))
    db = ref.attn_bwd(q, k, v, do, scale=0.5, causal=True, bias=bias)[3]
    np.testing.assert_allclose(db.sum(axis=-1), 0.0, atol=1e-13)


@pytest.mark.parametrize("kind", ["additive", "boolean"])
def test_bias_against_torch_sdpa(kind):
    """PyTorch float64 SDPA with the same attn_mask (and autograd for the bias gradient)."""
    r = rng(25)
    b, hq, hkv, nq, nkv, d = 2, 4, 2, 5, 7, 16
    q = r.standard_normal((b, hq, nq, d))
    k = r.standard_normal((b, hkv, nkv, d))
    v = r.standard_normal((b, hkv, nkv, d))
    do = r.standard_normal((b, hq, nq, d))
    scale = 1.0 / math.sqrt(d)
    if kind == "additive":
        mask_np = r.standard_normal((1, hq, nq, nkv))
        bias = mask_np
        tm = torch.tensor(mask_np, requires_grad=True)
    else:
        mask_np = r.random((b, 1, nq, nkv)) > 0.3
        mask_np[..., 0] = True  # SDPA gives NaN for a fully masked row; keep one key per row
        bias = ref.mask_to_bias(mask_np)
        tm = torch.tensor(mask_np)
    o, lse = ref.attn_fwd(q, k, v, scale=scale, causal=False, bias=bias)
    g = ref.attn_bwd(q, k, v, do, scale=scale, causal=False, bias=bias)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(2, dim=1), tv.repeat_interleave(2, dim=1), attn_mask=tm, scale=scale)
    to.backward(torch.tensor(do))
    np.testing.assert_allclose(o, to.detach().numpy(), atol=1e-12)
    for a, t in zip(g[:3], (tq, tk, tv)):
        np.testing.assert_allclose(a, t.grad.numpy(), atol=1e-12)
    if kind == "additive":
        np.testing.assert_allclose(g[3], tm.grad.numpy(), atol=1e-12)


# ----------------------------------------------------------------------------------------------
# P-n: the FP8 forward's emulation. e4m3 rounding is pinned to the format's definition (3 mantissa
# bits, exponent bias 7, subnormals below 2^-6, nearest even, 448 the largest finite value).
# ----------------------------------------------------------------------------------------------
def _e4m3_by_definition(x: float) -> float:
    if x == 0:
        return 0.0
    sgn = -1.0 if x < 0 else 1.0
    a = abs(x)
    e = max(math.floor(math.log2(a)), -6)      # subnormals share the exponent -6
    q = 2.0 ** (e - 3)                          # spacing with 3 mantissa bits
    n = a / q
    r = math.floor(n)
    frac = n - r
    if frac > 0.5 or (frac == 0.5 and r % 2 == 1):
        r += 1
    return sgn * min(r * q, 448.0)


def test_e4m3_matches_definition():
    r = rng(31)
    xs = np.concatenate([r.standard_normal(3000) * s for s in (1e-3, 0.1, 3.0, 100.0)]).astype(np.float32)
    xs = np.concatenate([xs, np.float32([1.0625, 1.1875, 0.00146484375, 0.0009765625, 448.0, 463.9, -3.3, 0.0])])
    got = ref.e4m3(xs)
    want = np.array([_e4m3_by_definition(float(x)) for x in xs])
    assert np.array_equal(got, want)


def test_fp8_oracle_exact_when_representable():
    """e4m3-representable inputs whose head amax is 448 quantize to themselves; with one key, P = 1
    and P8 = 448, so the FP8 forward gives exactly V (and LSE = S)."""
    r = rng(32)
    grid = np.array([_e4m3_by_definition(x) for x in np.linspace(-448, 448, 301)])
    q = r.choice(grid, size=(1, 2, 3, 32))
    k = r.choice(grid, size=(1, 2, 1, 32))
    v = r.choice(grid, size=(1, 2, 1, 32))
    for t in (q, k, v):
        t[..., 0, 0] = 448.0
    q8, aq = ref.fp8_quantize(q)
    assert np.array_equal(q8, q) and np.all(aq == 448.0)
    o, lse = ref.attn_fwd_fp8(q, k, v, scale=1e-4, causal=False)
    np.testing.assert_array_equal(o, np.broadcast_to(v, o.shape))
    o_ex, lse_ex = ref.attn_fwd(q, k, v, scale=1e-4, causal=False)
    np.testing.assert_allclose(lse, lse_ex, rtol=1e-14)


def test_fp8_oracle_close_to_exact():
    """The FP8 reading stays within e4m3's relative precision (2^-4) of exact attention."""
    r = rng(33)
    q = r.standard_normal((1, 2, 40, 64))
    k = r.standard_normal((1, 1, 50, 64))
    v = r.standard_normal((1, 1, 50, 64))
    for causal in (False, True):
        o8, l8 = ref.attn_fwd_fp8(q, k, v, scale=0.125, causal=causal)
        o, l_ = ref.attn_fwd(q, k, v, scale=0.125, causal=causal)
        assert np.linalg.norm(o8 - o) / np.linalg.norm(o) < 2.0 ** -4
        fin = np.isfinite(l_)
        assert np.max(np.abs(l8[fin] - l_[fin])) < 0.1


def test_fp8_oracle_parts():
    """The intermediates the FP8 oracle hands out: every row of P with a legal key peaks at exactly
    1 (the final max) and sums to l, and V's dequantized values lie within e4m3's half-step of V
    (2^-4 relative for normals, 2^-10 of the scale below 2^-6)."""
    r = rng(34)
    q = r.standard_normal((1, 2, 9, 64))
    k = r.standard_normal((1, 1, 7, 64))
    v = r.standard_normal((1, 1, 7, 64))
    o8, lse8, parts = ref.attn_fwd_fp8(q, k, v, scale=0.125, causal=True, parts=True)
    o8b, lse8b = ref.attn_fwd_fp8(q, k, v, scale=0.125, causal=True)
    assert np.array_equal(o8, o8b) and np.array_equal(lse8, lse8b)
    p, l_ = parts["p"], parts["l"]
    has = np.isfinite(lse8)
    assert np.all(p[~has] == 0) and np.allclose(p.max(axis=-1)[has], 1.0)
    assert np.allclose(p.sum(axis=-1), l_)
    step = 2.0 ** -10 * np.abs(v).max() / 448.0  # half the subnormal spacing, in V's units
    assert np.all(np.abs(parts["v"] - v) <= np.maximum(2.0 ** -4 * np.abs(v), step) * (1 + 1e-6))
