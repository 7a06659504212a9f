"""Shared helpers for the GPU parity tests: tolerances and comparisons against the oracle.

Tolerances (the contract for this path): O max-abs <= 2e-2 (bf16) / 4e-3 (fp16); LSE max-abs
<= 1e-3 over finite entries with -inf entries matching position for position; dQ/dK/dV relative
L2 <= 2e-2. O relative L2 is printed as a diagnostic.
"""
import numpy as np
import torch

O_TOL = {torch.bfloat16: 2e-2, torch.float16: 4e-3}
LSE_TOL = 1e-3
GRAD_RTOL = 2e-2


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def rel_l2(x: np.ndarray, y: np.ndarray) -> float:
    ny = np.linalg.norm(y)
    return float(np.linalg.norm(x - y) / ny) if ny > 0 else float(np.linalg.norm(x))


def check_o_lse(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    o = to64(o_gpu)
    lse = lse_gpu.detach().to("cpu").numpy().astype(np.float64)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref)), f"{what}: -inf LSE positions differ"
    assert np.all(np.isfinite(lse[fin])), f"{what}: non-finite LSE where the oracle is finite"
    err_o = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    err_l = float(np.max(np.abs(lse[fin] - lse_ref[fin]))) if fin.any() else 0.0
    print(f"{what}: O max-abs {err_o:.3e} (tol {O_TOL[dtype]:.0e}), O rel-L2 {rel_l2(o, o_ref):.3e}, "
          f"LSE max-abs {err_l:.3e}")
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    assert err_o <= O_TOL[dtype], f"{what}: O max-abs {err_o}"
    assert err_l <= LSE_TOL, f"{what}: LSE max-abs {err_l}"
    return err_o, err_l


def check_grads(grads_gpu, grads_ref, what=""):
    errs = []
    for name, g, r in zip(("dq", "dk", "dv"), grads_gpu, grads_ref):
        x = to64(g)
        assert np.all(np.isfinite(x)), f"{what}: non-finite {name}"
        e = rel_l2(x, r)
        errs.append(e)
    print(f"{what}: rel-L2 dq {errs[0]:.3e} dk {errs[1]:.3e} dv {errs[2]:.3e} (tol {GRAD_RTOL:.0e})")
    for name, e in zip(("dq", "dk", "dv"), errs):
        assert e <= GRAD_RTOL, f"{what}: {name} rel-L2 {e}"
    return errs
