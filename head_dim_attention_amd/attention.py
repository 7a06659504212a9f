"""Autograd entry points over the C ABI: the SDPA-style dense call and the packed varlen call.

ffpa_attn_func mirrors the dense entry point of the ffpa-attn user guide ("Backends Overview",
section "Choosing a backend": o = ffpa_attn_func(q, k, v), backward through autograd), and
ffpa_attn_varlen_func mirrors its FlashAttention-style varlen call ("CuTe-DSL Backend", section
"Varlen (packed THD) API": returns (out, lse) with return_lse=True). Both run only the library's
HIP kernels.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _binding as B

__all__ = ["ffpa_attn_func", "ffpa_attn_varlen_func"]


# Queries per head below which the forward takes the split-KV decode path ("Backends Overview",
# "Automatic SDPA fallback": Nq in [1, 8) uses the native decode path).
DECODE_MAX_NQ = 8


class _FFPAAttn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal, scale, mask):
        ctx.set_materialize_grads(False)  # an unused O or LSE gets None, not a zero tensor
        if mask is not None:
            if any(ctx.needs_input_grad[:3]):
                # The masked backward stores P and dS: fail before the forward when its workspace
                # can never fit on this device.
                total = torch.cuda.get_device_properties(q.device).total_memory
                B.masked_bwd_workspace_check(q.shape[0], q.shape[1], q.shape[2], k.shape[2], q.device, total)
            o, lse = B.ffpa_fwd(q, k, v, causal=causal, scale=scale, attn_mask=mask)
        else:
            fwd = B.ffpa_decode_fwd if q.shape[2] < DECODE_MAX_NQ else B.ffpa_fwd
            o, lse = fwd(q, k, v, causal=causal, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse, mask)
        ctx.causal, ctx.scale = causal, scale
        return o, lse

    @staticmethod
    def backward(ctx, do, dlse):
        # The returned LSE is differentiable: its gradient enters the preprocess stage
        # (delta = rowsum(dO * O) - dLSE) inside the library.
        q, k, v, o, lse, mask = ctx.saved_tensors
        if do is None:
            do = torch.zeros_like(o)
        if mask is None:
            dq, dk, dv = B.ffpa_bwd(q, k, v, o, do, lse, causal=ctx.causal, scale=ctx.scale, dlse=dlse)
            return dq, dk, dv, None, None, None
        want = ctx.needs_input_grad[5] and mask.dtype != torch.bool
        g = B.ffpa_bwd(q, k, v, o, do, lse, causal=ctx.causal, scale=ctx.scale, attn_mask=mask, mask_grad=want,
                       dlse=dlse)
        return g[0], g[1], g[2], None, None, (g[3] if want else None)


class _FFPAVarlen(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, cu_q, cu_k, max_q, max_k, causal, scale):
        ctx.set_materialize_grads(False)
        o, lse = B.ffpa_varlen_fwd(q, k, v, cu_q, cu_k, max_q, max_k, causal=causal, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse, cu_q, cu_k)
        # Host copies of the (validated) lengths size the backward's P/dS workspace exactly.
        host = (cu_q.detach().to("cpu").tolist(), cu_k.detach().to("cpu").tolist()) if any(ctx.needs_input_grad[:3]) \
            else None
        ctx.meta = (max_q, max_k, causal, scale, host)
        return o, lse

    @staticmethod
    def backward(ctx, do, dlse):
        q, k, v, o, lse, cu_q, cu_k = ctx.saved_tensors
        max_q, max_k, causal, scale, host = ctx.meta
        if do is None:
            do = torch.zeros_like(o)
        dq, dk, dv = B.ffpa_varlen_bwd(q, k, v, o, do, lse, cu_q, cu_k, max_q, max_k, causal=causal,
                                       scale=scale, validate=False, dlse=dlse, cu_seqlens_host=host)
        return dq, dk, dv, None, None, None, None, None, None


def ffpa_attn_func(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, attn_mask: Optional[torch.Tensor] = None,
                   is_causal: bool = False, scale: Optional[float] = None, return_lse: bool = False):
    """Attention over dense [B, H, N, D] tensors (fp16/bf16, D in 320..1024, D % 32 == 0).

    Causal masking is bottom-right aligned; Hq may be any multiple of Hkv (GQA/MQA). attn_mask:
    None, a bool mask (True keeps the key) or an additive bias in q's dtype, broadcastable to
    [B, Hq, Nq, Nkv] ("Triton Backend", "Feature support"); an additive mask that requires grad
    gets its gradient reduced to its own shape.
    """
    o, lse = _FFPAAttn.apply(q, k, v, bool(is_causal), scale, attn_mask)
    return (o, lse) if return_lse else o


def ffpa_attn_varlen_func(q, k, v, cu_seqlens_q, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None,
                          causal: bool = False, scale: Optional[float] = None, return_lse: bool = False):
    """Attention over packed [T, H, D] tensors with int32 cu_seqlens [B+1] (None for k means the q ones)."""
    if cu_seqlens_k is None:
        cu_seqlens_k = cu_seqlens_q
    if max_seqlen_q is None or max_seqlen_k is None:
        lq = (cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max().item()
        lk = (cu_seqlens_k[1:] - cu_seqlens_k[:-1]).max().item()
        max_seqlen_q = lq if max_seqlen_q is None else max_seqlen_q
        max_seqlen_k = lk if max_seqlen_k is None else max_seqlen_k
    o, lse = _FFPAVarlen.apply(q, k, v, cu_seqlens_q, cu_seqlens_k, int(max_seqlen_q), int(max_seqlen_k),
                               bool(causal), scale)
    return (o, lse) if return_lse else o
