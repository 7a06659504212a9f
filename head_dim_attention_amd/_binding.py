"""ctypes binding of libffpa.so: one Python function per C entry point, same names.

The functions only marshal arguments: they check tensor metadata, allocate outputs with PyTorch
(device memory), pass raw device pointers and the current HIP stream, and map status codes to
exceptions (INVALID_ARGUMENT -> ValueError, NOT_SUPPORTED -> NotImplementedError, HIP -> RuntimeError,
as the ffpa-attn user guide's "Backends Overview" and "CuTe-DSL Backend" pages describe the error
kinds). Every step of the computation runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional

import torch

__all__ = [
    "FFPA_OK", "FFPA_ERR_INVALID_ARGUMENT", "FFPA_ERR_NOT_SUPPORTED", "FFPA_ERR_HIP",
    "library_path", "load_library", "ffpa_status_string",
    "ffpa_fwd", "ffpa_bwd", "ffpa_bwd_stage", "ffpa_varlen_fwd", "ffpa_varlen_bwd",
    "ffpa_bwd_workspace_bytes", "ffpa_bwd_fused_products", "ffpa_varlen_bwd_workspace_bytes", "ffpa_varlen_bwd_workspace_bytes_exact",
    "ffpa_decode_fwd", "ffpa_decode_fwd_noalloc", "choose_store_ds",
    "ffpa_decode_workspace_bytes", "ffpa_fwd_fp8", "ffpa_fwd_fp8_workspace_bytes", "ffpa_fwd_split_workspace_bytes",
]

_i64p = ctypes.POINTER(ctypes.c_int64)

FFPA_OK = 0
FFPA_ERR_INVALID_ARGUMENT = 1
FFPA_ERR_NOT_SUPPORTED = 2
FFPA_ERR_HIP = 3
FFPA_ERR_TOO_LARGE = 4
# Fixed device scratch of ffpa_decode_fwd_noalloc (FFPA_NOALLOC_SCRATCH_BYTES in include/ffpa.h).
NOALLOC_SCRATCH_BYTES = 32 << 20

_DTYPES = {torch.bfloat16: 0, torch.float16: 1}
_LIB = None
_LOCK = threading.Lock()

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

_SIGNATURES = {
    "ffpa_fwd": [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp],
    "ffpa_decode_fwd": [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp, _sz, _vp],
    "ffpa_fwd_strided": [_vp] * 5 + [_i] * 6 + [_i64p, _i, _f, _i, _vp],
    "ffpa_fwd_masked": [_vp] * 5 + [_i] * 6 + [_vp, _i, _i64p, _i, _f, _i, _vp],
    "ffpa_fwd_fp8": [_vp] * 5 + [_i] * 7 + [_f, _i, _vp, _sz, _vp],
    "ffpa_fwd_split": [_vp] * 5 + [_i] * 7 + [_f, _i, _vp, _sz, _vp],
    "ffpa_bwd_masked": [_vp] * 11 + [_i] * 6 + [_vp, _i, _i64p, _vp, _i, _f, _i, _vp, _sz, _vp],
    "ffpa_decode_fwd_strided": [_vp] * 5 + [_i] * 6 + [_i64p, _i, _f, _i, _vp, _sz, _vp],
    "ffpa_decode_fwd_noalloc": [_vp] * 5 + [_i] * 7 + [_f, _i, _vp],
    "ffpa_bwd": [_vp] * 11 + [_i] * 7 + [_f, _i, _vp, _sz, _vp],
    "ffpa_bwd_stage": [_i] + [_vp] * 11 + [_i] * 7 + [_f, _i, _vp, _sz, _vp],
    "ffpa_varlen_fwd": [_vp] * 7 + [_i] * 9 + [_f, _i, _vp],
    "ffpa_varlen_bwd": [_vp] * 15 + [_i] * 9 + [_f, _i, _vp, _sz, _vp],
}
_SIZE_FUNCTIONS = {
    "ffpa_bwd_workspace_bytes": [_i] * 4,
    "ffpa_varlen_bwd_workspace_bytes": [_i] * 5,
    "ffpa_varlen_bwd_workspace_bytes_exact": [_i, _i, _vp, _vp, _i, _i, _i, _i],
    "ffpa_decode_workspace_bytes": [_i] * 6,
    "ffpa_fwd_fp8_workspace_bytes": [_i] * 6,
    "ffpa_fwd_split_workspace_bytes": [_i] * 6,
}


def library_path() -> str:
    return os.environ.get("FFPA_LIBRARY", os.path.join(os.path.dirname(os.path.abspath(__file__)), "libffpa.so"))


def load_library():
    """Load libffpa.so once; raise if it has not been built."""
    global _LIB
    with _LOCK:
        if _LIB is not None:
            return _LIB
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"libffpa.so not found at {path}; build it with "
                               "`python -m head_dim_attention_amd.build`")
        lib = ctypes.CDLL(path)
        for name, args in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        for name, args in _SIZE_FUNCTIONS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = _sz
        lib.ffpa_bwd_fused_products.argtypes = [_i] * 6
        lib.ffpa_bwd_fused_products.restype = ctypes.c_int
        lib.ffpa_status_string.argtypes = [ctypes.c_int]
        lib.ffpa_status_string.restype = ctypes.c_char_p
        _LIB = lib
        return lib


def ffpa_status_string(status: int) -> str:
    return load_library().ffpa_status_string(int(status)).decode()


def _raise_for(status: int, name: str) -> None:
    if status == FFPA_OK:
        return
    msg = f"{name}: {ffpa_status_string(status)}"
    if status in (FFPA_ERR_INVALID_ARGUMENT, FFPA_ERR_TOO_LARGE):
        raise ValueError(msg)
    if status == FFPA_ERR_NOT_SUPPORTED:
        raise NotImplementedError(msg)
    raise RuntimeError(msg)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise NotImplementedError(f"unsupported dtype {t.dtype}; ffpa kernels take float16 or bfloat16")
    return _DTYPES[t.dtype]


def _dev(t: torch.Tensor, what: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be a GPU tensor (got {t.device})")
    return t.contiguous()


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _scale(scale: Optional[float], d: int) -> float:
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def _same(ref: torch.Tensor, *ts):
    for t in ts:
        if t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError("q, k, v (and o, dout) must share dtype and device")


def _view(t: torch.Tensor, what: str) -> torch.Tensor:
    """A [B, H, N, D] GPU tensor the forward kernels can read in place (unit last stride, 16-byte
    aligned, other strides multiples of 8 elements, e.g. a [B, N, H, D] tensor transposed to
    [B, H, N, D] or a slice of a fused QKV tensor); anything else is copied to packed layout."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be a GPU tensor (got {t.device})")
    if t.dim() == 4 and t.stride(-1) == 1 and t.data_ptr() % 16 == 0 and \
            all(st % 8 == 0 and st >= 0 for sz, st in zip(t.shape[:-1], t.stride()[:-1]) if sz > 1):
        return t
    return t.contiguous()


def _strides(*ts) -> Optional[ctypes.Array]:
    """(batch, head, row) strides of each tensor for the strided entry points, or None when all
    are packed [B, H, N, D] (size-1 dims do not count)."""
    out = []
    packed = True
    for t in ts:
        for i in range(3):
            st = t.stride(i) if t.shape[i] > 1 else 0
            out.append(st)
        packed = packed and t.is_contiguous()
    return None if packed else (ctypes.c_int64 * 12)(*out)


def _fwd_prep(q, k, v):
    q, k, v = _view(q, "q"), _view(k, "k"), _view(v, "v")
    _same(q, k, v)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("expected q [B,Hq,Nq,D] and k, v [B,Hkv,Nkv,D]")
    b, hq, nq, d = q.shape
    _, hkv, nkv, dk = k.shape
    if k.shape[0] != b or dk != d:
        raise ValueError("batch and head dim of q, k, v must match")
    # O takes q's layout when q is a dense permutation (e.g. [B, N, H, D] viewed as [B, H, N, D]).
    o = torch.empty_like(q)
    if _view(o, "o") is not o:
        o = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    lse = torch.empty((b, hq, nq), dtype=torch.float32, device=q.device)
    return q, k, v, o, lse, (b, hq, hkv, nq, nkv, d)


MASK_ADDITIVE = 1
MASK_BOOL = 2


class _Mask:
    """An attn_mask prepared for the C ABI: a 4-d view (batch, head, query, key) whose dims are
    1 (broadcast, stride 0) or full, with unit key stride and rows of a multiple of 8 elements
    (copied into such a layout when the given tensor is not)."""

    def __init__(self, mask: torch.Tensor, q: torch.Tensor, nkv: int):
        if not isinstance(mask, torch.Tensor) or mask.device != q.device:
            raise ValueError("attn_mask must be a tensor on q's device")
        if mask.dtype == torch.bool:
            self.kind = MASK_BOOL
        elif mask.dtype == q.dtype:
            self.kind = MASK_ADDITIVE
        else:
            raise TypeError("attn_mask must be bool or have q's dtype")
        b, hq, nq, _ = q.shape
        full = (b, hq, nq, nkv)
        if mask.dim() > 4:
            raise ValueError("attn_mask must broadcast to [B, Hq, Nq, Nkv]")
        self.orig_shape = tuple(mask.shape)
        m = mask.reshape((1,) * (4 - mask.dim()) + self.orig_shape)
        for n, f in zip(m.shape, full):
            if n != 1 and n != f:
                raise ValueError(f"attn_mask of shape {self.orig_shape} does not broadcast to {full}")
        self.shape4 = tuple(m.shape)
        es = m.element_size()
        ok = (m.shape[3] == 1 or m.stride(3) == 1) and m.data_ptr() % (16 if es == 2 else 8) == 0 and \
            all(m.stride(i) % 8 == 0 for i in range(3) if m.shape[i] > 1)
        if not ok:
            kp = ((m.shape[3] + 7) // 8) * 8 if m.shape[3] > 1 else 1
            buf = torch.empty(self.shape4[:3] + (kp,), dtype=m.dtype, device=m.device)
            buf[..., :m.shape[3]] = m
            m = buf[..., :m.shape[3]]
        self.tensor = m
        self.strides = (ctypes.c_int64 * 4)(*[m.stride(i) if m.shape[i] > 1 else 0 for i in range(4)])


def ffpa_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
             scale: Optional[float] = None, attn_mask: Optional[torch.Tensor] = None, split: Optional[bool] = None):
    """Dense forward. q [B,Hq,Nq,D], k/v [B,Hkv,Nkv,D] -> (o [B,Hq,Nq,D], lse fp32 [B,Hq,Nq]).

    Strided views (for example [B, N, H, D] tensors transposed to [B, H, N, D], or the q, k, v
    slices of one fused QKV tensor) are read in place through ffpa_fwd_strided; o then takes q's
    layout when q is a dense permutation of [B, H, N, D].

    attn_mask: None, a bool tensor (True keeps the key) or an additive bias in q's dtype,
    broadcastable to [B, Hq, Nq, Nkv] (ffpa_fwd_masked; q, k, v then packed).

    split: packed inputs without a mask go through ffpa_fwd_split (key ranges merged by LSE, with a
    temporary workspace) when the library reports that the grid is too small to fill the GPU
    (None, the default) or never (False); the results agree up to fp32 summation order."""
    if attn_mask is not None:
        q, k, v = _dev(q, "q"), _dev(k, "k"), _dev(v, "v")
    q, k, v, o, lse, (b, hq, hkv, nq, nkv, d) = _fwd_prep(q, k, v)
    if attn_mask is not None:
        m = _Mask(attn_mask, q, nkv)
        st = load_library().ffpa_fwd_masked(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), b, hq, hkv, nq, nkv, d,
                                            _ptr(m.tensor), m.kind, m.strides, _dtype_code(q), _scale(scale, d),
                                            int(bool(causal)), _stream(q))
        _raise_for(st, "ffpa_fwd_masked")
        return o, lse
    strides = _strides(q, k, v, o)
    L = load_library()
    need = L.ffpa_fwd_split_workspace_bytes(b, hq, hkv, nq, nkv, d) if strides is None and split is not False else 0
    if need > 0:
        ws, nws = _workspace(need, q)
        st = L.ffpa_fwd_split(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), b, hq, hkv, nq, nkv, d,
                              _dtype_code(q), _scale(scale, d), int(bool(causal)), _ptr(ws), nws, _stream(q))
    elif strides is None:
        st = L.ffpa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), b, hq, hkv, nq, nkv, d,
                        _dtype_code(q), _scale(scale, d), int(bool(causal)), _stream(q))
    else:
        st = L.ffpa_fwd_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), b, hq, hkv, nq, nkv, d, strides,
                                _dtype_code(q), _scale(scale, d), int(bool(causal)), _stream(q))
    _raise_for(st, "ffpa_fwd")
    return o, lse


def ffpa_fwd_split_workspace_bytes(batch: int, hq: int, hkv: int, nq: int, nkv: int, d: int) -> int:
    """Bytes of the key-range split forward's workspace; 0 when the grid needs no split."""
    return int(load_library().ffpa_fwd_split_workspace_bytes(int(batch), int(hq), int(hkv), int(nq), int(nkv), int(d)))


def ffpa_decode_workspace_bytes(batch: int, hq: int, hkv: int, nq: int, nkv: int, d: int) -> int:
    """Bytes of the split-KV decode workspace (partial O and LSE per key range)."""
    return int(load_library().ffpa_decode_workspace_bytes(int(batch), int(hq), int(hkv), int(nq), int(nkv), int(d)))


def ffpa_decode_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                    scale: Optional[float] = None):
    """Split-KV decode forward (meant for Nq in [1, 8)); same shapes, results and strided views as
    ffpa_fwd."""
    q, k, v, o, lse, (b, hq, hkv, nq, nkv, d) = _fwd_prep(q, k, v)
    strides = _strides(q, k, v, o)
    ws, nws = _workspace(ffpa_decode_workspace_bytes(b, hq, hkv, nq, nkv, d), q)
    L = load_library()
    if strides is None:
        st = L.ffpa_decode_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), b, hq, hkv, nq, nkv, d,
                               _dtype_code(q), _scale(scale, d), int(bool(causal)), _ptr(ws), nws, _stream(q))
    else:
        st = L.ffpa_decode_fwd_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), b, hq, hkv, nq, nkv, d,
                                       strides, _dtype_code(q), _scale(scale, d), int(bool(causal)), _ptr(ws),
                                       nws, _stream(q))
    _raise_for(st, "ffpa_decode_fwd")
    return o, lse


def ffpa_decode_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                            scale: Optional[float] = None, out=None):
    """ffpa_decode_fwd through the library's fixed scratch (no workspace allocation). Packed
    [B, H, N, D] inputs; ``out`` = (o, lse) preallocated outputs (then this call allocates nothing
    at all), else they are allocated here. Sizes whose decode workspace exceeds
    NOALLOC_SCRATCH_BYTES raise ValueError. Calls that overlap on one GPU race on the scratch."""
    q, k, v = _dev(q, "q"), _dev(k, "k"), _dev(v, "v")
    _same(q, k, v)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("expected q [B,Hq,Nq,D] and k, v [B,Hkv,Nkv,D]")
    b, hq, nq, d = q.shape
    _, hkv, nkv, _ = k.shape
    if out is None:
        o = torch.empty_like(q)
        lse = torch.empty((b, hq, nq), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        if not (o.is_contiguous() and o.shape == q.shape and o.dtype == q.dtype and lse.is_contiguous()
                and lse.shape == (b, hq, nq) and lse.dtype == torch.float32):
            raise ValueError("out must be contiguous (o like q, lse float32 [B,Hq,Nq])")
    st = load_library().ffpa_decode_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), b, hq, hkv, nq, nkv,
                                                d, _dtype_code(q), _scale(scale, d), int(bool(causal)), _stream(q))
    _raise_for(st, "ffpa_decode_fwd_noalloc")
    return o, lse


def ffpa_fwd_fp8_workspace_bytes(batch: int, hq: int, hkv: int, nq: int, nkv: int, d: int) -> int:
    """Bytes of the FP8 forward's workspace (per-head amax, K8, transposed V8); 0: not available."""
    return int(load_library().ffpa_fwd_fp8_workspace_bytes(int(batch), int(hq), int(hkv), int(nq), int(nkv), int(d)))


def ffpa_fwd_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                 scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None):
    """FP8 forward (D 320..1024): fp16/bf16 q [B,Hq,Nq,D], k/v [B,Hkv,Nkv,D] quantized to e4m3 inside
    the library with one scale per head and tensor -> (o, lse) as ffpa_fwd. ``workspace`` (a byte
    tensor of at least ffpa_fwd_fp8_workspace_bytes()) keeps the quantized K8, V8^T and amax
    values for inspection; by default a temporary one is allocated."""
    q, k, v = _dev(q, "q"), _dev(k, "k"), _dev(v, "v")
    _same(q, k, v)
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("expected q [B,Hq,Nq,D] and k, v [B,Hkv,Nkv,D]")
    b, hq, nq, d = q.shape
    _, hkv, nkv, dk = k.shape
    if k.shape[0] != b or dk != d:
        raise ValueError("batch and head dim of q, k, v must match")
    o = torch.empty_like(q)
    lse = torch.empty((b, hq, nq), dtype=torch.float32, device=q.device)
    need = ffpa_fwd_fp8_workspace_bytes(b, hq, hkv, nq, nkv, d)
    if workspace is None:
        workspace, nws = _workspace(need, q)
    else:
        workspace = _dev(workspace, "workspace")
        nws = workspace.numel() * workspace.element_size()
    st = load_library().ffpa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), b, hq, hkv, nq, nkv, d,
                                     _dtype_code(q), _scale(scale, d), int(bool(causal)), _ptr(workspace), nws,
                                     _stream(q))
    _raise_for(st, "ffpa_fwd_fp8")
    return o, lse


def fp8_workspace_views(ws: torch.Tensor, b: int, hq: int, hkv: int, nkv: int, d: int):
    """(amax_q [B,Hq], amax_k [B,Hkv], amax_v [B,Hkv], K8 [B,Hkv,Nkv,D] uint8, V8T [B,Hkv,D,np] uint8)
    views of a filled FP8 workspace (the layout documented with ffpa_fwd_fp8 in include/ffpa.h)."""
    al = lambda x: (x + 255) // 256 * 256
    np_ = (nkv + 63) // 64 * 64
    k8_off = al((b * hq + 2 * b * hkv) * 4)
    v8_off = k8_off + al(b * hkv * nkv * d)
    am = ws[: (b * hq + 2 * b * hkv) * 4].view(torch.float32)
    return (am[: b * hq].view(b, hq), am[b * hq: b * hq + b * hkv].view(b, hkv), am[b * hq + b * hkv:].view(b, hkv),
            ws[k8_off: k8_off + b * hkv * nkv * d].view(b, hkv, nkv, d),
            ws[v8_off: v8_off + b * hkv * d * np_].view(b, hkv, d, np_))


def ffpa_bwd_fused_products(batch: int, hq: int, hkv: int, nq: int, nkv: int, d: int) -> bool:
    """Whether ffpa_bwd with a P/dS workspace forms dK, dV and dQ in one launch (stage 5)."""
    return bool(load_library().ffpa_bwd_fused_products(int(batch), int(hq), int(hkv), int(nq), int(nkv), int(d)))


def ffpa_bwd_workspace_bytes(batch: int, hq: int, nq: int, nkv: int) -> int:
    """Bytes of the optional P/dS workspace of the dense backward (0: not available)."""
    return int(load_library().ffpa_bwd_workspace_bytes(int(batch), int(hq), int(nq), int(nkv)))


def ffpa_varlen_bwd_workspace_bytes(hq: int, total_q: int, total_k: int, max_seqlen_q: int,
                                    max_seqlen_k: int) -> int:
    """Bytes of the optional P/dS workspace of the varlen backward (0: not available)."""
    return int(load_library().ffpa_varlen_bwd_workspace_bytes(int(hq), int(total_q), int(total_k),
                                                               int(max_seqlen_q), int(max_seqlen_k)))


def ffpa_varlen_bwd_workspace_bytes_exact(hq: int, cu_seqlens_q_host, cu_seqlens_k_host, total_q: int, total_k: int,
                                          max_seqlen_q: int, max_seqlen_k: int) -> int:
    """Exact bytes of the varlen P/dS workspace for these (host) cu_seqlens lists (k None: the q
    ones); 0 when they are invalid or the workspace is not available."""
    cq = (ctypes.c_int32 * len(cu_seqlens_q_host))(*cu_seqlens_q_host)
    ck = (ctypes.c_int32 * len(cu_seqlens_k_host))(*cu_seqlens_k_host) if cu_seqlens_k_host is not None else None
    return int(load_library().ffpa_varlen_bwd_workspace_bytes_exact(
        int(hq), len(cu_seqlens_q_host) - 1, ctypes.cast(cq, ctypes.c_void_p),
        ctypes.cast(ck, ctypes.c_void_p) if ck is not None else None, int(total_q), int(total_k),
        int(max_seqlen_q), int(max_seqlen_k)))


# Memory kept free beside a P/dS workspace when the backward decides whether to store P and dS.
DS_HEADROOM_BYTES = 1 << 30


def choose_store_ds(need: int, available: int, headroom: int = DS_HEADROOM_BYTES) -> bool:
    """Whether the backward stores P and dS: the workspace exists for these sizes (need > 0) and
    fits in the device memory available to the caller with `headroom` bytes to spare; otherwise
    the O(N)-memory recomputing kernels run."""
    return 0 < need and need + headroom <= available


def _available_bytes(dev: torch.device) -> int:
    """Device memory a new allocation can use: free on the device plus what PyTorch's caching
    allocator holds unused."""
    free, _ = torch.cuda.mem_get_info(dev)
    return int(free) + int(torch.cuda.memory_reserved(dev) - torch.cuda.memory_allocated(dev))


def _workspace(nbytes: int, like: torch.Tensor):
    """Device workspace of nbytes (None when nbytes is 0), and its size to pass."""
    if nbytes <= 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=like.device), nbytes


def _dlse_arg(dlse, lse):
    """The LSE gradient as a contiguous float32 tensor shaped like lse, or None."""
    if dlse is None:
        return None
    dlse = _dev(dlse, "dlse")
    if dlse.shape != lse.shape:
        raise ValueError(f"dlse must have lse's shape {tuple(lse.shape)}")
    return dlse.float().contiguous()


def ffpa_bwd(q, k, v, o, dout, lse, causal: bool = False, scale: Optional[float] = None,
             store_ds: Optional[bool] = None, attn_mask: Optional[torch.Tensor] = None, mask_grad: bool = False,
             dlse: Optional[torch.Tensor] = None):
    """Dense backward -> (dq, dk, dv) with the shapes and dtype of q, k, v.

    store_ds: True stores P and dS in a temporary workspace of ffpa_bwd_workspace_bytes() bytes so
    that dK = scale dS^T Q, dV = P^T dO and dQ = scale dS K are products instead of
    recomputations; False recomputes (O(N) memory); None (default) stores them when the workspace
    fits in the free device memory with DS_HEADROOM_BYTES to spare (choose_store_ds).
    attn_mask: the forward's mask (ffpa_bwd_masked, always with the workspace: a MemoryError when it
    does not fit); with mask_grad (additive masks) the result is (dq, dk, dv, dmask), dmask with the
    mask's shape.
    dlse: the gradient of the returned LSE (float32, lse's shape) or None; the loss is then
    sum(dout * o) + sum(dlse * lse).
    """
    if attn_mask is not None:
        return _bwd_masked(q, k, v, o, dout, lse, causal, scale, attn_mask, mask_grad, dlse)
    q, k, v, o, dout = (_dev(x, n) for x, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")))
    lse = _dev(lse, "lse")
    dlse = _dlse_arg(dlse, lse)
    _same(q, k, v, o, dout)
    b, hq, nq, d = q.shape
    _, hkv, nkv, _ = k.shape
    if o.shape != q.shape or dout.shape != q.shape or lse.shape != (b, hq, nq) or lse.dtype != torch.float32:
        raise ValueError("o and dout must match q; lse must be float32 [B,Hq,Nq]")
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    delta = torch.empty((b, hq, nq), dtype=torch.float32, device=q.device)
    need = ffpa_bwd_workspace_bytes(b, hq, nq, nkv)
    if store_ds is None:
        store_ds = choose_store_ds(need, _available_bytes(q.device))
    ws, nws = _workspace(need if store_ds else 0, q)
    st = load_library().ffpa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dlse), _ptr(delta),
                                 _ptr(dq), _ptr(dk), _ptr(dv), b, hq, hkv, nq, nkv, d,
                                 _dtype_code(q), _scale(scale, d), int(bool(causal)), _ptr(ws), nws, _stream(q))
    _raise_for(st, "ffpa_bwd")
    return dq, dk, dv


def masked_bwd_workspace_check(b: int, hq: int, nq: int, nkv: int, dev: torch.device, available: Optional[int] = None):
    """The masked backward always stores P and dS: raise MemoryError (before anything is launched
    or allocated) when its workspace does not fit in the device memory (`available` bytes, default
    the free memory now)."""
    need = ffpa_bwd_workspace_bytes(b, hq, nq, nkv)
    if need == 0:
        raise NotImplementedError("the attn_mask backward needs a P/dS workspace, which is not available for "
                                  f"nq={nq}, nkv={nkv} (a head's block above 2^31 bytes)")
    have = _available_bytes(dev) if available is None else int(available)
    if need > have:
        raise MemoryError(f"the attn_mask backward needs a {need / 2**30:.2f} GiB P/dS workspace; "
                          f"only {have / 2**30:.2f} GiB of device memory is available")
    return need


def _bwd_masked(q, k, v, o, dout, lse, causal, scale, attn_mask, mask_grad, dlse=None):
    q, k, v, o, dout = (_dev(x, n) for x, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")))
    lse = _dev(lse, "lse")
    dlse = _dlse_arg(dlse, lse)
    _same(q, k, v, o, dout)
    b, hq, nq, d = q.shape
    _, hkv, nkv, _ = k.shape
    if o.shape != q.shape or dout.shape != q.shape or lse.shape != (b, hq, nq) or lse.dtype != torch.float32:
        raise ValueError("o and dout must match q; lse must be float32 [B,Hq,Nq]")
    m = _Mask(attn_mask, q, nkv)
    if mask_grad and m.kind != MASK_ADDITIVE:
        raise ValueError("only an additive attn_mask has a gradient")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((b, hq, nq), dtype=torch.float32, device=q.device)
    dm = torch.empty(m.shape4, dtype=q.dtype, device=q.device) if mask_grad else None
    ws, nws = _workspace(masked_bwd_workspace_check(b, hq, nq, nkv, q.device), q)
    st = load_library().ffpa_bwd_masked(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dlse),
                                        _ptr(delta),
                                        _ptr(dq), _ptr(dk), _ptr(dv), b, hq, hkv, nq, nkv, d, _ptr(m.tensor),
                                        m.kind, m.strides, _ptr(dm), _dtype_code(q), _scale(scale, d),
                                        int(bool(causal)), _ptr(ws), nws, _stream(q))
    _raise_for(st, "ffpa_bwd_masked")
    if not mask_grad:
        return dq, dk, dv
    return dq, dk, dv, dm.reshape(m.orig_shape)


def ffpa_bwd_stage(stage: int, q, k, v, o, dout, lse, delta, dq, dk, dv, causal: bool = False,
                   scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
                   dlse: Optional[torch.Tensor] = None):
    """Run one backward stage (0 preprocess, 4 P and dS, 1 dK, 2 dV, 3 dQ, 5 dK + dV + dQ in one
    launch, workspace only) into caller buffers.

    ffpa_bwd runs the stages in the order 0, 4, 1, 2, 3 (0, 4, 5 when ffpa_bwd_fused_products()). All tensors must be contiguous GPU tensors
    with ffpa_bwd's shapes; delta is float32 [B,Hq,Nq]. workspace: optional P/dS workspace (a GPU
    tensor of at least ffpa_bwd_workspace_bytes() bytes), the same for stages 4, 1, 2 and 3: stage 4
    fills it, and stages 1, 2 and 3 read it. Without a workspace stage 4
    launches nothing and stages 1-3 recompute. dlse (stage 0 only reads it): as in ffpa_bwd.
    """
    if dlse is not None:
        dlse = _dlse_arg(dlse, lse)
    if workspace is not None and not (isinstance(workspace, torch.Tensor) and workspace.device.type == "cuda"
                                      and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous GPU tensor")
    for x, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (lse, "lse"), (delta, "delta"),
                 (dq, "dq"), (dk, "dk"), (dv, "dv")):
        if not (isinstance(x, torch.Tensor) and x.device.type == "cuda" and x.is_contiguous()):
            raise ValueError(f"{n} must be a contiguous GPU tensor")
    b, hq, nq, d = q.shape
    _, hkv, nkv, _ = k.shape
    nws = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load_library().ffpa_bwd_stage(int(stage), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                       _ptr(dlse), _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv), b, hq, hkv, nq, nkv, d,
                                       _dtype_code(q), _scale(scale, d), int(bool(causal)), _ptr(workspace), nws,
                                       _stream(q))
    _raise_for(st, "ffpa_bwd_stage")


def _check_cu(cu: torch.Tensor, total: int, what: str) -> list[int]:
    if cu.dtype != torch.int32 or cu.dim() != 1 or cu.numel() < 2:
        raise ValueError(f"{what} must be int32 [batch+1]")
    host = cu.detach().to("cpu").tolist()
    if host[0] != 0 or any(b < a for a, b in zip(host, host[1:])) or host[-1] != total:
        raise ValueError(f"{what} must start at 0, be non-decreasing and end at {total}")
    return host


def _varlen_meta(q, k, cu_q, cu_k, max_q, max_k, validate, host=None):
    """(cu_k, max_q, max_k, host lists or None). With validate the host copies of cu_seqlens are
    checked (and returned); ``host`` passes lists the caller already checked."""
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("varlen expects packed q [Tq,Hq,D] and k, v [Tk,Hkv,D]")
    tq, tk = q.shape[0], k.shape[0]
    if cu_k is None:
        if tk != tq:
            raise ValueError("cu_seqlens_k is required when k and q have different total lengths")
        cu_k = cu_q
    if validate:
        hq_ = _check_cu(cu_q, tq, "cu_seqlens_q")
        hk_ = _check_cu(cu_k, tk, "cu_seqlens_k")
        if len(hq_) != len(hk_):
            raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
        lq = [b - a for a, b in zip(hq_, hq_[1:])]
        lk = [b - a for a, b in zip(hk_, hk_[1:])]
        if max_q is None:
            max_q = max(lq)
        if max_k is None:
            max_k = max(lk)
        if max(lq) > max_q or max(lk) > max_k:
            raise ValueError("max_seqlen_q / max_seqlen_k smaller than a sequence length")
        host = (hq_, hk_)
    if max_q is None or max_k is None:
        raise ValueError("max_seqlen_q and max_seqlen_k are required when validate=False")
    return cu_k, int(max_q), int(max_k), host


def ffpa_varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None,
                    causal: bool = False, scale: Optional[float] = None, validate: bool = True):
    """Packed forward. q [Tq,Hq,D], k/v [Tk,Hkv,D] -> (o [Tq,Hq,D], lse fp32 [Hq,Tq])."""
    q, k, v = _dev(q, "q"), _dev(k, "k"), _dev(v, "v")
    _same(q, k, v)
    cu_q = _dev(cu_seqlens_q, "cu_seqlens_q")
    cu_k = _dev(cu_seqlens_k, "cu_seqlens_k") if cu_seqlens_k is not None else None
    cu_k, max_q, max_k, _ = _varlen_meta(q, k, cu_q, cu_k, max_seqlen_q, max_seqlen_k, validate)
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    o = torch.empty_like(q)
    lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    st = load_library().ffpa_varlen_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_q), _ptr(cu_k),
                                        cu_q.numel() - 1, max_q, max_k, tq, tk, hq, hkv, d, _dtype_code(q),
                                        _scale(scale, d), int(bool(causal)), _stream(q))
    _raise_for(st, "ffpa_varlen_fwd")
    return o, lse


def ffpa_varlen_bwd(q, k, v, o, dout, lse, cu_seqlens_q, cu_seqlens_k=None, max_seqlen_q=None,
                    max_seqlen_k=None, causal: bool = False, scale: Optional[float] = None,
                    validate: bool = True, store_ds: Optional[bool] = None, dlse: Optional[torch.Tensor] = None,
                    cu_seqlens_host=None):
    """Packed backward -> (dq [Tq,Hq,D], dk [Tk,Hkv,D], dv [Tk,Hkv,D]). store_ds and dlse ([Hq,Tq])
    as in ffpa_bwd. With host copies of cu_seqlens (validate=True makes them, or pass
    cu_seqlens_host=(list_q, list_k) already checked) the P/dS workspace has the exact size of these
    sequences (ffpa_varlen_bwd_workspace_bytes_exact) instead of the bound for any lengths."""
    q, k, v, o, dout = (_dev(x, n) for x, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")))
    lse = _dev(lse, "lse")
    _same(q, k, v, o, dout)
    cu_q = _dev(cu_seqlens_q, "cu_seqlens_q")
    cu_k = _dev(cu_seqlens_k, "cu_seqlens_k") if cu_seqlens_k is not None else None
    cu_k, max_q, max_k, host = _varlen_meta(q, k, cu_q, cu_k, max_seqlen_q, max_seqlen_k, validate,
                                            cu_seqlens_host)
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    if o.shape != q.shape or dout.shape != q.shape or lse.shape != (hq, tq) or lse.dtype != torch.float32:
        raise ValueError("o and dout must match q; lse must be float32 [Hq,Tq]")
    dlse = _dlse_arg(dlse, lse)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    delta = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    hq_arr = hk_arr = None
    if host is not None:
        hq_arr = (ctypes.c_int32 * len(host[0]))(*host[0])
        hk_arr = (ctypes.c_int32 * len(host[1]))(*host[1])
        need = ffpa_varlen_bwd_workspace_bytes_exact(hq, host[0], host[1], tq, tk, max_q, max_k)
    else:
        need = ffpa_varlen_bwd_workspace_bytes(hq, tq, tk, max_q, max_k)
    if store_ds is None:
        store_ds = choose_store_ds(need, _available_bytes(q.device))
    ws, nws = _workspace(need if store_ds else 0, q)
    vp = lambda a: ctypes.cast(a, ctypes.c_void_p) if a is not None else ctypes.c_void_p(0)
    st = load_library().ffpa_varlen_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dlse),
                                        _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(cu_q), _ptr(cu_k),
                                        vp(hq_arr), vp(hk_arr), cu_q.numel() - 1, max_q, max_k, tq, tk, hq, hkv,
                                        d, _dtype_code(q), _scale(scale, d), int(bool(causal)), _ptr(ws), nws,
                                        _stream(q))
    _raise_for(st, "ffpa_varlen_bwd")
    return dq, dk, dv
