"""MI355X (gfx950) large-head-dim fused attention.

The compute runs in libffpa.so (hand-written HIP kernels behind a C ABI, see include/ffpa.h);
this package is its ctypes binding plus autograd wrappers. PyTorch provides device memory and
streams only.
"""
from ._binding import (  # noqa: F401
    FFPA_ERR_HIP, FFPA_ERR_INVALID_ARGUMENT, FFPA_ERR_NOT_SUPPORTED, FFPA_ERR_TOO_LARGE, FFPA_OK,
    NOALLOC_SCRATCH_BYTES, choose_store_ds, ffpa_bwd, ffpa_bwd_fused_products, ffpa_bwd_stage, ffpa_bwd_workspace_bytes,
    ffpa_decode_fwd,
    ffpa_decode_fwd_noalloc, ffpa_decode_workspace_bytes, ffpa_fwd, ffpa_fwd_fp8, ffpa_fwd_fp8_workspace_bytes,
    ffpa_fwd_split_workspace_bytes, ffpa_status_string, ffpa_varlen_bwd, ffpa_varlen_bwd_workspace_bytes,
    ffpa_varlen_bwd_workspace_bytes_exact, ffpa_varlen_fwd, library_path, load_library,
)
from .attention import ffpa_attn_func, ffpa_attn_varlen_func  # noqa: F401
