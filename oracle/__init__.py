"""CPU float64 oracle for large-head-dim attention -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg may import
this package. The HIP library and its Python binding never do.
"""
from .ref import (  # noqa: F401
    attn_bwd, attn_fwd, fwd_rows, group_backward, group_forward, legal_mask, preprocess_delta,
    softmax_rows, varlen_bwd, varlen_fwd,
)
