"""Hybrid sliding-window / INT8 / block-sparse attention for MI355X (gfx950).

The kernels live in libhybrid_swa_kv.so (built from csrc/ by ``build.py``); the
functions below are a thin torch binding of its C ABI (include/hybrid_swa_kv.h).
Importing the package does not load the library; the first call does, and
raises if it is missing.
"""

from .api import (  # noqa: F401
    attn_decode_int8kv,
    attn_decode_int8kv_workspace_size,
    attn_decode_int8kv_noalloc,
    attn_decode_int8kv_sparse,
    attn_decode_int8kv_sparse_workspace_size,
    kv_block_means_int8,
    blocksparse_select_attend,
    blocksparse_workspace_size,
    kv_quant_int8_b32,
    swa_decode_ring,
    swa_prefill,
    swa_prefill_chunk,
    swa_window_safe_len,
)
