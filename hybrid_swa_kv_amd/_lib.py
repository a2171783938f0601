"""ctypes loader for libhybrid_swa_kv.so (argument types only, no logic)."""

from __future__ import annotations

import ctypes
import os

# the in-tree build; HYBRID_SWA_KV_LIB names another build of the same sources
# (e.g. the host-sanitized one the ABI tests also run against)
LIB_PATH = os.environ.get("HYBRID_SWA_KV_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                              "libhybrid_swa_kv.so")
ABI_VERSION = 5  # the signatures below; hsk_abi_version() of the loaded library must match

# every symbol declared in include/hybrid_swa_kv.h
EXPORTS = (
    "hsk_strerror",
    "hsk_abi_version",
    "swa_prefill",
    "swa_decode_ring",
    "kv_quant_int8_b32",
    "attn_decode_int8kv",
    "attn_decode_int8kv_workspace_size",
    "attn_decode_int8kv_noalloc",
    "blocksparse_select_attend",
    "blocksparse_workspace_size",
    "swa_window_safe_len",
    "swa_prefill_chunk",
    "kv_block_means_int8",
    "attn_decode_int8kv_sparse",
    "attn_decode_int8kv_sparse_workspace_size",
)

_P, _I, _F, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

_SIGS = {
    "hsk_strerror": (ctypes.c_char_p, [_I]),
    "hsk_abi_version": (_I, []),
    "swa_prefill": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _I, _P]),
    "swa_decode_ring": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]),
    "kv_quant_int8_b32": (_I, [_P, _P, _P, _I, _I, _I, _I, _P]),
    "attn_decode_int8kv": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _S, _P]),
    "attn_decode_int8kv_workspace_size": (_S, [_I, _I, _I, _I, _I, _I]),
    "attn_decode_int8kv_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P]),
    "blocksparse_select_attend": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P, _S, _P]),
    "blocksparse_workspace_size": (_S, [_I, _I, _I, _I, _I, _I]),
    "swa_window_safe_len": (_I, [_P, _P, _P, _I, _I, _P]),
    "swa_prefill_chunk": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P]),
    "kv_block_means_int8": (_I, [_P, _P, _P, _I, _I, _I, _I, _P]),
    "attn_decode_int8kv_sparse": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F,
                                       _P, _S, _P]),
    "attn_decode_int8kv_sparse_workspace_size": (_S, [_I, _I, _I, _I, _I, _I, _I]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load the library once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m hybrid_swa_kv_amd.build` "
                "(the HIP library is the only implementation; there is no fallback)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        got = lib.hsk_abi_version()
        if got != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {got}, these bindings expect {ABI_VERSION}: "
                               "rebuild it with `python -m hybrid_swa_kv_amd.build`")
        _lib = lib
    return _lib
