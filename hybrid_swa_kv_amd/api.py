"""Python binding of the C ABI: torch tensors in, torch tensors out.

Argument marshalling only: shape/dtype/device checks, output and workspace
allocation through torch, raw pointers and torch's current HIP stream handed to
libhybrid_swa_kv.so.  Every arithmetic step runs in the library's kernels.  A
non-zero status raises RuntimeError with the library's message.
"""

from __future__ import annotations

import math

import torch

from . import _lib

F32, BF16 = 0, 1


def _check(rc: int) -> None:
    if rc != 0:
        msg = _lib.load().hsk_strerror(rc).decode()
        raise RuntimeError(f"hybrid_swa_kv error {rc}: {msg}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _out(t, name, dtype, shape, device):
    """A caller-supplied output must be exactly what the kernel writes (a contiguous
    GPU tensor of this dtype and shape); None allocates one."""
    shape = tuple(int(x) for x in shape)
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _need(t, name, dtype)
    if tuple(t.shape) != shape:
        raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
    return t


def _scratch(t, name, nbytes, device):
    """Workspace: a contiguous GPU tensor of at least nbytes (None allocates one)."""
    if t is None:
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    _need(t, name)
    return t


def _need(t, name, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def swa_prefill(q, k, v, window: int, scale: float | None = None, out=None, ring_k=None, ring_v=None,
                stream=None):
    """Sliding-window (window >= 1) or full causal (window <= 0) GQA prefill.

    q [B, L, Hq, D] or [L, Hq, D]; k, v [B, L, Hkv, D] (same rank); bf16 or fp32.
    Optional ring_k/ring_v [B, Hkv, W, D] receive the last W tokens' K/V at
    slot position mod W.  Returns out shaped like q.
    """
    squeeze = q.dim() == 3
    dtype = q.dtype
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, dtype, 3 if squeeze else 4)
    if dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("dtype must be bfloat16 or float32")
    B, L, Hq, D = (1, *q.shape) if squeeze else q.shape
    Hkv = k.shape[-2]
    out = _out(out, "out", q.dtype, q.shape, q.device)
    _need(out, "out", dtype)
    W = 0
    if ring_k is not None or ring_v is not None:
        _need(ring_k, "ring_k", dtype, 4)
        _need(ring_v, "ring_v", dtype, 4)
        W = ring_k.shape[2]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(_lib.load().swa_prefill(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, L, Hq, Hkv, D, int(window), scale,
        BF16 if dtype == torch.bfloat16 else F32, _ptr(ring_k), _ptr(ring_v), W, _stream(stream)))
    return out


def swa_decode_ring(q, k_new, v_new, ring_k, ring_v, pos, scale: float | None = None, out=None,
                    slot_out=None, stream=None):
    """Append each sequence's new K/V at slot pos mod W and attend the last W tokens.

    q [B, Hq, D]; k_new, v_new [B, Hkv, D]; ring_k, ring_v [B, Hkv, W, D] (bf16,
    updated in place); pos [B] int32.  Returns (out [B, Hq, D], slot_out [B] int32).
    """
    _need(q, "q", torch.bfloat16, 3)
    _need(k_new, "k_new", torch.bfloat16, 3)
    _need(v_new, "v_new", torch.bfloat16, 3)
    _need(ring_k, "ring_k", torch.bfloat16, 4)
    _need(ring_v, "ring_v", torch.bfloat16, 4)
    _need(pos, "pos", torch.int32, 1)
    B, Hq, D = q.shape
    Hkv, W = ring_k.shape[1], ring_k.shape[2]
    out = _out(out, "out", q.dtype, q.shape, q.device)
    slot_out = _out(slot_out, "slot_out", torch.int32, (B,), q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(_lib.load().swa_decode_ring(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(ring_k), _ptr(ring_v), _ptr(pos), _ptr(out), _ptr(slot_out),
        B, Hq, Hkv, D, W, scale, _stream(stream)))
    return out, slot_out


def kv_quant_int8_b32(x, codes=None, scales=None, stream=None):
    """INT8 block-wise encoding of x [B, Hkv, T, D] bf16 (T % 32 == 0).

    Returns (codes int8 [B, Hkv, T, D], scales float32 [B, Hkv, T/32]).
    """
    _need(x, "x", torch.bfloat16, 4)
    B, Hkv, T, D = x.shape
    codes = _out(codes, "codes", torch.int8, x.shape, x.device)
    scales = _out(scales, "scales", torch.float32, (B, Hkv, T // 32), x.device)
    _check(_lib.load().kv_quant_int8_b32(_ptr(x), _ptr(codes), _ptr(scales), B, Hkv, T, D, _stream(stream)))
    return codes, scales


def attn_decode_int8kv_workspace_size(B, Hq, Hkv, D, T8, Th) -> int:
    return int(_lib.load().attn_decode_int8kv_workspace_size(B, Hq, Hkv, D, T8, Th))


def attn_decode_int8kv(q, k_codes, k_scales, v_codes, v_scales, k_hot, v_hot, scale: float | None = None,
                       out=None, workspace=None, stream=None):
    """Decode one token over INT8 positions 0..T8-1 and bf16 positions T8..T8+Th-1.

    q [B, Hq, D] bf16; *_codes [B, Hkv, T8, D] int8; *_scales [B, Hkv, T8/32] fp32;
    *_hot [B, Hkv, Th, D] bf16.  Returns out [B, Hq, D] bf16.
    """
    _need(q, "q", torch.bfloat16, 3)
    _need(k_hot, "k_hot", torch.bfloat16, 4)
    _need(v_hot, "v_hot", torch.bfloat16, 4)
    B, Hq, D = q.shape
    Hkv, Th = k_hot.shape[1], k_hot.shape[2]
    T8 = 0 if k_codes is None else k_codes.shape[2]
    if T8 > 0:
        _need(k_codes, "k_codes", torch.int8, 4)
        _need(v_codes, "v_codes", torch.int8, 4)
        _need(k_scales, "k_scales", torch.float32, 3)
        _need(v_scales, "v_scales", torch.float32, 3)
    out = _out(out, "out", torch.bfloat16, q.shape, q.device)
    need = attn_decode_int8kv_workspace_size(B, Hq, Hkv, D, T8, Th)
    workspace = _scratch(workspace, "workspace", need, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(_lib.load().attn_decode_int8kv(
        _ptr(q), _ptr(k_codes) if T8 else None, _ptr(k_scales) if T8 else None,
        _ptr(v_codes) if T8 else None, _ptr(v_scales) if T8 else None, _ptr(k_hot), _ptr(v_hot),
        _ptr(out), B, Hq, Hkv, D, T8, Th, scale, _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out


def blocksparse_workspace_size(L, Hq, Hkv, D, block=64, topk=64) -> int:
    return int(_lib.load().blocksparse_workspace_size(L, Hq, Hkv, D, block, topk))


def blocksparse_select_attend(q, k, v, block: int = 64, topk: int = 64, window: int = 1024,
                              scale: float | None = None, out=None, sel=None, workspace=None, stream=None):
    """Top-k block selection plus attention over selected blocks and the local window.

    q [L, Hq, D], k, v [L, Hkv, D] bf16.  Returns (out [L, Hq, D] bf16,
    sel [Hq, L/block, topk] int32 ascending, -1 padded).
    """
    _need(q, "q", torch.bfloat16, 3)
    _need(k, "k", torch.bfloat16, 3)
    _need(v, "v", torch.bfloat16, 3)
    L, Hq, D = q.shape
    Hkv = k.shape[1]
    out = _out(out, "out", torch.bfloat16, q.shape, q.device)
    sel = _out(sel, "sel", torch.int32, (Hq, L // block, topk), q.device)
    need = blocksparse_workspace_size(L, Hq, Hkv, D, block, topk)
    workspace = _scratch(workspace, "workspace", need, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(_lib.load().blocksparse_select_attend(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(sel) if topk > 0 else None, L, Hq, Hkv, D, block, topk,
        window, scale, _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, sel


def swa_window_safe_len(slot_pos, match_len, out=None, stream=None):
    """Longest reusable prefix per sequence whose last W positions keep their SWA slots.

    slot_pos [B, W] int32 (position held by each slot, -1 empty); match_len [B]
    int32.  Returns safe_len [B] int32.
    """
    _need(slot_pos, "slot_pos", torch.int32, 2)
    _need(match_len, "match_len", torch.int32, 1)
    B, W = slot_pos.shape
    if match_len.shape[0] != B:
        raise ValueError("match_len must have one entry per sequence")
    out = _out(out, "out", torch.int32, (B,), slot_pos.device)
    _check(_lib.load().swa_window_safe_len(_ptr(slot_pos), _ptr(match_len), _ptr(out), B, W, _stream(stream)))
    return out


def swa_prefill_chunk(q, k, v, ring_k, ring_v, pos0: int, scale: float | None = None, out=None, stream=None):
    """Sliding-window prefill of a chunk at positions pos0 .. pos0+C-1, continuing from a ring.

    q [B, C, Hq, D]; k, v [B, C, Hkv, D]; ring_k, ring_v [B, Hkv, W, D] (bf16; on
    entry positions before pos0, updated in place to the last W positions).
    The window is the ring size W.  Returns out [B, C, Hq, D].
    """
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    _need(ring_k, "ring_k", torch.bfloat16, 4)
    _need(ring_v, "ring_v", torch.bfloat16, 4)
    B, C, Hq, D = q.shape
    Hkv, W = ring_k.shape[1], ring_k.shape[2]
    out = _out(out, "out", q.dtype, q.shape, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(_lib.load().swa_prefill_chunk(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(ring_k), _ptr(ring_v),
                                         B, C, Hq, Hkv, D, W, int(pos0), scale, _stream(stream)))
    return out


def kv_block_means_int8(codes, scales, means=None, stream=None):
    """K block means of INT8 codes [B, Hkv, T8, D] with scales [B, Hkv, T8/32].

    Returns means float32 [B, Hkv, D, T8/32] (d-major).
    """
    _need(codes, "codes", torch.int8, 4)
    _need(scales, "scales", torch.float32, 3)
    B, Hkv, T8, D = codes.shape
    means = _out(means, "means", torch.float32, (B, Hkv, D, T8 // 32), codes.device)
    _check(_lib.load().kv_block_means_int8(_ptr(codes), _ptr(scales), _ptr(means), B, Hkv, T8, D,
                                           _stream(stream)))
    return means


def attn_decode_int8kv_sparse_workspace_size(B, Hq, Hkv, D, T8, Th, topk) -> int:
    return int(_lib.load().attn_decode_int8kv_sparse_workspace_size(B, Hq, Hkv, D, T8, Th, topk))


def attn_decode_int8kv_sparse(q, k_codes, k_scales, v_codes, v_scales, k_means, k_hot, v_hot, topk: int = 64,
                              scale: float | None = None, out=None, sel=None, workspace=None, stream=None):
    """Decode over the bf16 hot tail and each head's top-k INT8 blocks (by q . block mean).

    Returns (out [B, Hq, D] bf16, sel [B, Hq, topk] int32).
    """
    _need(q, "q", torch.bfloat16, 3)
    _need(k_hot, "k_hot", torch.bfloat16, 4)
    _need(v_hot, "v_hot", torch.bfloat16, 4)
    B, Hq, D = q.shape
    Hkv, Th = k_hot.shape[1], k_hot.shape[2]
    T8 = 0 if k_codes is None else k_codes.shape[2]
    if T8:
        _need(k_codes, "k_codes", torch.int8, 4)
        _need(v_codes, "v_codes", torch.int8, 4)
        _need(k_scales, "k_scales", torch.float32, 3)
        _need(v_scales, "v_scales", torch.float32, 3)
        _need(k_means, "k_means", torch.float32, 4)
    out = _out(out, "out", torch.bfloat16, q.shape, q.device)
    sel = _out(sel, "sel", torch.int32, (B, Hq, topk), q.device)
    need = attn_decode_int8kv_sparse_workspace_size(B, Hq, Hkv, D, T8, Th, topk)
    workspace = _scratch(workspace, "workspace", need, q.device)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    opt = (lambda t: _ptr(t) if T8 else None)
    _check(_lib.load().attn_decode_int8kv_sparse(
        _ptr(q), opt(k_codes), opt(k_scales), opt(v_codes), opt(v_scales), opt(k_means), _ptr(k_hot), _ptr(v_hot),
        _ptr(out), _ptr(sel) if topk > 0 else None, B, Hq, Hkv, D, T8, Th, topk, scale, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out, sel
