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


def _call(dev, name, *args):
    """Calls the library entry point `name` with `dev` as the current device (the
    kernels run there, on a stream of that device)."""
    with torch.cuda.device(dev):
        _check(getattr(_lib.load(), name)(*args))


def _stream(stream, dev):
    """torch's current stream of `dev`, or the caller's stream, which must belong to `dev`."""
    if stream is None:
        return torch.cuda.current_stream(dev).cuda_stream
    if stream.device != dev:
        raise ValueError(f"stream is on {stream.device}, the tensors on {dev}")
    return stream.cuda_stream


def _out(t, name, dtype, shape, device):
    """A caller-supplied output must be exactly what the kernel writes (a contiguous
    tensor of this dtype and shape on the inputs' GPU); None allocates one."""
    shape = tuple(int(x) for x in shape)
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _need(t, name, dtype, shape=shape)
    _same_device(device, t, name)
    return t


def _scratch(t, name, nbytes, device):
    """Workspace: a contiguous tensor of at least nbytes on the inputs' GPU (None
    allocates one)."""
    if t is None:
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    _need(t, name)
    _same_device(device, t, name)
    return t


def _need(t, name, dtype=None, ndim=None, shape=None):
    """Type, dtype, rank, exact shape and contiguity of one tensor argument.

    Every tensor the kernels read or write is checked against the sizes the call
    derives, so a short or mis-shaped buffer is refused here instead of being read
    or written past its end on the device.  The device is checked separately
    (``_device``), after all shapes, so shape errors read the same on any device.
    """
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(int(x) for x in shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _device(*named):
    """named: tensor, name, tensor, name, ... (None tensors are skipped).  Every
    tensor must be on a GPU, and all on the same one (a pointer from another
    device would be read by kernels that cannot reach it); returns that device."""
    dev = None
    for t, name in zip(named[::2], named[1::2]):
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")
    return dev


def _same_device(dev, t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")


def _blocks32(T, name):
    if T % 32 != 0:
        raise ValueError(f"{name} has {T} tokens, not a multiple of the 32-token block")
    return T // 32


def swa_prefill(q, k, v, window: int, scale: float | None = None, out=None, ring_k=None, ring_v=None,
                stream=None):
    """Sliding-window (window >= 1) or full causal (window <= 0) GQA prefill.

    q [B, L, Hq, D] or [L, Hq, D]; k, v [B, L, Hkv, D] (same rank); bf16 or fp32.
    Optional ring_k/ring_v [B, Hkv, W, D] receive the last W tokens' K/V at
    slot position mod W.  Returns out shaped like q.
    """
    if not isinstance(q, torch.Tensor):
        raise TypeError("q must be a torch.Tensor")
    squeeze = q.dim() == 3
    dtype = q.dtype
    if dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("dtype must be bfloat16 or float32")
    _need(q, "q", dtype, 3 if squeeze else 4)
    B, L, Hq, D = (1, *q.shape) if squeeze else q.shape
    _need(k, "k", dtype, q.dim())
    Hkv = k.shape[-2]
    kv_shape = (L, Hkv, D) if squeeze else (B, L, Hkv, D)
    _need(k, "k", dtype, shape=kv_shape)
    _need(v, "v", dtype, shape=kv_shape)
    W = 0
    if ring_k is not None or ring_v is not None:
        _need(ring_k, "ring_k", dtype, 4)
        W = ring_k.shape[2]
        _need(ring_k, "ring_k", dtype, shape=(B, Hkv, W, D))
        _need(ring_v, "ring_v", dtype, shape=(B, Hkv, W, D))
    dev = _device(q, "q", k, "k", v, "v", ring_k, "ring_k", ring_v, "ring_v")
    out = _out(out, "out", q.dtype, q.shape, dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _call(dev, "swa_prefill",
          _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, L, Hq, Hkv, D, int(window), scale,
          BF16 if dtype == torch.bfloat16 else F32, _ptr(ring_k), _ptr(ring_v), W, _stream(stream, dev))
    return out


def swa_decode_ring(q, k_new, v_new, ring_k, ring_v, pos, scale: float | None = None, out=None,
                    slot_out=None, stream=None):
    """Append each sequence's new K/V at slot pos mod W and attend the last W tokens.

    q [B, Hq, D]; k_new, v_new [B, Hkv, D]; ring_k, ring_v [B, Hkv, W, D] (bf16,
    updated in place); pos [B] int32.  Returns (out [B, Hq, D], slot_out [B] int32).
    """
    _need(q, "q", torch.bfloat16, 3)
    _need(ring_k, "ring_k", torch.bfloat16, 4)
    B, Hq, D = q.shape
    Hkv, W = ring_k.shape[1], ring_k.shape[2]
    _need(ring_k, "ring_k", torch.bfloat16, shape=(B, Hkv, W, D))
    _need(ring_v, "ring_v", torch.bfloat16, shape=(B, Hkv, W, D))
    _need(k_new, "k_new", torch.bfloat16, shape=(B, Hkv, D))
    _need(v_new, "v_new", torch.bfloat16, shape=(B, Hkv, D))
    _need(pos, "pos", torch.int32, shape=(B,))
    dev = _device(q, "q", k_new, "k_new", v_new, "v_new", ring_k, "ring_k", ring_v, "ring_v", pos, "pos")
    out = _out(out, "out", q.dtype, q.shape, dev)
    slot_out = _out(slot_out, "slot_out", torch.int32, (B,), dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _call(dev, "swa_decode_ring",
          _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(ring_k), _ptr(ring_v), _ptr(pos), _ptr(out), _ptr(slot_out),
          B, Hq, Hkv, D, W, scale, _stream(stream, dev))
    return out, slot_out


def kv_quant_int8_b32(x, codes=None, scales=None, stream=None):
    """INT8 block-wise encoding of x [B, Hkv, T, D] bf16 (T % 32 == 0).

    Returns (codes int8 [B, Hkv, T, D], scales float32 [B, Hkv, T/32]).
    """
    _need(x, "x", torch.bfloat16, 4)
    B, Hkv, T, D = x.shape
    nblk = _blocks32(T, "x")
    dev = _device(x, "x")
    codes = _out(codes, "codes", torch.int8, x.shape, dev)
    scales = _out(scales, "scales", torch.float32, (B, Hkv, nblk), dev)
    _call(dev, "kv_quant_int8_b32", _ptr(x), _ptr(codes), _ptr(scales), B, Hkv, T, D, _stream(stream, dev))
    return codes, scales


def attn_decode_int8kv_workspace_size(B, Hq, Hkv, D, T8, Th) -> int:
    return int(_lib.load().attn_decode_int8kv_workspace_size(B, Hq, Hkv, D, T8, Th))


def _int8_pool(q, k_codes, k_scales, v_codes, v_scales, k_hot, v_hot, k_means=None, with_means=False):
    """Checks the INT8 + bf16 pool arguments of the decodes; returns
    (B, Hq, Hkv, D, T8, Th, device)."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_hot, "k_hot", torch.bfloat16, 4)
    B, Hq, D = q.shape
    Hkv, Th = k_hot.shape[1], k_hot.shape[2]
    _need(k_hot, "k_hot", torch.bfloat16, shape=(B, Hkv, Th, D))
    _need(v_hot, "v_hot", torch.bfloat16, shape=(B, Hkv, Th, D))
    T8 = 0 if k_codes is None else int(k_codes.shape[2]) if k_codes.dim() == 4 else -1
    if k_codes is not None:
        _need(k_codes, "k_codes", torch.int8, 4)
    if T8 > 0:
        nblk = _blocks32(T8, "k_codes")
        _need(k_codes, "k_codes", torch.int8, shape=(B, Hkv, T8, D))
        _need(v_codes, "v_codes", torch.int8, shape=(B, Hkv, T8, D))
        _need(k_scales, "k_scales", torch.float32, shape=(B, Hkv, nblk))
        _need(v_scales, "v_scales", torch.float32, shape=(B, Hkv, nblk))
        if with_means:
            _need(k_means, "k_means", torch.float32, shape=(B, Hkv, D, nblk))
    cold = T8 > 0
    dev = _device(q, "q", k_hot, "k_hot", v_hot, "v_hot",
                  k_codes if cold else None, "k_codes", v_codes if cold else None, "v_codes",
                  k_scales if cold else None, "k_scales", v_scales if cold else None, "v_scales",
                  k_means if cold and with_means else None, "k_means")
    return B, Hq, Hkv, D, T8, Th, dev


def attn_decode_int8kv(q, k_codes, k_scales, v_codes, v_scales, k_hot, v_hot, scale: float | None = None,
                       out=None, workspace=None, stream=None):
    """Decode one token over INT8 positions 0..T8-1 and bf16 positions T8..T8+Th-1.

    q [B, Hq, D] bf16; *_codes [B, Hkv, T8, D] int8; *_scales [B, Hkv, T8/32] fp32;
    *_hot [B, Hkv, Th, D] bf16.  Returns out [B, Hq, D] bf16.
    """
    B, Hq, Hkv, D, T8, Th, dev = _int8_pool(q, k_codes, k_scales, v_codes, v_scales, k_hot, v_hot)
    out = _out(out, "out", torch.bfloat16, q.shape, dev)
    need = attn_decode_int8kv_workspace_size(B, Hq, Hkv, D, T8, Th)
    workspace = _scratch(workspace, "workspace", need, dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _call(dev, "attn_decode_int8kv",
          _ptr(q), _ptr(k_codes) if T8 else None, _ptr(k_scales) if T8 else None,
          _ptr(v_codes) if T8 else None, _ptr(v_scales) if T8 else None, _ptr(k_hot), _ptr(v_hot),
          _ptr(out), B, Hq, Hkv, D, T8, Th, scale, _ptr(workspace), workspace.numel() * workspace.element_size(),
          _stream(stream, dev))
    return out


def attn_decode_int8kv_noalloc(q, k_codes, k_scales, v_codes, v_scales, k_hot, v_hot, scale: float | None = None,
                               out=None, stream=None):
    """attn_decode_int8kv with the split records in the library's static device
    array (no workspace argument; nothing allocated when ``out`` is given).
    Calls that overlap on one GPU race on that array."""
    B, Hq, Hkv, D, T8, Th, dev = _int8_pool(q, k_codes, k_scales, v_codes, v_scales, k_hot, v_hot)
    out = _out(out, "out", torch.bfloat16, q.shape, dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _call(dev, "attn_decode_int8kv_noalloc",
          _ptr(q), _ptr(k_codes) if T8 else None, _ptr(k_scales) if T8 else None,
          _ptr(v_codes) if T8 else None, _ptr(v_scales) if T8 else None, _ptr(k_hot), _ptr(v_hot),
          _ptr(out), B, Hq, Hkv, D, T8, Th, scale, _stream(stream, dev))
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
    L, Hq, D = q.shape
    Hkv = k.shape[1]
    _need(k, "k", torch.bfloat16, shape=(L, Hkv, D))
    _need(v, "v", torch.bfloat16, shape=(L, Hkv, D))
    if block <= 0 or L % block != 0:
        raise ValueError(f"L = {L} must be a multiple of block = {block}")
    dev = _device(q, "q", k, "k", v, "v")
    out = _out(out, "out", torch.bfloat16, q.shape, dev)
    sel = _out(sel, "sel", torch.int32, (Hq, L // block, topk), dev)
    need = blocksparse_workspace_size(L, Hq, Hkv, D, block, topk)
    workspace = _scratch(workspace, "workspace", need, dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _call(dev, "blocksparse_select_attend",
          _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(sel) if topk > 0 else None, L, Hq, Hkv, D, block, topk,
          window, scale, _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, dev))
    return out, sel


def swa_window_safe_len(slot_pos, match_len, out=None, stream=None):
    """Longest reusable prefix per sequence whose last W positions keep their SWA slots.

    slot_pos [B, W] int32 (position held by each slot, -1 empty); match_len [B]
    int32.  Returns safe_len [B] int32.
    """
    _need(slot_pos, "slot_pos", torch.int32, 2)
    B, W = slot_pos.shape
    _need(match_len, "match_len", torch.int32, shape=(B,))
    dev = _device(slot_pos, "slot_pos", match_len, "match_len")
    out = _out(out, "out", torch.int32, (B,), dev)
    _call(dev, "swa_window_safe_len", _ptr(slot_pos), _ptr(match_len), _ptr(out), B, W, _stream(stream, dev))
    return out


def swa_prefill_chunk(q, k, v, ring_k, ring_v, pos0: int, scale: float | None = None, out=None, stream=None):
    """Sliding-window prefill of a chunk at positions pos0 .. pos0+C-1, continuing from a ring.

    q [B, C, Hq, D]; k, v [B, C, Hkv, D]; ring_k, ring_v [B, Hkv, W, D] (bf16; on
    entry positions before pos0, updated in place to the last W positions).
    The window is the ring size W.  Returns out [B, C, Hq, D].
    """
    _need(q, "q", torch.bfloat16, 4)
    _need(ring_k, "ring_k", torch.bfloat16, 4)
    B, C, Hq, D = q.shape
    Hkv, W = ring_k.shape[1], ring_k.shape[2]
    _need(k, "k", torch.bfloat16, shape=(B, C, Hkv, D))
    _need(v, "v", torch.bfloat16, shape=(B, C, Hkv, D))
    _need(ring_k, "ring_k", torch.bfloat16, shape=(B, Hkv, W, D))
    _need(ring_v, "ring_v", torch.bfloat16, shape=(B, Hkv, W, D))
    dev = _device(q, "q", k, "k", v, "v", ring_k, "ring_k", ring_v, "ring_v")
    out = _out(out, "out", q.dtype, q.shape, dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _call(dev, "swa_prefill_chunk", _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(ring_k), _ptr(ring_v),
          B, C, Hq, Hkv, D, W, int(pos0), scale, _stream(stream, dev))
    return out


def kv_block_means_int8(codes, scales, means=None, stream=None):
    """K block means of INT8 codes [B, Hkv, T8, D] with scales [B, Hkv, T8/32].

    Returns means float32 [B, Hkv, D, T8/32] (d-major).
    """
    _need(codes, "codes", torch.int8, 4)
    B, Hkv, T8, D = codes.shape
    nblk = _blocks32(T8, "codes")
    _need(scales, "scales", torch.float32, shape=(B, Hkv, nblk))
    dev = _device(codes, "codes", scales, "scales")
    means = _out(means, "means", torch.float32, (B, Hkv, D, nblk), dev)
    _call(dev, "kv_block_means_int8", _ptr(codes), _ptr(scales), _ptr(means), B, Hkv, T8, D, _stream(stream, dev))
    return means


def attn_decode_int8kv_sparse_workspace_size(B, Hq, Hkv, D, T8, Th, topk) -> int:
    return int(_lib.load().attn_decode_int8kv_sparse_workspace_size(B, Hq, Hkv, D, T8, Th, topk))


def attn_decode_int8kv_sparse(q, k_codes, k_scales, v_codes, v_scales, k_means, k_hot, v_hot, topk: int = 64,
                              scale: float | None = None, out=None, sel=None, workspace=None, stream=None):
    """Decode over the bf16 hot tail and each head's top-k INT8 blocks (by q . block mean).

    Returns (out [B, Hq, D] bf16, sel [B, Hq, topk] int32).
    """
    B, Hq, Hkv, D, T8, Th, dev = _int8_pool(q, k_codes, k_scales, v_codes, v_scales, k_hot, v_hot, k_means,
                                            with_means=True)
    out = _out(out, "out", torch.bfloat16, q.shape, dev)
    sel = _out(sel, "sel", torch.int32, (B, Hq, topk), dev)
    need = attn_decode_int8kv_sparse_workspace_size(B, Hq, Hkv, D, T8, Th, topk)
    workspace = _scratch(workspace, "workspace", need, dev)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    opt = (lambda t: _ptr(t) if T8 else None)
    _call(dev, "attn_decode_int8kv_sparse",
          _ptr(q), opt(k_codes), opt(k_scales), opt(v_codes), opt(v_scales), opt(k_means), _ptr(k_hot), _ptr(v_hot),
          _ptr(out), _ptr(sel) if topk > 0 else None, B, Hq, Hkv, D, T8, Th, topk, scale, _ptr(workspace),
          workspace.numel() * workspace.element_size(), _stream(stream, dev))
    return out, sel
