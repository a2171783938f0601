"""Attention by its plain definition: explicit visibility masks, fp64 softmax.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Definition used by every call (the pages describe attention layers but never
write the formula out; this is the textbook scaled dot-product attention,
restricted to a visible key set):

  for query row i at position p_i, query head h, KV head g = h // (Hq / Hkv):
    V_i  = { j : key j is visible to query i }      (never empty)
    s_j  = scale * sum_d Q[i,h,d] * K[j,g,d]         (fp64)
    m    = max_{j in V_i} s_j
    out  = sum_{j in V_i} exp(s_j - m) V[j,g,:] / sum_{j in V_i} exp(s_j - m)

Masked keys are *excluded* from the max and from both sums.

Visibility rules:

* sliding window of W tokens, including the query itself: 0 <= p_i - j < W
  ([MiMo-inf] section 1: the SWA layers keep only the latest 128 tokens;
  [K25-arch] section 2.2 "direction two": local sliding window of 1024).
  W <= 0 or W >= L means plain causal attention (the full-attention layers of
  [MiMo-inf] section 1).
* the INT8 decode attends every cached position (full-attention layer of the
  tiered cache, [K25-arch] section 2.2 "direction one").
* block-sparse: the window rule above OR the key's 64-token block is one of the
  blocks selected for the query's block ([K25-arch] section 2.2 "direction
  two", sparse long-range attention; selection in ``oracle/select.py``).

GQA head grouping is contiguous: query head h reads KV head h // (Hq // Hkv).
The pages never name GQA; this is the plainest reading and the one torch's
``enable_gqa`` uses, which the pins exploit.
"""

from __future__ import annotations

import math

import numpy as np

from .quant import dequant_int8_b32


def default_scale(D: int) -> float:
    """Softmax scale 1/sqrt(head_dim) (textbook scaled dot-product attention)."""
    return 1.0 / math.sqrt(D)


def visible_prefill(pos_q: np.ndarray, pos_k: np.ndarray, window: int, L: int) -> np.ndarray:
    """Boolean [nq, nk]: is key position pos_k[j] visible to query position pos_q[i].

    Sliding window of ``window`` tokens including the query's own position;
    ``window <= 0`` or ``window >= L`` selects plain causal attention.
    """
    d = np.asarray(pos_q, dtype=np.int64)[:, None] - np.asarray(pos_k, dtype=np.int64)[None, :]
    if window <= 0 or window >= L:
        return d >= 0
    return (d >= 0) & (d < window)


def attend_masked(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
                  scale: float) -> np.ndarray:
    """Masked softmax attention for one head.

    q [nq, D], k [nk, D], v [nk, D], mask [nq, nk] bool -> out [nq, D] fp64.
    Every row of ``mask`` must contain at least one visible key.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    mask = np.asarray(mask, dtype=bool)
    if not mask.any(axis=1).all():
        raise ValueError("a query row has no visible key")
    s = float(scale) * (q @ k.T)
    m = np.where(mask, s, -np.inf).max(axis=1, keepdims=True)
    w = np.exp(np.where(mask, s - m, -np.inf))
    return (w @ v) / w.sum(axis=1, keepdims=True)


def _kv_head(h: int, Hq: int, Hkv: int) -> int:
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


def swa_prefill(q, k, v, window: int, scale: float | None = None, rows=None,
                row_block: int = 128) -> np.ndarray:
    """Causal sliding-window (or full causal) GQA prefill.

    q [L, Hq, D] or [B, L, Hq, D]; k, v [L, Hkv, D] or [B, L, Hkv, D]
    (token-major).  Position of token t is t.  ``rows`` optionally restricts the
    query rows computed (sorted or not); the result is [B?, len(rows), Hq, D]
    in fp64.  ``window`` as in ``visible_prefill``.
    """
    squeeze = np.ndim(q) == 3
    if squeeze:
        q, k, v = q[None], k[None], v[None]
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    if scale is None:
        scale = default_scale(D)
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((B, len(rows), Hq, D), dtype=np.float64)
    full = window <= 0 or window >= L
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            for r0 in range(0, len(rows), row_block):
                rb = rows[r0:r0 + row_block]
                lo = 0 if full else max(0, int(rb.min()) - window + 1)
                hi = int(rb.max()) + 1
                keys = np.arange(lo, hi)
                mask = visible_prefill(rb, keys, window, L)
                out[b, r0:r0 + len(rb), h] = attend_masked(
                    q[b, rb, h], k[b, lo:hi, g], v[b, lo:hi, g], mask, scale)
    return out[0] if squeeze else out


def swa_decode(q, k_seq, v_seq, seq_start, pos, window: int,
               scale: float | None = None) -> np.ndarray:
    """One-token sliding-window decode against the *logical* sequence.

    q [B, Hq, D]; k_seq, v_seq [B, Hkv, P, D] hold positions
    seq_start[b] .. seq_start[b]+P-1 of sequence b; pos[b] is the position of
    the query token (its own K/V is part of k_seq).  Visible keys:
    max(0, pos-W+1) .. pos ([MiMo-inf] section 1, window of 128 tokens);
    ``window <= 0`` means all of 0..pos.  The ring buffer is never read here.
    Returns [B, Hq, D] fp64.
    """
    B, Hq, D = q.shape
    Hkv = k_seq.shape[1]
    P = k_seq.shape[2]
    if scale is None:
        scale = default_scale(D)
    out = np.empty((B, Hq, D), dtype=np.float64)
    for b in range(B):
        p = int(pos[b])
        base = int(seq_start[b])
        lo = 0 if window <= 0 else max(0, p - window + 1)
        if lo < base or p >= base + P:
            raise ValueError("k_seq does not cover the visible positions")
        keys = np.arange(lo, p + 1)
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            mask = visible_prefill(np.array([p]), keys, window if window > 0 else 0, p + 1)
            out[b, h] = attend_masked(q[b, h][None], k_seq[b, g, keys - base],
                                      v_seq[b, g, keys - base], mask, scale)[0]
    return out


def attn_decode_int8kv(q, k_codes, k_scales, v_codes, v_scales, k_hot, v_hot,
                       scale: float | None = None, block: int = 32) -> np.ndarray:
    """Full-attention decode over an INT8 warm region followed by a bf16 hot tail.

    [K25-arch] section 2.2 "direction one": the newest tokens (2K) stay as
    full-precision KV, the middle region is INT8 with a block-wise scale
    (section 2.3: one scale per 32 tokens).  Positions 0..T8-1 are the
    dequantized codes code*scale (exact in fp64), positions T8..T8+Th-1 the hot
    rows.  The query sits at position T8+Th-1, so every cached key is visible.

    q [B, Hq, D]; *_codes [B, Hkv, T8, D] int8; *_scales [B, Hkv, T8/block];
    *_hot [B, Hkv, Th, D].  Returns [B, Hq, D] fp64.
    """
    B, Hq, D = q.shape
    Hkv = k_hot.shape[1]
    if scale is None:
        scale = default_scale(D)
    out = np.empty((B, Hq, D), dtype=np.float64)
    for b in range(B):
        for g in range(Hkv):
            kk = np.concatenate([dequant_int8_b32(k_codes[b, g], k_scales[b, g], block),
                                 np.asarray(k_hot[b, g], dtype=np.float64)], axis=0)
            vv = np.concatenate([dequant_int8_b32(v_codes[b, g], v_scales[b, g], block),
                                 np.asarray(v_hot[b, g], dtype=np.float64)], axis=0)
            n = kk.shape[0]
            heads = [h for h in range(Hq) if _kv_head(h, Hq, Hkv) == g]
            mask = np.ones((len(heads), n), dtype=bool)
            out[b, heads] = attend_masked(q[b, heads], kk, vv, mask, scale)
    return out


def blocksparse_visible(pos_q: np.ndarray, sel_rows: np.ndarray, L: int, block: int,
                        window: int) -> np.ndarray:
    """Boolean [nq, L]: local window OR the key's block is selected.

    ``sel_rows[r]`` holds the selected block indices (-1 padded) for the query
    block of pos_q[r].  Selected blocks are strictly earlier than the query's
    block, so causality holds without a separate test; the window part follows
    ``visible_prefill``.
    """
    keys = np.arange(L)
    mask = visible_prefill(pos_q, keys, window, L)
    key_block = keys // block
    for r in range(len(pos_q)):
        chosen = sel_rows[r][sel_rows[r] >= 0]
        mask[r] |= np.isin(key_block, chosen)
    return mask


def blocksparse_attend(q, k, v, sel, block: int, window: int, scale: float | None = None,
                       rows=None, row_block: int = 64) -> np.ndarray:
    """Attention over the union of a causal local window and selected key blocks.

    q [L, Hq, D]; k, v [L, Hkv, D]; sel [Hq, L/block, topk] (from
    ``oracle.select.block_select``).  Returns [len(rows), Hq, D] fp64.
    """
    L, Hq, D = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = default_scale(D)
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), Hq, D), dtype=np.float64)
    for h in range(Hq):
        g = _kv_head(h, Hq, Hkv)
        for r0 in range(0, len(rows), row_block):
            rb = rows[r0:r0 + row_block]
            hi = int(rb.max()) + 1
            mask = blocksparse_visible(rb, sel[h, rb // block], L, block, window)[:, :hi]
            out[r0:r0 + len(rb), h] = attend_masked(q[rb, h], k[:hi, g], v[:hi, g], mask, scale)
    return out
