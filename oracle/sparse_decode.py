"""Top-k block-sparse decode over the hot + INT8 KV pool.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[K25-arch] section 2.2 joins two structures: "direction one" keeps the newest
tokens (2K, the hot zone) as full-precision KV and older ones as INT8 with one
scale per 32 tokens (section 2.3); "direction two" lets a query see a local
window plus its top-64 long-range keys.  Block form used here (readings):

* the local window is the hot tail: every bf16 hot token is attended;
* the long-range candidates are the 32-token INT8 blocks, each summarised by
  the mean of its dequantised K, stored with the block:
  mean_d = fl32(fl32(sum of the 32 codes) * scale) / 32 (the code sum is an
  exact integer, so one fp32 rounding; the division by 32 is exact);
* per query head the score of block j is q . mean_j in fp64 (q is bf16, the
  mean fp32: every product is exact in fp64); the topk highest scores are kept,
  ties to the lower block; all blocks when there are at most topk;
* the query attends the hot tail and every token of its kept blocks.
"""

from __future__ import annotations

import numpy as np

from .attention import _kv_head, attend_masked, default_scale
from .quant import dequant_int8_b32

BLOCK = 32


def int8_block_means(codes, scales) -> np.ndarray:
    """Means [B, Hkv, T8/32, D] float32 of the dequantised blocks, per the rule above."""
    codes = np.asarray(codes, dtype=np.int64)
    B, Hkv, T8, D = codes.shape
    sums = codes.reshape(B, Hkv, T8 // BLOCK, BLOCK, D).sum(axis=3)          # exact integers
    prod = sums.astype(np.float32) * np.asarray(scales, dtype=np.float32)[..., None]   # one rounding
    return (prod * np.float32(1.0 / BLOCK)).astype(np.float32)              # exact scaling


def sparse_select(q, means, topk: int, return_scores: bool = False):
    """Kept INT8 blocks [B, Hq, topk] int32 per query head (ascending, -1 padded)."""
    q = np.asarray(q, dtype=np.float64)
    means = np.asarray(means, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv, nblk = means.shape[1], means.shape[2]
    sel = np.full((B, Hq, max(topk, 0)), -1, dtype=np.int32)
    scores = np.empty((B, Hq, nblk))
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            sc = means[b, g] @ q[b, h]
            scores[b, h] = sc
            n = min(nblk, topk)
            if n <= 0:
                continue
            order = np.argsort(-sc, kind="stable")          # stable: ties keep block order
            sel[b, h, :n] = np.sort(order[:n])
    return (sel, scores) if return_scores else sel


def attn_decode_int8kv_sparse(q, k_codes, k_scales, v_codes, v_scales, k_hot, v_hot, sel,
                              scale: float | None = None) -> np.ndarray:
    """Decode over the hot tail and the kept INT8 blocks ``sel`` [B, Hq, topk].
    Returns [B, Hq, D] fp64."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k_hot.shape[1]
    T8 = k_codes.shape[2]
    Th = k_hot.shape[2]
    if scale is None:
        scale = default_scale(D)
    out = np.empty((B, Hq, D), dtype=np.float64)
    for b in range(B):
        for g in range(Hkv):
            kk = np.concatenate([dequant_int8_b32(k_codes[b, g], k_scales[b, g], BLOCK),
                                 np.asarray(k_hot[b, g], dtype=np.float64)], axis=0)
            vv = np.concatenate([dequant_int8_b32(v_codes[b, g], v_scales[b, g], BLOCK),
                                 np.asarray(v_hot[b, g], dtype=np.float64)], axis=0)
            for h in range(Hq):
                if _kv_head(h, Hq, Hkv) != g:
                    continue
                visible = np.zeros(T8 + Th, dtype=bool)
                visible[T8:] = True
                for j in sel[b, h]:
                    if j >= 0:
                        visible[BLOCK * j:BLOCK * (j + 1)] = True
                out[b, h] = attend_masked(q[b, h][None], kk, vv, visible[None], scale)[0]
    return out
