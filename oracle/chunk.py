"""Chunked sliding-window prefill that continues from a ring buffer.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[K25-arch] section 4.2 prefills a long document in chunks (prefill_chunk_size
4096, compared with 8192); [MiMo-inf] section 2 keeps a sliding-window layer's
KV in a W-slot ring (slot = position mod W, see ``oracle.ring``).  Put together,
a chunk of C tokens at positions pos0 .. pos0+C-1 attends, for each of its
queries, the window of W positions ending at the query; positions before pos0
are no longer in any chunk and are read from the ring, which on entry holds the
previous chunks' last W positions.  After the chunk the ring holds the last W
positions up to pos0+C-1.
"""

from __future__ import annotations

import numpy as np

from .attention import _kv_head, attend_masked, default_scale, visible_prefill


def swa_prefill_chunk(q, k, v, ring_k, ring_v, pos0: int, window: int, scale: float | None = None):
    """One chunk.  q [B, C, Hq, D]; k, v [B, C, Hkv, D] (the chunk's K/V, token-major);
    ring_k, ring_v [B, Hkv, W, D] holding positions max(0, pos0-W) .. pos0-1 at slot
    position mod W (W = window).  Returns (out [B, C, Hq, D] fp64, ring_k', ring_v')."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, C, Hq, D = q.shape
    Hkv = k.shape[2]
    W = int(window)
    if scale is None:
        scale = default_scale(D)
    first = max(0, pos0 - W)                     # oldest position a chunk query can see
    keys = np.arange(first, pos0 + C)            # absolute key positions
    rows = np.arange(pos0, pos0 + C)             # absolute query positions
    mask = visible_prefill(rows, keys, W, 1 << 62)
    out = np.empty((B, C, Hq, D), dtype=np.float64)
    for b in range(B):
        # the logical K/V of every needed position: ring below pos0, the chunk above
        kl = np.empty((len(keys), Hkv, D))
        vl = np.empty((len(keys), Hkv, D))
        for j, p in enumerate(keys):
            if p < pos0:
                kl[j] = ring_k[b, :, p % W]
                vl[j] = ring_v[b, :, p % W]
            else:
                kl[j] = k[b, p - pos0]
                vl[j] = v[b, p - pos0]
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            out[b, :, h] = attend_masked(q[b, :, h], kl[:, g], vl[:, g], mask, scale)
    # the ring after the chunk: each chunk position, in order, overwrites its slot
    rk = np.array(ring_k, dtype=np.float64, copy=True)
    rv = np.array(ring_v, dtype=np.float64, copy=True)
    for p in range(pos0, pos0 + C):
        rk[:, :, p % W] = k[:, p - pos0]
        rv[:, :, p % W] = v[:, p - pos0]
    return out, rk, rv
