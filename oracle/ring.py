"""Ring-buffer state of a sliding-window KV pool, step by step.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[MiMo-inf] section 2, "dual pools": the SWA pool is sized by the window only,
is a ring buffer, evicts by window, and its storage is strictly O(W); the
full-attention index stays authoritative and maps sequence positions to SWA
slots.  The plainest map with exactly W slots is slot = position mod W: the
slot that position p overwrites is the one that held p - W, the token that just
left the window.

Ring layout: [B, Hkv, W, D]; slot s of sequence b is ring[b, :, s, :].
"""

from __future__ import annotations

import numpy as np


def ring_slot(pos, W: int):
    """Slot written by the token at position ``pos`` (integer, exact)."""
    if W <= 0:
        raise ValueError("ring capacity must be positive")
    return np.asarray(pos, dtype=np.int64) % W


def ring_positions(last_pos: int, W: int) -> np.ndarray:
    """Position held by each slot after positions 0..last_pos were appended in order.

    Returns [W] int64; -1 marks a slot that was never written.  Computed by
    replaying the appends one at a time with an explicit write pointer.
    """
    held = np.full(W, -1, dtype=np.int64)
    for p in range(max(0, last_pos - W + 1), last_pos + 1):
        held[int(ring_slot(p, W))] = p
    return held


def ring_fill(seq: np.ndarray, seq_start, last_pos, W: int, init: np.ndarray) -> np.ndarray:
    """Ring contents after appending positions 0..last_pos[b] of each sequence.

    seq [B, Hkv, P, D] holds positions seq_start[b]..seq_start[b]+P-1 (only the
    last W appended positions can still be in the ring, so only those need to
    be present).  ``init`` [B, Hkv, W, D] is the content of never-written slots.
    Appends are replayed in position order.
    """
    ring = np.array(init, copy=True)
    B = ring.shape[0]
    for b in range(B):
        lp = int(last_pos[b])
        base = int(seq_start[b])
        for p in range(max(0, lp - W + 1), lp + 1):
            t = p - base
            if t < 0 or t >= seq.shape[2]:
                raise ValueError("seq does not cover the appended positions")
            ring[b, :, int(ring_slot(p, W))] = seq[b, :, t]
    return ring


def ring_append(ring: np.ndarray, pos, new: np.ndarray) -> np.ndarray:
    """Ring after sequence b appends ``new[b]`` [Hkv, D] at position pos[b].

    Only slot pos[b] mod W changes; every other slot keeps its bytes.
    """
    out = np.array(ring, copy=True)
    W = ring.shape[2]
    for b in range(ring.shape[0]):
        out[b, :, int(ring_slot(int(pos[b]), W))] = new[b]
    return out
