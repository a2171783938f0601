"""Window-safe prefix length of a sliding-window KV pool.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[MiMo-inf] section 2, the prefix-cache paragraph: with sliding-window layers a
token-level prefix match no longer implies that the KV it needs still exists;
a node's SWA KV may keep only its tail or be gone.  The matching rule becomes
the "window-safe length": a reused prefix is usable only if its last W tokens
still have valid SWA slots.

Readings used here (the pages give the rule in prose only):

* the prefix to reuse has length ell (positions 0 .. ell-1); the sliding-window
  layers of the next token need positions max(0, ell - W) .. ell - 1, i.e. the
  last min(ell, W) tokens;
* position p is present in the SWA pool when its slot, p mod W (the ring map
  of ``oracle.ring``), still holds p;
* the answer is the largest ell <= match_len (the token-level match) whose
  needed positions are all present; ell = 0 needs nothing and is always safe.
"""

from __future__ import annotations

import numpy as np


def position_present(slot_pos: np.ndarray, p: int, W: int) -> bool:
    """True when slot p mod W of this sequence holds position p."""
    return int(slot_pos[p % W]) == p


def window_safe_len(slot_pos, match_len, W: int) -> np.ndarray:
    """Largest reusable prefix length per sequence, by the definition above.

    slot_pos: [B, W] integers, the position each SWA slot holds (-1: empty).
    match_len: [B] token-level prefix match lengths (>= 0).
    Returns [B] int64.  Walks ell downwards from match_len and checks every
    needed position: plain and O(match_len * W), for small cases.
    """
    slot_pos = np.asarray(slot_pos, dtype=np.int64)
    match_len = np.asarray(match_len, dtype=np.int64)
    out = np.zeros(len(match_len), dtype=np.int64)
    for b in range(len(match_len)):
        for ell in range(int(match_len[b]), 0, -1):
            if all(position_present(slot_pos[b], p, W) for p in range(max(0, ell - W), ell)):
                out[b] = ell
                break
    return out
