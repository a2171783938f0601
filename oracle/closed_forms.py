"""Closed forms for pair counts, FLOPs and the hybrid KV ratio.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).
"""

from __future__ import annotations


def visible_pairs_prefill(L: int, W: int) -> int:
    """Number of visible (query, key) pairs of one head in a length-L prefill.

    Full causal (W <= 0 or W >= L): L(L+1)/2.  Window W < L: the first W rows see
    1..W keys, every later row sees W keys.
    """
    if W <= 0 or W >= L:
        return L * (L + 1) // 2
    return W * (W + 1) // 2 + (L - W) * W


def attention_flops(pairs: int, Hq: int, D: int) -> int:
    """Algorithmic FLOPs: QK^T and PV each cost 2*D per visible pair per head."""
    return 4 * D * Hq * pairs


def hybrid_kv_ratio(L: int, n_full: int = 10, n_swa: int = 60, W: int = 128) -> float:
    """KV bytes of a hybrid stack relative to an all-full-attention stack.

    [MiMo-inf] section 1: 70 layers, 10 with full attention and 60 with a
    128-token sliding window; the SWA layers keep only min(L, W) tokens.
    """
    return (n_full * L + n_swa * min(L, W)) / ((n_full + n_swa) * L)


def hybrid_prefill_pair_ratio(L: int, n_full: int = 10, n_swa: int = 60, W: int = 128) -> float:
    """Prefill attention work of the same hybrid stack relative to all-full."""
    full = visible_pairs_prefill(L, 0)
    return (n_full * full + n_swa * visible_pairs_prefill(L, W)) / ((n_full + n_swa) * full)
