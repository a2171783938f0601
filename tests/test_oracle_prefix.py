"""Pins for the window-safe prefix length oracle ([MiMo-inf] section 2, prefix cache)."""

import numpy as np
import pytest

import oracle


def test_hand_cases_window_4():
    W = 4
    # positions 0..9 appended: slots hold 8, 9, 6, 7 (the last four)
    full = [8, 9, 6, 7]
    # the whole cached prefix is reusable: its last four positions are present
    assert oracle.window_safe_len([full], [10], W)[0] == 10
    # a match one token shorter needs 5..8, but 5 was evicted: a "pseudo-hit";
    # no shorter prefix has its window either (0 is gone), so nothing is reusable
    assert oracle.window_safe_len([full], [9], W)[0] == 0
    # positions 0..2 appended (slot 3 never written)
    early = [0, 1, 2, -1]
    assert oracle.window_safe_len([early], [3], W)[0] == 3
    assert oracle.window_safe_len([early], [2], W)[0] == 2
    # a longer token match is cut back to what the pool still holds
    assert oracle.window_safe_len([early], [5], W)[0] == 3
    # position 7 freed: the tail window 6..9 is broken
    assert oracle.window_safe_len([[8, 9, 6, -1]], [10], W)[0] == 0
    # a slot holding a position of another wrap (3 instead of 7) is not position 7
    assert oracle.window_safe_len([[8, 9, 6, 3]], [10], W)[0] == 0
    # empty pool, or a zero / negative match: nothing to reuse
    assert oracle.window_safe_len([[-1] * 4], [7], W)[0] == 0
    assert oracle.window_safe_len([full], [0], W)[0] == 0
    assert oracle.window_safe_len([full], [-3], W)[0] == 0


@pytest.mark.parametrize("W", [1, 3, 4, 7])
def test_closed_form_for_replayed_rings(W):
    """After positions 0..P-1 are appended the ring holds max(0, P-W)..P-1.  A prefix
    of length l needs max(0, l-W)..l-1.  If P <= W everything up to P is there, so
    every l <= P is safe; if P > W the needed block lies inside P-W..P-1 only for
    l = P.  Hence safe(M) = M when M == P or P <= W (M <= P), and 0 otherwise."""
    for P in range(0, 3 * W + 2):
        held = oracle.ring_positions(P - 1, W) if P > 0 else np.full(W, -1)
        for M in range(0, P + 1):
            want = M if (M == P or P <= W) else 0
            got = oracle.window_safe_len([held], [M], W)[0]
            assert got == want, (W, P, M, got, want)
