"""Pins for the chunked sliding-window prefill oracle."""

import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("L,C,W,Hq,Hkv,D", [(96, 32, 16, 2, 1, 8), (120, 40, 64, 4, 2, 8), (64, 64, 8, 2, 2, 4),
                                            (100, 25, 100, 2, 1, 8)])
def test_chunks_carrying_the_ring_equal_one_shot_prefill(L, C, W, Hq, Hkv, D):
    """Chunk after chunk, each continuing from the ring the previous one left, gives
    the rows of swa_prefill over the whole sequence, and the final ring holds the
    last W positions (as a write-pointer replay of the whole sequence leaves it)."""
    rng = np.random.default_rng(L + C + W)
    B = 2
    q = rng.standard_normal((B, L, Hq, D))
    k = rng.standard_normal((B, L, Hkv, D))
    v = rng.standard_normal((B, L, Hkv, D))
    want = oracle.swa_prefill(q, k, v, W)
    junk = rng.standard_normal((B, Hkv, W, D))          # never-written slots hold garbage
    rk, rv = junk.copy(), junk.copy()
    got = np.empty_like(want)
    for pos0 in range(0, L, C):
        c = min(C, L - pos0)
        out, rk, rv = oracle.swa_prefill_chunk(q[:, pos0:pos0 + c], k[:, pos0:pos0 + c], v[:, pos0:pos0 + c],
                                               rk, rv, pos0, W)
        got[:, pos0:pos0 + c] = out
    assert np.allclose(got, want, rtol=0, atol=1e-12)
    held = oracle.ring_positions(L - 1, W)
    for s in range(W):
        if held[s] >= 0:
            assert np.array_equal(rk[:, :, s], k[:, held[s]])
            assert np.array_equal(rv[:, :, s], v[:, held[s]])


def test_first_chunk_reads_no_ring():
    """At pos0 = 0 the ring's contents (garbage) cannot matter."""
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((1, 16, 2, 4)) for _ in range(3))
    a, _, _ = oracle.swa_prefill_chunk(q, k[:, :, :1], v[:, :, :1], np.zeros((1, 1, 8, 4)), np.zeros((1, 1, 8, 4)), 0, 8)
    b, _, _ = oracle.swa_prefill_chunk(q, k[:, :, :1], v[:, :, :1], np.full((1, 1, 8, 4), 7.0),
                                       np.full((1, 1, 8, 4), -3.0), 0, 8)
    assert np.array_equal(a, b)
