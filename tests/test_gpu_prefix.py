"""swa_window_safe_len on the GPU equals the oracle bit for bit."""

import numpy as np
import pytest
import torch

import hybrid_swa_kv_amd as hsk
import oracle
from hybrid_swa_kv_amd import synth
from tests.helpers import announce

pytestmark = pytest.mark.gpu


def _states(seed, B, W, max_len):
    """Rings replayed to random lengths, then damaged in seeded ways: evicted slots
    (-1), stale positions of an older wrap (p - W), unrelated garbage."""
    P = synth.integers(600, seed, (B,), 0, max_len + 1)
    pos = np.full((B, W), -1, dtype=np.int64)
    for b in range(B):
        if P[b] > 0:
            pos[b] = oracle.ring_positions(int(P[b]) - 1, W)
    kind = synth.integers(600, seed + 1, (B,), 0, 4)
    slot = synth.integers(600, seed + 2, (B,), 0, W)
    junk = synth.integers(600, seed + 3, (B,), 0, 1 << 20)
    for b in range(B):
        s = int(slot[b])
        if kind[b] == 1:
            pos[b, s] = -1
        elif kind[b] == 2 and pos[b, s] >= W:
            pos[b, s] -= W
        elif kind[b] == 3:
            pos[b, s] = int(junk[b])
    # token matches: the whole prefix, a random shorter one, or a longer one
    mk = synth.integers(600, seed + 4, (B,), 0, 3)
    frac = synth.integers(600, seed + 5, (B,), 0, 1001)
    M = np.where(mk == 0, P, np.where(mk == 1, (P * frac) // 1000, P + frac))
    return pos.astype(np.int32), M.astype(np.int32)


def _run(pos, M):
    sp = torch.from_numpy(pos).cuda()
    ml = torch.from_numpy(M).cuda()
    got = hsk.swa_window_safe_len(sp, ml)
    torch.cuda.synchronize()
    return got.cpu().numpy()


@pytest.mark.parametrize("W,B,max_len", [(1, 64, 8), (4, 300, 40), (100, 200, 500), (128, 256, 700), (1024, 64, 3000)])
def test_window_safe_len_matches_oracle(W, B, max_len):
    announce(f"window_safe W={W} B={B}")
    pos, M = _states(W, B, W, max_len)
    want = oracle.window_safe_len(pos, M, W)
    got = _run(pos, M)
    assert np.array_equal(got.astype(np.int64), want), np.nonzero(got != want)[0][:8]


def test_window_safe_len_ring_decode_shape():
    """Batch 32, window 128, contexts of 32768 tokens (the ring-decode workload)."""
    announce("window_safe C2 shape")
    B, W, ctx = 32, 128, 32768
    pos = np.stack([oracle.ring_positions(ctx - 1, W)] * B).astype(np.int32)
    M = np.full(B, ctx, dtype=np.int32)
    M[1::4] = ctx - 1          # one token short: its window lost a position
    M[2::4] = ctx + 500        # token match past the pool: cut back to ctx
    pos[3::4, 5] = -1          # a freed slot
    want = oracle.window_safe_len(pos, M, W)
    got = _run(pos, M)
    assert np.array_equal(got.astype(np.int64), want)
    assert set(np.unique(want)) <= {0, ctx}


def test_window_safe_len_empty_batch():
    sp = torch.empty((0, 16), dtype=torch.int32, device="cuda")
    ml = torch.empty((0,), dtype=torch.int32, device="cuda")
    assert hsk.swa_window_safe_len(sp, ml).numel() == 0


def test_window_safe_len_window_limit():
    """W = 65536, the largest window: a wrapped ring matched in full, one token
    short (its window lost a position), one token past the pool, and a ring that
    has not filled yet."""
    announce("window_safe W=65536")
    W, ctx = 65536, 70000
    pos = np.stack([oracle.ring_positions(ctx - 1, W)] * 3 + [oracle.ring_positions(999, W)]).astype(np.int32)
    M = np.array([ctx, ctx - 1, ctx + 1, 1000], dtype=np.int32)
    want = oracle.window_safe_len(pos, M, W)
    got = _run(pos, M)
    assert np.array_equal(got.astype(np.int64), want)
    assert list(want) == [ctx, 0, ctx, 1000]
