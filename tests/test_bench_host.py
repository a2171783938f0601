"""bench.py's accounting (host only): algorithmic bytes and FLOP of each workload
against the figures the workload shapes fix, and the block-sparse counters
against brute force on small inputs."""

import os
import subprocess
import sys

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_ring_decode_bytes():
    # batch 32, 8 KV heads, window 128, head_dim 128: ring K+V 16,777,216 B, q and out
    # 262,144 B each, the new token's K/V 131,072 B
    assert bench.ring_bytes_per_call() == 16_777_216 + 262_144 + 262_144 + 131_072 == 17_432_576


def test_int8_decode_and_quant_bytes():
    # batch 16, context 65536 (63488 INT8 + 2048 bf16), 8 KV heads, 32 q heads, d 128
    codes = 2 * 16 * 8 * 63488 * 128
    scales = 2 * 16 * 8 * (63488 // 32) * 4
    hot = 2 * 16 * 8 * 2048 * 128 * 2
    assert bench.int8_decode_bytes() == codes + scales + hot + 2 * 16 * 32 * 128 * 2 == 2_216_886_272
    assert bench.int8_quant_bytes() == 6_243_155_968


def test_prefill_pairs_and_flop_ratio():
    # one head, L 131072: window 1024 -> 133,693,952 visible pairs; full causal 8,590,000,128
    assert bench.pairs_prefill(131072, 1024) == 133_693_952
    assert bench.pairs_prefill(131072, 0) == 8_590_000_128
    assert bench.pairs_prefill(131072, 131072) == 8_590_000_128
    flop_swa = 4 * 128 * 64 * bench.pairs_prefill(131072, 1024)
    assert flop_swa == 4_380_883_419_136
    assert round(bench.pairs_prefill(131072, 0) / bench.pairs_prefill(131072, 1024), 4) == 64.2512
    # brute force on a small case
    for L, W in ((37, 5), (64, 64), (100, 1)):
        i, j = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
        assert bench.pairs_prefill(L, W) == int(((i - j >= 0) & (i - j < W)).sum())


def _random_sel(rng, Hq, nb, topk):
    sel = np.full((Hq, nb, topk), -1, dtype=np.int32)
    for h in range(Hq):
        for qb in range(nb):
            k = min(qb, topk)
            sel[h, qb, :k] = np.sort(rng.choice(qb, size=k, replace=False)) if k else []
    return sel


def test_sparse_counters_brute_force():
    rng = np.random.default_rng(11)
    L, block, W, Hq, Hkv, D, topk = 768, 64, 130, 3, 1, 128, 4
    nb = L // block
    sel = _random_sel(rng, Hq, nb, topk)
    pairs, tiles = 0, 0
    for h in range(Hq):
        for i in range(L):
            kept = set(int(x) for x in sel[h, i // block] if x >= 0)
            for j in range(i + 1):
                if i - j < W or (j // block) in kept:
                    pairs += 1
        for qb in range(nb):
            kw0 = max(0, qb * block - W + 1) // block
            union = set(range(kw0, qb + 1)) | set(int(x) for x in sel[h, qb] if x >= 0)
            tiles += len(union)
    assert bench.sparse_pairs(sel, L, block, W) == pairs
    assert bench.sparse_tile_bytes(sel, L, block, W, Hkv, D) == tiles * 2 * block * D * 2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
