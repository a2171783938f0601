"""Pins for the block-selection, ring-buffer and closed-form oracles (CPU only)."""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from hybrid_swa_kv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- selection --

def brute_select(q, k, block, topk):
    """Pure Python: fsum means, fsum dot products, sorted() on (-score, kb)."""
    L, Hq, D = q.shape
    Hkv = k.shape[1]
    nb = L // block
    out = np.full((Hq, nb, topk), -1, dtype=np.int32)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        qm = [[math.fsum(q[t, h, d] for t in range(b * block, b * block + block)) / block
               for d in range(D)] for b in range(nb)]
        km = [[math.fsum(k[t, g, d] for t in range(b * block, b * block + block)) / block
               for d in range(D)] for b in range(nb)]
        for qb in range(nb):
            cand = [(-math.fsum(qm[qb][d] * km[kb][d] for d in range(D)), kb) for kb in range(qb)]
            chosen = sorted(kb for _, kb in sorted(cand)[:topk])
            out[h, qb, : len(chosen)] = chosen
    return out


@pytest.mark.parametrize("L,Hq,Hkv,D,block,topk", [
    (64, 2, 1, 4, 4, 3), (96, 4, 2, 8, 8, 5), (120, 3, 3, 2, 6, 1), (64, 2, 2, 4, 2, 31)])
def test_select_bruteforce(L, Hq, Hkv, D, block, topk):
    rng = np.random.default_rng(L + D)
    q, k = rng.standard_normal((L, Hq, D)), rng.standard_normal((L, Hkv, D))
    assert np.array_equal(oracle.block_select(q, k, block, topk), brute_select(q, k, block, topk))


def test_select_exact_tie_keeps_lower_index():
    L, D, block = 64, 4, 4
    rng = np.random.default_rng(7)
    q, k = rng.standard_normal((L, 1, D)), rng.standard_normal((L, 1, D))
    k[20:24] = k[8:12]                                  # block 5 duplicates block 2
    sel, sc = oracle.block_select(q, k, block, 1, return_scores=True)
    for qb in range(6, 16):
        assert sc[0][qb, 2] == sc[0][qb, 5]
        if np.argmax(sc[0][qb, :qb]) in (2, 5):
            assert sel[0, qb, 0] == 2


def test_select_early_blocks_take_everything_and_padding():
    L, D, block, topk = 80, 4, 8, 4
    rng = np.random.default_rng(8)
    q, k = rng.standard_normal((L, 2, D)), rng.standard_normal((L, 1, D))
    sel = oracle.block_select(q, k, block, topk)
    for qb in range(topk + 1):
        assert sel[:, qb, :qb].tolist() == [list(range(qb))] * 2
        assert (sel[:, qb, qb:] == -1).all()
    assert (sel[:, topk + 1:] >= 0).all()
    assert (np.diff(sel[:, topk + 1:], axis=-1) > 0).all()           # ascending, distinct


def test_block_sums_of_bf16_are_exact_in_fp64():
    # the precondition that makes selection independent of summation order
    bits = synth.token_major(60, synth.Q, 256, 2, 16)
    x = synth.bf16_bits_to_f32(bits)
    sums = oracle.block_sums(x, 64)
    for h in range(2):
        for b in range(4):
            for d in range(0, 16, 5):
                exact = sum(Fraction(float(v)) for v in x[64 * b: 64 * b + 64, h, d])
                assert Fraction(float(sums[h, b, d])) == exact


# --------------------------------------------------------------------- ring --

def pointer_ring(tokens, W):
    """Explicit write pointer: each append writes the pointer's slot, then advances."""
    ring = [None] * W
    wp = 0
    for t in tokens:
        ring[wp] = t
        wp = (wp + 1) % W
    return ring


@pytest.mark.parametrize("W", [1, 3, 8, 128])
def test_ring_matches_write_pointer(W):
    for T in range(1, 3 * W + 2):
        ref = pointer_ring(list(range(T)), W)
        held = oracle.ring_positions(T - 1, W)
        assert [(-1 if r is None else r) for r in ref] == held.tolist()
        assert int(oracle.ring_slot(T - 1, W)) == (ref.index(T - 1))
        window = set(range(max(0, T - W), T))
        assert set(int(p) for p in held if p >= 0) == window


def test_ring_fill_and_append():
    B, H, W, D = 2, 3, 8, 4
    rng = np.random.default_rng(9)
    seq = rng.standard_normal((B, H, 40, D))
    init = np.full((B, H, W, D), 7.0)
    last = [5, 33]
    ring = oracle.ring_fill(seq, [0, 0], last, W, init)
    for b in range(B):
        held = oracle.ring_positions(last[b], W)
        for s in range(W):
            if held[s] < 0:
                assert (ring[b, :, s] == 7.0).all()
            else:
                assert np.array_equal(ring[b, :, s], seq[b, :, held[s]])
    new = rng.standard_normal((B, H, D))
    after = oracle.ring_append(ring, [6, 34], new)
    for b, p in enumerate([6, 34]):
        s = p % W
        assert np.array_equal(after[b, :, s], new[b])
        others = [x for x in range(W) if x != s]
        assert np.array_equal(after[b, :, others], ring[b, :, others])


def test_decode_from_ring_slots_equals_logical_decode():
    # attending over the ring's valid slots gives the logical window decode
    B, Hq, Hkv, W, D = 3, 4, 2, 16, 8
    rng = np.random.default_rng(10)
    seq_k, seq_v = rng.standard_normal((B, Hkv, 100, D)), rng.standard_normal((B, Hkv, 100, D))
    q = rng.standard_normal((B, Hq, D))
    pos = [3, 15, 77]
    rk = oracle.ring_fill(seq_k, [0] * B, pos, W, np.zeros((B, Hkv, W, D)))
    rv = oracle.ring_fill(seq_v, [0] * B, pos, W, np.zeros((B, Hkv, W, D)))
    ref = oracle.swa_decode(q, seq_k, seq_v, [0] * B, pos, W)
    for b in range(B):
        held = oracle.ring_positions(pos[b], W)
        slots = np.nonzero(held >= 0)[0]
        for h in range(Hq):
            g = h // 2
            o = oracle.attend_masked(q[b, h][None], rk[b, g, slots], rv[b, g, slots],
                                     np.ones((1, len(slots)), bool), 1 / math.sqrt(D))
            assert np.max(np.abs(o[0] - ref[b, h])) <= 1e-13


# ------------------------------------------------------------- closed forms --

@pytest.mark.parametrize("L,W", [(1, 1), (5, 2), (64, 64), (100, 0), (257, 64), (512, 128), (300, 1000)])
def test_pair_counts(L, W):
    mask = oracle.visible_prefill(np.arange(L), np.arange(L), W, L)
    assert oracle.visible_pairs_prefill(L, W) == int(mask.sum())
    ones = torch.ones(L, L, dtype=torch.bool)
    band = torch.tril(ones, 0) if (W <= 0 or W >= L) else (torch.tril(ones, 0) & ~torch.tril(ones, -W))
    assert oracle.visible_pairs_prefill(L, W) == int(band.sum())


def test_page_constants_golden():
    with open(os.path.join(GOLDEN, "page_constants.json")) as f:
        g = json.load(f)
    mix = g["mimo_hybrid_stack"]
    assert mix["full_layers"] + mix["swa_layers"] == mix["layers"]
    # the KV and prefill ratios of the 10 + 60 (W = 128) stack are "about 1/7"
    for L in (32768, 65536, 131072, 262144, 1048576):
        r = oracle.hybrid_kv_ratio(L, mix["full_layers"], mix["swa_layers"], mix["window"])
        assert abs(r - mix["kv_ratio_approx"]) / mix["kv_ratio_approx"] < mix["approx_rel_tol"]
        p = oracle.hybrid_prefill_pair_ratio(L, mix["full_layers"], mix["swa_layers"], mix["window"])
        assert abs(p - mix["prefill_ratio_approx"]) / mix["prefill_ratio_approx"] < mix["approx_rel_tol"]
    # limit: only the full layers grow with L
    assert oracle.hybrid_kv_ratio(10 ** 12) == pytest.approx(1 / 7, rel=1e-9)
    assert round(oracle.hybrid_kv_ratio(131072), 6) == 0.143694
    k25 = g["k25_lightengine_yaml"]
    assert (k25["hot_size"], k25["window_size"], k25["sparse_topk"], k25["warm_quant_bits"]) == (2048, 1024, 64, 8)
    assert g["k25_int8_block_tokens"] == 32


def test_workload_closed_forms():
    # 512-token window-128 prefill and the 131072-token window-1024 / full pair
    assert oracle.visible_pairs_prefill(512, 128) == 57408
    assert oracle.attention_flops(57408, 2, 64) == 29392896
    swa = oracle.visible_pairs_prefill(131072, 1024)
    full = oracle.visible_pairs_prefill(131072, 0)
    assert (swa, full) == (133693952, 8590000128)
    assert round(full / swa, 4) == 64.2512
    assert oracle.attention_flops(swa, 64, 128) == 4380883419136
