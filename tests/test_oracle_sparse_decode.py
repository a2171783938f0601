"""Pins for the block-sparse decode over the hot + INT8 pool."""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from hybrid_swa_kv_amd import synth


def _pool(seed, B, Hq, Hkv, D, T8, Th):
    kx = synth.head_major(seed, synth.K, B, Hkv, T8 + Th, D, outlier_p=0.01)
    vx = synth.head_major(seed, synth.V, B, Hkv, T8 + Th, D, outlier_p=0.01)
    q = synth.bf16_bits_to_f32(synth.normal(seed, synth.Q, (B, Hq, D), 1)).astype(np.float64)
    kc, ks = oracle.kv_quant_int8_b32(synth.bf16_bits_to_f32(kx[:, :, :T8]))
    vc, vs = oracle.kv_quant_int8_b32(synth.bf16_bits_to_f32(vx[:, :, :T8]))
    kh = synth.bf16_bits_to_f32(kx[:, :, T8:]).astype(np.float64)
    vh = synth.bf16_bits_to_f32(vx[:, :, T8:]).astype(np.float64)
    return q, kc, ks, vc, vs, kh, vh


def test_block_means_are_the_correctly_rounded_mean():
    """Each mean is the dequantised block mean rounded once to fp32 (exact rationals)."""
    q, kc, ks, _, _, _, _ = _pool(3, 1, 2, 1, 8, 96, 1)
    m = oracle.int8_block_means(kc, ks)
    for j in range(3):
        for d in range(8):
            exact = sum(Fraction(int(c)) for c in kc[0, 0, 32 * j:32 * j + 32, d]) * Fraction(float(ks[0, 0, j])) / 32
            assert float(m[0, 0, j, d]) == float(np.float32(float(exact)))


def test_keeping_every_block_is_the_dense_decode():
    q, kc, ks, vc, vs, kh, vh = _pool(5, 2, 4, 2, 16, 256, 40)
    sel = oracle.sparse_select(q, oracle.int8_block_means(kc, ks), 1000)
    assert (sel[:, :, :8] >= 0).all() and (sel[:, :, 8:] == -1).all()
    got = oracle.attn_decode_int8kv_sparse(q, kc, ks, vc, vs, kh, vh, sel)
    want = oracle.attn_decode_int8kv(q, kc, ks, vc, vs, kh, vh)
    assert np.allclose(got, want, rtol=0, atol=1e-13)


def test_keeping_no_block_is_the_hot_tail_alone():
    q, kc, ks, vc, vs, kh, vh = _pool(6, 1, 2, 1, 16, 128, 33)
    sel = np.full((1, 2, 4), -1, dtype=np.int32)
    got = oracle.attn_decode_int8kv_sparse(q, kc, ks, vc, vs, kh, vh, sel)
    want = oracle.swa_decode(q, kh, vh, [0], [32], 0)      # the 33 hot tokens, full attention
    assert np.allclose(got, want, rtol=0, atol=1e-13)


def test_select_brute_force_and_ties():
    """The kept set is the topk blocks of a pure-Python sort by (-score, block)."""
    q, kc, ks, _, _, _, _ = _pool(7, 2, 4, 2, 16, 640, 1)
    means = oracle.int8_block_means(kc, ks)
    means[0, 0, 5] = means[0, 0, 2]                 # an exact tie: block 2 must win it
    sel, scores = oracle.sparse_select(q, means, 6, return_scores=True)
    for b in range(2):
        for h in range(4):
            g = h // 2
            sc = [float(sum(float(a) * float(c) for a, c in zip(q[b, h], means[b, g, j]))) for j in range(20)]
            order = sorted(range(20), key=lambda j: (-scores[b, h, j], j))
            assert list(sel[b, h]) == sorted(order[:6])
            assert np.allclose(sc, scores[b, h], rtol=1e-12, atol=0)
    assert scores[0, 0, 5] == scores[0, 0, 2]


def test_partial_selection_equals_attention_over_the_gathered_tokens():
    """A kept block j stands for tokens 32 j .. 32 j + 31: attending the hot tail
    plus the kept blocks equals torch's attention (fp64, CPU) over exactly those
    tokens, gathered in order, with no mask (the query sees every cached token)."""
    import torch
    import torch.nn.functional as F

    q, kc, ks, vc, vs, kh, vh = _pool(8, 1, 4, 2, 16, 320, 7)
    kd = oracle.dequant_int8_b32(kc, ks)
    vd = oracle.dequant_int8_b32(vc, vs)
    sel = np.array([[[0, 3, 9, -1], [2, -1, -1, -1], [-1, -1, -1, -1], [1, 2, 3, 4]]], dtype=np.int32)
    got = oracle.attn_decode_int8kv_sparse(q, kc, ks, vc, vs, kh, vh, sel)
    for h in range(4):
        g = h // 2
        blocks = [int(j) for j in sel[0, h] if j >= 0]
        toks = [t for j in blocks for t in range(32 * j, 32 * j + 32)]
        kk = np.concatenate([kd[0, g][toks], kh[0, g]], axis=0)
        vv = np.concatenate([vd[0, g][toks], vh[0, g]], axis=0)
        want = F.scaled_dot_product_attention(torch.from_numpy(q[0, h][None, None]), torch.from_numpy(kk[None]),
                                              torch.from_numpy(vv[None]), scale=0.25)[0, 0].numpy()
        assert np.allclose(got[0, h], want, rtol=0, atol=1e-13), h
    # the selection changes the result: a head keeping nothing differs from one keeping blocks
    assert not np.allclose(got[0, 2], got[0, 3])
