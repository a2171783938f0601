"""Pins for the attention oracle (CPU only).

Each pin is independent of the oracle's own code: pure-Python brute force with
math.fsum, torch's CPU scaled_dot_product_attention in float64, closed-form
special cases, and identities between calls.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from hybrid_swa_kv_amd import synth

def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def brute_prefill(q, k, v, W, scale):
    """Loops over every (row, head, key); visibility written as i-W < j <= i."""
    L, Hq, D = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    out = np.zeros((L, Hq, D))
    for i in range(L):
        for h in range(Hq):
            g = h // group
            keys = [j for j in range(L) if j <= i and (W <= 0 or W >= L or j > i - W)]
            s = [scale * math.fsum(q[i, h, d] * k[j, g, d] for d in range(D)) for j in keys]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = math.fsum(e)
            for d in range(D):
                out[i, h, d] = math.fsum(e[t] * v[keys[t], g, d] for t in range(len(keys))) / z
    return out


@pytest.mark.parametrize("L,Hq,Hkv,D,W", [
    (1, 1, 1, 2, 4), (7, 2, 1, 4, 3), (12, 4, 2, 2, 1), (16, 2, 2, 8, 5),
    (20, 4, 1, 4, 0), (24, 2, 1, 4, 24), (24, 4, 4, 2, 23), (9, 1, 1, 3, 100),
])
def test_bruteforce_prefill(L, Hq, Hkv, D, W):
    q, k, v = _rand((L, Hq, D), 1), _rand((L, Hkv, D), 2), _rand((L, Hkv, D), 3)
    scale = 0.7
    got = oracle.swa_prefill(q, k, v, W, scale)
    ref = brute_prefill(q, k, v, W, scale)
    assert np.max(np.abs(got - ref)) <= 1e-12


def _sdpa(q, k, v, mask=None, causal=False, gqa=False):
    # q [L, Hq, D] -> torch [1, Hq, L, D], float64 on the CPU (library routine)
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))[None]
    tk = torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None]
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None]
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=mask, is_causal=causal, enable_gqa=gqa)
    return o[0].numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("L,Hq,Hkv,D", [(64, 4, 4, 16), (200, 8, 2, 32), (130, 6, 3, 64)])
def test_full_causal_equals_sdpa(L, Hq, Hkv, D):
    q, k, v = _rand((L, Hq, D), 4), _rand((L, Hkv, D), 5), _rand((L, Hkv, D), 6)
    ref = _sdpa(q, k, v, causal=True, gqa=Hq != Hkv)       # default scale 1/sqrt(D)
    for W in (0, -3, L, L + 7):
        got = oracle.swa_prefill(q, k, v, W)
        assert np.max(np.abs(got - ref)) <= 1e-12


@pytest.mark.parametrize("L,W", [(100, 1), (100, 17), (257, 64), (300, 128), (129, 128)])
def test_window_equals_sdpa_band(L, W):
    Hq, Hkv, D = 4, 2, 16
    q, k, v = _rand((L, Hq, D), 7), _rand((L, Hkv, D), 8), _rand((L, Hkv, D), 9)
    ones = torch.ones(L, L, dtype=torch.bool)
    band = torch.tril(ones, 0) & ~torch.tril(ones, -W)       # keys i-W < j <= i
    ref = _sdpa(q, k, v, mask=band, gqa=True)
    got = oracle.swa_prefill(q, k, v, W)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_zero_query_gives_window_mean():
    L, H, D, W = 50, 2, 4, 7
    q = np.zeros((L, H, D))
    k, v = _rand((L, H, D), 10), _rand((L, H, D), 11)
    got = oracle.swa_prefill(q, k, v, W)
    c = np.concatenate([np.zeros((1, H, D)), np.cumsum(v, axis=0)], axis=0)
    for i in range(L):
        lo = max(0, i - W + 1)
        mean = (c[i + 1] - c[lo]) / (i + 1 - lo)
        assert np.max(np.abs(got[i] - mean)) <= 1e-12


def test_window_one_returns_own_value_and_row0():
    L, Hq, Hkv, D = 33, 4, 2, 8
    q, k, v = _rand((L, Hq, D), 12), _rand((L, Hkv, D), 13), _rand((L, Hkv, D), 14)
    got = oracle.swa_prefill(q, k, v, 1)
    assert np.array_equal(got, np.repeat(v, 2, axis=1))
    got = oracle.swa_prefill(q, k, v, 0)
    assert np.allclose(got[0], np.repeat(v[0:1], 2, axis=1)[0], atol=1e-15, rtol=0)


def test_gqa_equals_repeated_mha():
    L, Hq, Hkv, D, W = 90, 8, 2, 16, 20
    q, k, v = _rand((L, Hq, D), 15), _rand((L, Hkv, D), 16), _rand((L, Hkv, D), 17)
    got = oracle.swa_prefill(q, k, v, W)
    ref = oracle.swa_prefill(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), W)
    assert np.max(np.abs(got - ref)) == 0.0


def test_rows_subset_and_batch():
    B, L, Hq, Hkv, D, W = 2, 70, 4, 2, 8, 9
    q, k, v = _rand((B, L, Hq, D), 18), _rand((B, L, Hkv, D), 19), _rand((B, L, Hkv, D), 20)
    full = oracle.swa_prefill(q, k, v, W)
    rows = np.array([69, 0, 8, 9, 10, 33])
    part = oracle.swa_prefill(q, k, v, W, rows=rows)
    assert np.max(np.abs(full[:, rows] - part)) <= 1e-15
    for b in range(B):
        assert np.max(np.abs(full[b] - oracle.swa_prefill(q[b], k[b], v[b], W))) <= 1e-15


@pytest.mark.parametrize("W", [1, 5, 16, 40, 0])
def test_decode_equals_last_prefill_row(W):
    L, Hq, Hkv, D = 40, 4, 2, 8
    q, k, v = _rand((L, Hq, D), 21), _rand((L, Hkv, D), 22), _rand((L, Hkv, D), 23)
    pre = oracle.swa_prefill(q, k, v, W)
    for p in (0, 1, 3, 15, 16, 39):
        kseq = k[None].transpose(0, 2, 1, 3)[..., : p + 1, :]
        vseq = v[None].transpose(0, 2, 1, 3)[..., : p + 1, :]
        dec = oracle.swa_decode(q[p][None], kseq, vseq, [0], [p], W)
        assert np.max(np.abs(dec[0] - pre[p])) <= 1e-13


def test_key_permutation_invariance():
    rng = np.random.default_rng(24)
    q, k, v = rng.standard_normal((1, 8)), rng.standard_normal((30, 8)), rng.standard_normal((30, 8))
    mask = rng.random((1, 30)) < 0.5
    mask[0, 3] = True
    perm = rng.permutation(30)
    a = oracle.attend_masked(q, k, v, mask, 0.3)
    b = oracle.attend_masked(q, k[perm], v[perm], mask[:, perm], 0.3)
    assert np.max(np.abs(a - b)) <= 1e-14


def test_int8_decode_equals_sdpa_on_dequantized():
    B, Hq, Hkv, D, T8, Th = 2, 4, 2, 16, 96, 13
    rng = np.random.default_rng(25)
    kc = rng.integers(-127, 128, size=(B, Hkv, T8, D), dtype=np.int8)
    vc = rng.integers(-127, 128, size=(B, Hkv, T8, D), dtype=np.int8)
    ks = rng.random((B, Hkv, T8 // 32)).astype(np.float32) * 0.05
    vs = rng.random((B, Hkv, T8 // 32)).astype(np.float32) * 0.05
    kh, vh = rng.standard_normal((B, Hkv, Th, D)), rng.standard_normal((B, Hkv, Th, D))
    q = rng.standard_normal((B, Hq, D))
    got = oracle.attn_decode_int8kv(q, kc, ks, vc, vs, kh, vh)
    # independent dequantisation: per-token scale via torch.repeat_interleave
    tks = torch.from_numpy(ks.astype(np.float64)).repeat_interleave(32, dim=2)[..., None]
    tvs = torch.from_numpy(vs.astype(np.float64)).repeat_interleave(32, dim=2)[..., None]
    tk = torch.cat([torch.from_numpy(kc).double() * tks, torch.from_numpy(kh)], dim=2)
    tv = torch.cat([torch.from_numpy(vc).double() * tvs, torch.from_numpy(vh)], dim=2)
    tq = torch.from_numpy(q)[:, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, enable_gqa=True)[:, :, 0]
    assert np.max(np.abs(got - ref.numpy())) <= 1e-12


def brute_blocksparse_row(q, k, v, i, h, sel_row, block, W, scale):
    Hq, Hkv = q.shape[1], k.shape[1]
    g = h // (Hq // Hkv)
    keys = [j for j in range(i + 1) if (i - j < W) or (j // block in set(int(x) for x in sel_row if x >= 0))]
    s = [scale * math.fsum(q[i, h] * k[j, g]) for j in keys]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    z = math.fsum(e)
    return np.array([math.fsum(e[t] * v[keys[t], g, d] for t in range(len(keys))) / z
                     for d in range(q.shape[2])])


def test_blocksparse_bruteforce():
    L, Hq, Hkv, D, block, topk, W = 48, 4, 2, 4, 4, 3, 6
    q, k, v = _rand((L, Hq, D), 26), _rand((L, Hkv, D), 27), _rand((L, Hkv, D), 28)
    sel = oracle.block_select(q, k, block, topk)
    got = oracle.blocksparse_attend(q, k, v, sel, block, W, 0.5)
    for i in range(L):
        for h in range(Hq):
            ref = brute_blocksparse_row(q, k, v, i, h, sel[h, i // block], block, W, 0.5)
            assert np.max(np.abs(got[i, h] - ref)) <= 1e-12


def test_blocksparse_reductions():
    L, Hq, Hkv, D, block = 256, 4, 2, 8, 16
    q, k, v = _rand((L, Hq, D), 29), _rand((L, Hkv, D), 30), _rand((L, Hkv, D), 31)
    # top-0: only the local window
    sel0 = oracle.block_select(q, k, block, 0)
    assert np.max(np.abs(oracle.blocksparse_attend(q, k, v, sel0, block, 40)
                         - oracle.swa_prefill(q, k, v, 40))) <= 1e-13
    # window covering everything: full causal whatever is selected
    sel = oracle.block_select(q, k, block, 2)
    assert np.max(np.abs(oracle.blocksparse_attend(q, k, v, sel, block, L)
                         - oracle.swa_prefill(q, k, v, 0))) <= 1e-13
    # topk >= number of blocks and a window of one block (covers the diagonal
    # block): every earlier block kept -> full causal
    selall = oracle.block_select(q, k, block, L // block)
    assert np.max(np.abs(oracle.blocksparse_attend(q, k, v, selall, block, block)
                         - oracle.swa_prefill(q, k, v, 0))) <= 1e-13


def test_synth_bf16_rounding_and_determinism():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.0078125, 3.4e38, 1e-40], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(x)
    # 1+2^-8 is a tie -> even (1.0); 1+1.5*2^-8 rounds up to 1+2^-7
    assert list(synth.bf16_bits_to_f32(bits)[:3]) == [1.0, 1.0, 1.0078125]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    a = synth.token_major(9, synth.Q, 40, 3, 8)
    b = synth.token_major(9, synth.Q, 40, 3, 8)
    assert np.array_equal(a, b)
    h1 = synth.normal(9, synth.Q, (3, 40, 8), 1)
    assert np.array_equal(a.transpose(1, 0, 2), h1)
    o = synth.head_major(9, synth.K, 2, 2, 4096, 8, dtype="f32", outlier_p=0.01)
    frac = np.mean(np.abs(o) > 6.0)
    assert 0.003 < frac < 0.02
