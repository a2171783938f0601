"""GPU parity: swa_decode_ring (ring append, slot map, window attention)."""

import numpy as np
import pytest
import torch

import hybrid_swa_kv_amd as hsk
import oracle
from hybrid_swa_kv_amd import synth
from tests.helpers import bf16_excess, announce, f64, gpu_bf16, max_abs, out_f64

pytestmark = pytest.mark.gpu


def run_case(seed, B, Hq, Hkv, D, W, pos):
    """Logical K/V of positions pos-W .. pos per sequence; the ring holds 0..pos-1."""
    pos = np.asarray(pos, dtype=np.int64)
    P = W + 1
    start = pos - W                                  # may be negative: those rows are unused
    kseq = synth.head_major(seed, synth.K, B, Hkv, P, D)
    vseq = synth.head_major(seed, synth.V, B, Hkv, P, D)
    q = synth.normal(seed, synth.Q, (B, Hq, D), 1)
    # the slot of a never-written position holds garbage on purpose
    junk_k = synth.head_major(seed, synth.MISC, B, Hkv, W, D)
    junk_v = synth.head_major(seed, synth.MISC + 1, B, Hkv, W, D)
    kf, vf = f64(kseq), f64(vseq)
    rk_pre = np.empty_like(f64(junk_k))
    rv_pre = np.empty_like(rk_pre)
    for b in range(B):
        s0 = int(start[b])
        off = max(0, -s0)
        seq_k = kf[b:b + 1, :, off:]
        seq_v = vf[b:b + 1, :, off:]
        rk_pre[b] = oracle.ring_fill(seq_k, [s0 + off], [int(pos[b]) - 1], W, f64(junk_k)[b:b + 1])[0]
        rv_pre[b] = oracle.ring_fill(seq_v, [s0 + off], [int(pos[b]) - 1], W, f64(junk_v)[b:b + 1])[0]
    # device tensors: ring pre-state in bf16 (exact: every value came from bf16)
    to_bits = lambda x: synth.f32_to_bf16_bits(x.astype(np.float32))
    d_rk = gpu_bf16(to_bits(rk_pre))
    d_rv = gpu_bf16(to_bits(rv_pre))
    k_new = np.ascontiguousarray(kseq[:, :, W, :])
    v_new = np.ascontiguousarray(vseq[:, :, W, :])
    d_pos = torch.from_numpy(pos.astype(np.int32)).cuda()
    out, slots = hsk.swa_decode_ring(gpu_bf16(q), gpu_bf16(k_new), gpu_bf16(v_new), d_rk, d_rv, d_pos)
    # expected
    ref = np.empty((B, Hq, D))
    for b in range(B):
        s0 = int(start[b])
        off = max(0, -s0)
        ref[b] = oracle.swa_decode(f64(q)[b:b + 1], kf[b:b + 1, :, off:], vf[b:b + 1, :, off:],
                                   [s0 + off], [int(pos[b])], W)[0]
    exp_rk = oracle.ring_append(rk_pre, pos, f64(k_new))
    exp_rv = oracle.ring_append(rv_pre, pos, f64(v_new))
    assert np.array_equal(slots.cpu().numpy(), oracle.ring_slot(pos, W))
    assert np.array_equal(out_f64(d_rk), exp_rk)
    assert np.array_equal(out_f64(d_rv), exp_rv)
    ex = bf16_excess(out_f64(out), ref)
    assert ex <= 0, (ex, max_abs(out_f64(out), ref))


@pytest.mark.parametrize("W", [1, 16, 128, 200, 640, 1024])
def test_ring_positions(W):
    B = 7
    pos = [0, 1, max(0, W - 2), W - 1, W, W + 1, 12345]
    announce("ring", W=W)
    run_case(20 + W, B, 8, 2, 128, W, pos)


@pytest.mark.parametrize("Hq,Hkv,D", [(4, 4, 64), (16, 1, 128), (12, 4, 128), (32, 2, 64), (64, 2, 128)])
def test_ring_heads(Hq, Hkv, D):
    announce("ring_heads", Hq=Hq, Hkv=Hkv, D=D)
    rng = np.random.default_rng(Hq * 10 + D)
    pos = rng.integers(0, 5000, size=5)
    run_case(30 + Hq, 5, Hq, Hkv, D, 128, pos)


def test_ring_large_window():
    announce("ring_W1024")
    run_case(41, 4, 8, 2, 128, 1024, [0, 500, 1023, 99999])


def test_ring_decode_workload():
    # batch 32, context 32768 (query at position 32767), 32/8 heads, head_dim 128, window 128
    announce("ring_workload")
    run_case(2, 32, 32, 8, 128, 128, [32767] * 32)


def test_ring_window_limit():
    """W = 65536, the largest ring: a fresh sequence, one that fills the ring
    exactly and one that has wrapped."""
    announce("ring_W65536")
    run_case(43, 3, 4, 1, 64, 65536, [0, 65535, 70000])
