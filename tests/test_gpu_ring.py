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


def test_negative_position_skips_the_sequence():
    """A sequence whose pos is negative (nothing to decode) is skipped: its ring
    and its slot_out entry keep their bytes and its output rows are zero, while
    the other sequences of the batch are decoded as usual."""
    B, Hq, Hkv, D, W = 4, 8, 2, 128, 128
    pos = np.array([5, -1, 300, -7], dtype=np.int64)
    announce("ring_negative_pos", B=B, W=W, pos=list(pos))
    q = synth.normal(711, synth.Q, (B, Hq, D), 1)
    kn = synth.normal(711, synth.K_NEW, (B, Hkv, D), 1)
    vn = synth.normal(711, synth.V_NEW, (B, Hkv, D), 1)
    rk_bits = synth.head_major(711, synth.K, B, Hkv, W, D)
    rv_bits = synth.head_major(711, synth.V, B, Hkv, W, D)
    d_rk, d_rv = gpu_bf16(rk_bits), gpu_bf16(rv_bits)
    slot_out = torch.full((B,), -99, dtype=torch.int32, device="cuda")
    d_pos = torch.from_numpy(pos.astype(np.int32)).cuda()
    out, slots = hsk.swa_decode_ring(gpu_bf16(q), gpu_bf16(kn), gpu_bf16(vn), d_rk, d_rv, d_pos, slot_out=slot_out)
    got_out, got_rk, got_rv = out_f64(out), out_f64(d_rk), out_f64(d_rv)
    got_slots = slots.cpu().numpy()
    rk0, rv0 = f64(rk_bits), f64(rv_bits)
    for b in (1, 3):
        assert np.all(got_out[b] == 0.0)
        assert np.array_equal(got_rk[b], rk0[b]) and np.array_equal(got_rv[b], rv0[b])
        assert got_slots[b] == -99
    for b in (0, 2):
        p = int(pos[b])
        exp_rk = oracle.ring_append(rk0[b:b + 1], [p], f64(kn)[b:b + 1])
        exp_rv = oracle.ring_append(rv0[b:b + 1], [p], f64(vn)[b:b + 1])
        assert got_slots[b] == int(oracle.ring_slot(p, W))
        assert np.array_equal(got_rk[b:b + 1], exp_rk) and np.array_equal(got_rv[b:b + 1], exp_rv)
        # the logical sequence the ring now holds: positions max(0, p-W+1) .. p
        first = max(0, p - W + 1)
        slots_seq = [int(oracle.ring_slot(t, W)) for t in range(first, p + 1)]
        kseq = exp_rk[:, :, slots_seq]
        vseq = exp_rv[:, :, slots_seq]
        ref = oracle.swa_decode(f64(q)[b:b + 1], kseq, vseq, [first], [p], W)
        ex = bf16_excess(got_out[b:b + 1], ref)
        assert ex <= 0, (b, ex, max_abs(got_out[b:b + 1], ref))
