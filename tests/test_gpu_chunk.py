"""GPU parity: swa_prefill_chunk, chunk after chunk, carrying the ring."""

import numpy as np
import pytest
import torch

import hybrid_swa_kv_amd as hsk
import oracle
from hybrid_swa_kv_amd import synth
from tests.helpers import announce, bf16_excess, f64, gpu_bf16, max_abs, out_f64

pytestmark = pytest.mark.gpu


def _run_chunks(seed, B, L, C, Hq, Hkv, D, W, check_rows=None):
    q = synth.token_major(seed, synth.Q, L, Hq, D, B=B)
    k = synth.token_major(seed, synth.K, L, Hkv, D, B=B)
    v = synth.token_major(seed, synth.V, L, Hkv, D, B=B)
    dq, dk, dv = gpu_bf16(q), gpu_bf16(k), gpu_bf16(v)
    # slots never written hold garbage: they must never be read
    rk = gpu_bf16(synth.head_major(seed, synth.MISC, B, Hkv, W, D))
    rv = gpu_bf16(synth.head_major(seed, synth.MISC + 1, B, Hkv, W, D))
    out = torch.empty_like(dq)
    for pos0 in range(0, L, C):
        c = min(C, L - pos0)
        sl = slice(pos0, pos0 + c)
        oc = hsk.swa_prefill_chunk(dq[:, sl].contiguous(), dk[:, sl].contiguous(), dv[:, sl].contiguous(), rk, rv,
                                   pos0)
        out[:, sl] = oc
    torch.cuda.synchronize()
    return q, k, v, out, rk, rv


@pytest.mark.parametrize("L,C,W,Hq,Hkv,D", [
    (1636, 512, 1024, 8, 2, 128),   # window longer than a chunk, ragged last chunk
    (1636, 512, 128, 8, 2, 128),
    (1000, 256, 128, 4, 4, 64),
    (700, 128, 64, 16, 1, 128),
])
def test_chunked_prefill_equals_one_shot(L, C, W, Hq, Hkv, D):
    announce("prefill_chunk", L=L, C=C, W=W, Hq=Hq, Hkv=Hkv, D=D)
    B = 2
    q, k, v, out, rk, rv = _run_chunks(800 + W + C, B, L, C, Hq, Hkv, D, W)
    ref = oracle.swa_prefill(f64(q), f64(k), f64(v), W)
    ex = bf16_excess(out_f64(out), ref)
    assert ex <= 0, (ex, max_abs(out_f64(out), ref))
    # the ring holds the last W positions, bit for bit
    held = oracle.ring_positions(L - 1, W)
    got_k, got_v = out_f64(rk), out_f64(rv)
    for s in range(W):
        assert np.array_equal(got_k[:, :, s], f64(k)[:, held[s]])
        assert np.array_equal(got_v[:, :, s], f64(v)[:, held[s]])


def test_chunked_prefill_131072_in_4096_chunks_sampled():
    """The hybrid-layer prefill shape (L 131072, 64/8 heads, window 1024) as 32
    chunks of 4096; sampled rows of several chunks against the oracle."""
    announce("prefill_chunk_131072")
    L, C, W, Hq, Hkv, D = 131072, 4096, 1024, 64, 8, 128
    q, k, v, out, rk, rv = _run_chunks(880, 1, L, C, Hq, Hkv, D, W)
    rows = np.array([0, 1, 1023, 1024, 4095, 4096, 4097, 5120, 65535, 65536, 99999, 131071], dtype=np.int64)
    ref = oracle.swa_prefill(f64(q), f64(k), f64(v), W, rows=rows)
    got = out_f64(out)[:, rows]
    ex = bf16_excess(got, ref)
    assert ex <= 0, (ex, max_abs(got, ref))
    held = oracle.ring_positions(L - 1, W)
    assert np.array_equal(out_f64(rk)[0, :, 5], f64(k)[0, held[5]])


def test_chunks_of_8192_rows_sampled():
    """Chunks of 8192 rows with 64 query heads; rows around query block edges of
    both chunks and the chunk boundary."""
    L, C, W, Hq, Hkv, D = 16384, 8192, 1024, 64, 8, 128
    announce("prefill_chunk_8192", L=L, C=C, W=W)
    q, k, v, out, rk, rv = _run_chunks(890, 1, L, C, Hq, Hkv, D, W)
    edges = np.arange(0, L, 128)
    rnd = np.random.default_rng(5).integers(0, L, size=48)
    rows = np.concatenate([edges[::3], edges[1::3] - 1, edges[2::3] + 127, [C - 1, C, C + 1, L - 1], rnd])
    rows = np.unique(rows[(rows >= 0) & (rows < L)]).astype(np.int64)
    ref = oracle.swa_prefill(f64(q), f64(k), f64(v), W, rows=rows)
    got = out_f64(out)[:, rows]
    ex = bf16_excess(got, ref)
    assert ex <= 0, (ex, max_abs(got, ref))


def test_chunked_prefill_window_limit():
    """W = 65536, longer than the sequence: every chunk reads the whole earlier
    prefix from the ring (full causal attention); slots past the sequence keep
    their garbage, written by no chunk and read by none."""
    L, C, W, Hq, Hkv, D = 1636, 512, 65536, 8, 2, 128
    announce("prefill_chunk_W65536", L=L, C=C, W=W)
    B = 2
    q, k, v, out, rk, rv = _run_chunks(870, B, L, C, Hq, Hkv, D, W)
    ref = oracle.swa_prefill(f64(q), f64(k), f64(v), W)
    ex = bf16_excess(out_f64(out), ref)
    assert ex <= 0, (ex, max_abs(out_f64(out), ref))
    got_k, got_v = rk.view(torch.int16).cpu().numpy(), rv.view(torch.int16).cpu().numpy()
    assert np.array_equal(got_k[:, :, :L].view(np.uint16), np.ascontiguousarray(k.transpose(0, 2, 1, 3)))
    assert np.array_equal(got_v[:, :, :L].view(np.uint16), np.ascontiguousarray(v.transpose(0, 2, 1, 3)))
    assert np.array_equal(got_k[:, :, L:].view(np.uint16), synth.head_major(870, synth.MISC, B, Hkv, W, D)[:, :, L:])
    assert np.array_equal(got_v[:, :, L:].view(np.uint16),
                          synth.head_major(870, synth.MISC + 1, B, Hkv, W, D)[:, :, L:])
