"""GPU parity: swa_prefill (bf16 MFMA path and fp32 path) against the CPU oracle."""

import numpy as np
import pytest
import torch

import hybrid_swa_kv_amd as hsk
import oracle
from hybrid_swa_kv_amd import synth
from tests.helpers import bf16_excess, F32_TOL, announce, dev, f64, gpu_bf16, max_abs, out_f64

pytestmark = pytest.mark.gpu


def _case(seed, B, L, Hq, Hkv, D, dtype):
    q = synth.token_major(seed, synth.Q, L, Hq, D, dtype, B=B)
    k = synth.token_major(seed, synth.K, L, Hkv, D, dtype, B=B)
    v = synth.token_major(seed, synth.V, L, Hkv, D, dtype, B=B)
    return q, k, v


def test_tiny_window_fp32_config():
    # 1 sequence, L=512, 2 heads, head_dim 64, window 128, fp32, scale 1/8
    announce("prefill_f32_512")
    q, k, v = _case(1, None, 512, 2, 2, 64, "f32")
    out = hsk.swa_prefill(torch.from_numpy(q).to(dev()), torch.from_numpy(k).to(dev()),
                          torch.from_numpy(v).to(dev()), 128, scale=1 / 8)
    ref = oracle.swa_prefill(q, k, v, 128, 1 / 8)
    assert out.shape == (512, 2, 64)
    assert max_abs(out_f64(out), ref) <= F32_TOL


@pytest.mark.parametrize("B,L,Hq,Hkv,D,W", [(None, 37, 4, 2, 128, 5), (None, 200, 2, 1, 64, 0), (None, 130, 3, 3, 64, 64),
                                             (None, 300, 4, 2, 128, 0), (2, 193, 4, 1, 128, 129)])
def test_fp32_small(B, L, Hq, Hkv, D, W):
    # several 64-key blocks per row (full causal at L 300; window 129), GQA, a batch of 2
    announce("prefill_f32", B=B, L=L, Hq=Hq, Hkv=Hkv, D=D, W=W)
    q, k, v = _case(2, B, L, Hq, Hkv, D, "f32")
    out = hsk.swa_prefill(torch.from_numpy(q).to(dev()), torch.from_numpy(k).to(dev()),
                          torch.from_numpy(v).to(dev()), W)
    assert max_abs(out_f64(out), oracle.swa_prefill(q, k, v, W)) <= F32_TOL


CASES = [
    # (L, Hq, Hkv, D, W)
    (1, 2, 2, 128, 128), (2, 4, 1, 128, 1), (63, 2, 2, 64, 0), (64, 4, 1, 128, 64),
    (65, 8, 2, 128, 64), (127, 2, 2, 128, 127), (128, 4, 2, 64, 128), (129, 8, 2, 128, 129),
    (300, 4, 4, 128, 1), (513, 8, 2, 128, 100), (1000, 8, 2, 128, 0), (1000, 4, 1, 64, 256),
    (777, 16, 2, 128, 1024), (2048, 8, 1, 128, 333), (259, 3, 1, 128, 70), (190, 6, 2, 64, 0),
]


@pytest.mark.parametrize("L,Hq,Hkv,D,W", CASES)
def test_bf16_parity(L, Hq, Hkv, D, W):
    announce("prefill_bf16", L=L, Hq=Hq, Hkv=Hkv, D=D, W=W)
    q, k, v = _case(3 + L, None, L, Hq, Hkv, D, "bf16")
    out = hsk.swa_prefill(gpu_bf16(q), gpu_bf16(k), gpu_bf16(v), W)
    ref = oracle.swa_prefill(f64(q), f64(k), f64(v), W)
    ex = bf16_excess(out_f64(out), ref)
    assert ex <= 0, (ex, max_abs(out_f64(out), ref))


def _block_edge_rows(L, seed, extra=64):
    edges = np.arange(0, L, 128)
    rnd = np.random.default_rng(seed).integers(0, L, size=extra)
    rows = np.concatenate([edges, edges - 1, edges + 31, edges + 127, [L - 2, L - 1], rnd])
    return np.unique(rows[(rows >= 0) & (rows < L)]).astype(np.int64)


@pytest.mark.parametrize("L,W", [(8190, 128), (8325, 1024)])
def test_bf16_64_heads_block_edges(L, W):
    """64 query heads (8 per KV head) over about 8K rows, as in the long-context
    workloads; rows around every 128-row query block edge and the ragged end."""
    Hq, Hkv, D = 64, 8, 128
    announce("prefill_bf16_64_heads", L=L, Hq=Hq, W=W)
    q, k, v = _case(40 + L, None, L, Hq, Hkv, D, "bf16")
    out = hsk.swa_prefill(gpu_bf16(q), gpu_bf16(k), gpu_bf16(v), W)
    rows = _block_edge_rows(L, L)
    got = out_f64(out)[rows]
    ref = oracle.swa_prefill(f64(q), f64(k), f64(v), W, rows=rows)
    ex = bf16_excess(got, ref)
    assert ex <= 0, (ex, max_abs(got, ref))


def test_bf16_batch_and_ring_output():
    B, L, Hq, Hkv, D, W = 3, 300, 4, 2, 128, 96
    announce("prefill_bf16_batch_ring", B=B, L=L)
    q, k, v = _case(5, B, L, Hq, Hkv, D, "bf16")
    rk = torch.full((B, Hkv, W, D), 7.0, dtype=torch.bfloat16, device=dev())
    rv = torch.full((B, Hkv, W, D), -7.0, dtype=torch.bfloat16, device=dev())
    out = hsk.swa_prefill(gpu_bf16(q), gpu_bf16(k), gpu_bf16(v), W, ring_k=rk, ring_v=rv)
    ref = oracle.swa_prefill(f64(q), f64(k), f64(v), W)
    assert bf16_excess(out_f64(out), ref) <= 0
    kseq = np.ascontiguousarray(f64(k).transpose(0, 2, 1, 3))
    vseq = np.ascontiguousarray(f64(v).transpose(0, 2, 1, 3))
    init_k = np.full((B, Hkv, W, D), 7.0)
    init_v = np.full((B, Hkv, W, D), -7.0)
    exp_k = oracle.ring_fill(kseq, [0] * B, [L - 1] * B, W, init_k)
    exp_v = oracle.ring_fill(vseq, [0] * B, [L - 1] * B, W, init_v)
    assert np.array_equal(out_f64(rk), exp_k)
    assert np.array_equal(out_f64(rv), exp_v)


def test_deterministic():
    L, Hq, Hkv, D = 700, 8, 2, 128
    q, k, v = _case(6, None, L, Hq, Hkv, D, "bf16")
    a = hsk.swa_prefill(gpu_bf16(q), gpu_bf16(k), gpu_bf16(v), 200)
    b = hsk.swa_prefill(gpu_bf16(q), gpu_bf16(k), gpu_bf16(v), 200)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
