"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

Integer outputs (INT8 codes, scales, selected blocks) are compared exactly over
whole units; attention outputs on seeded samples the oracle can compute one by one.
Inputs come from the same seeded generators as every other test.
"""

import numpy as np
import pytest
import torch

import hybrid_swa_kv_amd as hsk
import oracle
from hybrid_swa_kv_amd import synth
from tests.helpers import announce, bf16_excess, gpu_bf16, max_abs, out_f64
from tests.test_gpu_blocksparse import check_selection

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _rows(L, extra, seed):
    fixed = [0, 1, 2, 63, 64, 127, 128, 1022, 1023, 1024, 1025, 2047, 2048, 4159, 4160, L // 2, L - 2, L - 1]
    rnd = np.random.default_rng(seed).integers(0, L, size=extra)
    return np.unique(np.concatenate([fixed, rnd]).astype(np.int64))


@pytest.fixture(scope="module")
def prefill_inputs():
    L, Hq, Hkv, D = 131072, 64, 8, 128
    q = synth.token_major(3, synth.Q, L, Hq, D)
    k = synth.token_major(3, synth.K, L, Hkv, D)
    v = synth.token_major(3, synth.V, L, Hkv, D)
    return q, k, v


@pytest.mark.parametrize("W", [1024, 0])
def test_prefill_131072_sampled(prefill_inputs, W):
    q, k, v = prefill_inputs
    L = q.shape[0]
    announce("prefill_full_size", L=L, W=W)
    out = hsk.swa_prefill(gpu_bf16(q), gpu_bf16(k), gpu_bf16(v), W)
    rows = _rows(L, 12, 7 + W)
    got = synth.from_torch_bf16(out[torch.from_numpy(rows).cuda()]).astype(np.float64)
    del out
    ref = oracle.swa_prefill(synth.bf16_bits_to_f32(q), synth.bf16_bits_to_f32(k),
                             synth.bf16_bits_to_f32(v), W, rows=rows)
    ex = bf16_excess(got, ref)
    assert ex <= 0, (ex, max_abs(got, ref))


def test_int8_decode_65536():
    B, Hq, Hkv, D, T, hot = 16, 32, 8, 128, 65536, 2048
    T8 = T - hot
    G = Hq // Hkv
    announce("int8_full_size", B=B, T=T)
    kx = synth.head_major(4, synth.K, B, Hkv, T, D, outlier_p=0.01)
    vx = synth.head_major(4, synth.V, B, Hkv, T, D, outlier_p=0.01)
    q = synth.normal(4, synth.Q, (B, Hq, D), 1)
    dk, dv = gpu_bf16(kx), gpu_bf16(vx)
    kc, ks = hsk.kv_quant_int8_b32(dk[:, :, :T8].contiguous())
    vc, vs = hsk.kv_quant_int8_b32(dv[:, :, :T8].contiguous())
    out = hsk.attn_decode_int8kv(gpu_bf16(q), kc, ks, vc, vs, dk[:, :, T8:].contiguous(), dv[:, :, T8:].contiguous())
    got = out_f64(out)
    units = [(0, 0), (3, 5), (7, 7), (9, 2), (15, 7), (11, 0)]
    for b, g in units:
        okc, oks = oracle.kv_quant_int8_b32(synth.bf16_bits_to_f32(kx[b, g, :T8]))
        ovc, ovs = oracle.kv_quant_int8_b32(synth.bf16_bits_to_f32(vx[b, g, :T8]))
        assert np.array_equal(kc[b, g].cpu().numpy(), okc)
        assert np.array_equal(vc[b, g].cpu().numpy(), ovc)
        assert np.array_equal(ks[b, g].cpu().numpy().view(np.uint32), oks.view(np.uint32))
        assert np.array_equal(vs[b, g].cpu().numpy().view(np.uint32), ovs.view(np.uint32))
        hs = slice(g * G, (g + 1) * G)
        ref = oracle.attn_decode_int8kv(
            synth.bf16_bits_to_f32(q[b:b + 1, hs]).astype(np.float64),
            okc[None, None], oks[None, None], ovc[None, None], ovs[None, None],
            synth.bf16_bits_to_f32(kx[b:b + 1, g:g + 1, T8:]), synth.bf16_bits_to_f32(vx[b:b + 1, g:g + 1, T8:]))
        ex = bf16_excess(got[b:b + 1, hs], ref)
        assert ex <= 0, ((b, g), ex, max_abs(got[b:b + 1, hs], ref))


def test_blocksparse_131072():
    L, Hq, Hkv, D, block, topk, W = 131072, 32, 8, 128, 64, 64, 1024
    announce("blocksparse_full_size", L=L)
    q = synth.token_major(5, synth.Q, L, Hq, D)
    k = synth.token_major(5, synth.K, L, Hkv, D)
    v = synth.token_major(5, synth.V, L, Hkv, D)
    out, sel = hsk.blocksparse_select_attend(gpu_bf16(q), gpu_bf16(k), gpu_bf16(v), block, topk, W)
    sel_np = sel.cpu().numpy()
    rows = _rows(L, 10, 11)
    got = synth.from_torch_bf16(out[torch.from_numpy(rows).cuda()]).astype(np.float64)
    del out
    qf, kf, vf = synth.bf16_bits_to_f32(q), synth.bf16_bits_to_f32(k), synth.bf16_bits_to_f32(v)
    check_selection(sel_np, qf, kf, block, topk)          # every (head, query block), exact
    ref = oracle.blocksparse_attend(qf, kf, vf, sel_np, block, W, rows=rows)
    ex = bf16_excess(got, ref)
    assert ex <= 0, (ex, max_abs(got, ref))
