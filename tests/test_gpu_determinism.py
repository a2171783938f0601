"""Two calls on the same inputs give bit-identical results (fixed split, merge and
reduction orders): ring decode, block-sparse prefill, block-sparse INT8 decode and
chunked prefill.  The prefill and the dense INT8 decode are checked the same way
in their own files."""

import numpy as np
import pytest
import torch

import hybrid_swa_kv_amd as hsk
from hybrid_swa_kv_amd import synth
from tests.helpers import announce, gpu_bf16

pytestmark = pytest.mark.gpu


def same(a, b):
    torch.cuda.synchronize()
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    return torch.equal(a, b)


def test_ring_decode_repeatable():
    B, Hq, Hkv, D, W = 8, 32, 8, 128, 128
    announce("determinism_ring", B=B, W=W)
    q = synth.normal_gpu(700, synth.Q, (B, Hq, D))
    kn = synth.normal_gpu(700, synth.K_NEW, (B, Hkv, D))
    vn = synth.normal_gpu(700, synth.V_NEW, (B, Hkv, D))
    rk = synth.normal_gpu(700, synth.K, (B, Hkv, W, D))
    rv = synth.normal_gpu(700, synth.V, (B, Hkv, W, D))
    pos = torch.tensor(np.arange(B) * 977 + 5, dtype=torch.int32, device="cuda")
    # the append writes the same row into the same slot both times, so the ring
    # state is the same for the second call
    o1, s1 = hsk.swa_decode_ring(q, kn, vn, rk, rv, pos)
    ring_after = (rk.clone(), rv.clone())
    o2, s2 = hsk.swa_decode_ring(q, kn, vn, rk, rv, pos)
    assert same(o1, o2) and same(s1, s2)
    assert same(rk, ring_after[0]) and same(rv, ring_after[1])


def test_blocksparse_repeatable():
    L, Hq, Hkv, D = 4096, 8, 2, 128
    announce("determinism_blocksparse", L=L)
    q = gpu_bf16(synth.token_major(701, synth.Q, L, Hq, D))
    k = gpu_bf16(synth.token_major(701, synth.K, L, Hkv, D))
    v = gpu_bf16(synth.token_major(701, synth.V, L, Hkv, D))
    o1, s1 = hsk.blocksparse_select_attend(q, k, v, 64, 16, 512)
    o2, s2 = hsk.blocksparse_select_attend(q, k, v, 64, 16, 512)
    assert same(s1, s2) and same(o1, o2)


def test_sparse_int8_decode_repeatable():
    B, Hq, Hkv, D, T8, Th, topk = 4, 32, 8, 128, 8192, 512, 32
    announce("determinism_sparse_decode", B=B, T8=T8)
    q = synth.normal_gpu(702, synth.Q, (B, Hq, D))
    kx = synth.normal_gpu(702, synth.K, (B, Hkv, T8 + Th, D), outlier_p=0.01)
    vx = synth.normal_gpu(702, synth.V, (B, Hkv, T8 + Th, D), outlier_p=0.01)
    kc, ks = hsk.kv_quant_int8_b32(kx[:, :, :T8].contiguous())
    vc, vs = hsk.kv_quant_int8_b32(vx[:, :, :T8].contiguous())
    km = hsk.kv_block_means_int8(kc, ks)
    kh, vh = kx[:, :, T8:].contiguous(), vx[:, :, T8:].contiguous()
    o1, s1 = hsk.attn_decode_int8kv_sparse(q, kc, ks, vc, vs, km, kh, vh, topk=topk)
    o2, s2 = hsk.attn_decode_int8kv_sparse(q, kc, ks, vc, vs, km, kh, vh, topk=topk)
    assert same(s1, s2) and same(o1, o2)


def test_chunked_prefill_repeatable():
    B, C, Hq, Hkv, D, W = 1, 1024, 8, 2, 128, 256
    announce("determinism_chunk", C=C, W=W)
    q = synth.normal_gpu(703, synth.Q, (B, C, Hq, D))
    k = synth.normal_gpu(703, synth.K, (B, C, Hkv, D))
    v = synth.normal_gpu(703, synth.V, (B, C, Hkv, D))
    ring0 = (synth.normal_gpu(703, synth.K_NEW, (B, Hkv, W, D)), synth.normal_gpu(703, synth.V_NEW, (B, Hkv, W, D)))
    outs, rings = [], []
    for _ in range(2):
        rk, rv = ring0[0].clone(), ring0[1].clone()
        outs.append(hsk.swa_prefill_chunk(q, k, v, rk, rv, 2048))
        rings.append((rk, rv))
    assert same(outs[0], outs[1])
    assert same(rings[0][0], rings[1][0]) and same(rings[0][1], rings[1][1])
