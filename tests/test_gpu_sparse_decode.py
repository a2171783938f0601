"""GPU parity: block means of the INT8 pool and the top-k block-sparse decode over
the hot + INT8 pool (kv_block_means_int8, attn_decode_int8kv_sparse)."""

import numpy as np
import pytest
import torch

import hybrid_swa_kv_amd as hsk
import oracle
from hybrid_swa_kv_amd import synth
from tests.helpers import announce, bf16_excess, f64, gpu_bf16, max_abs, out_f64
from tests.test_gpu_blocksparse import near_tie_bound

pytestmark = pytest.mark.gpu


def _pool(seed, B, Hq, Hkv, D, T8, Th):
    kx = synth.head_major(seed, synth.K, B, Hkv, T8 + Th, D, outlier_p=0.01)
    vx = synth.head_major(seed, synth.V, B, Hkv, T8 + Th, D, outlier_p=0.01)
    q = synth.normal(seed, synth.Q, (B, Hq, D), 1)
    return q, kx, vx


def _gpu_pool(q, kx, vx, T8):
    """Codes and scales from the GPU encoder (bit-exact with the oracle's, tested
    elsewhere), means from the GPU kernel."""
    kc, ks = hsk.kv_quant_int8_b32(gpu_bf16(np.ascontiguousarray(kx[:, :, :T8])))
    vc, vs = hsk.kv_quant_int8_b32(gpu_bf16(np.ascontiguousarray(vx[:, :, :T8])))
    km = hsk.kv_block_means_int8(kc, ks)
    kh = gpu_bf16(np.ascontiguousarray(kx[:, :, T8:]))
    vh = gpu_bf16(np.ascontiguousarray(vx[:, :, T8:]))
    return kc, ks, vc, vs, km, kh, vh


def check_rows(sel_gpu, scores, topk, rows):
    """Kept blocks equal the oracle's, except where a block sits at an fp64 near-tie
    with the cut (the order of an fp64 dot product is not fixed).  Returns the
    number of rows that needed that acceptance; it is printed and bounded."""
    near = 0
    for (b, h) in rows:
        n = scores.shape[-1]
        got = sel_gpu[b, h]
        sc = scores[b, h]
        k = min(n, topk)
        want = np.sort(np.argsort(-sc, kind="stable")[:k])
        if np.array_equal(got[:k], want) and (got[k:] == -1).all():
            continue
        a, c = set(got[got >= 0]), set(want)
        assert len(a) == len(c) == k, (b, h)
        cut = np.sort(sc)[::-1][k - 1]
        tol = 1e-12 * max(1.0, float(np.max(np.abs(sc))))
        for j in a ^ c:
            assert abs(sc[j] - cut) <= tol, ("selection differs away from a tie", b, h, j)
        assert np.array_equal(got[:k], np.sort(got[:k]))
        near += 1
    print(f"[select] near-tie rows: {near} of {len(rows)}", flush=True)
    assert near <= near_tie_bound(len(rows)), ("too many near-tie rows", near, len(rows))
    return near


@pytest.mark.parametrize("B,Hq,Hkv,D,T8,Th,topk", [
    (2, 8, 2, 128, 4096, 256, 16),
    (1, 16, 1, 128, 2048, 100, 8),     # 16 heads per group
    (2, 4, 4, 64, 1024, 33, 5),        # head_dim 64
    (2, 8, 2, 128, 320, 64, 64),       # fewer blocks than topk: every block kept
    (2, 8, 2, 128, 640, 64, 0),        # no block kept: the hot tail alone
    (2, 8, 2, 128, 0, 70, 16),         # no INT8 region
    (1, 8, 2, 128, 131072, 32, 64),    # 4096 blocks
    (1, 8, 1, 128, 22400, 64, 16),     # 700 blocks, 8 heads per group
    (1, 8, 2, 128, 32768, 64, 256),    # topk at its limit, 1024 blocks to choose from
    (2, 8, 2, 64, 12800, 40, 100),     # topk above 64, 400 blocks
])
def test_sparse_decode_parity(B, Hq, Hkv, D, T8, Th, topk):
    announce("sparse_decode", B=B, Hq=Hq, Hkv=Hkv, D=D, T8=T8, Th=Th, topk=topk)
    seed = 1200 + T8 // 32 + topk
    q, kx, vx = _pool(seed, B, Hq, Hkv, D, T8, Th)
    kc, ks, vc, vs, km, kh, vh = _gpu_pool(q, kx, vx, T8) if T8 else (None,) * 5 + (
        gpu_bf16(np.ascontiguousarray(kx)), gpu_bf16(np.ascontiguousarray(vx)))
    out, sel = hsk.attn_decode_int8kv_sparse(gpu_bf16(q), kc, ks, vc, vs, km, kh, vh, topk=topk)
    torch.cuda.synchronize()
    sel_np = sel.cpu().numpy()
    okc, oks = oracle.kv_quant_int8_b32(synth.bf16_bits_to_f32(kx[:, :, :T8]))
    ovc, ovs = oracle.kv_quant_int8_b32(synth.bf16_bits_to_f32(vx[:, :, :T8]))
    if T8:
        means = oracle.int8_block_means(okc, oks)
        assert np.array_equal(km.cpu().numpy(), means.transpose(0, 1, 3, 2))    # bit-exact means
        if topk:
            _, scores = oracle.sparse_select(f64(q), means, topk, return_scores=True)
            check_rows(sel_np, scores, topk, [(b, h) for b in range(B) for h in range(Hq)])
    else:
        assert (sel_np == -1).all()
    ref = oracle.attn_decode_int8kv_sparse(f64(q), okc, oks, ovc, ovs, f64(kx[:, :, T8:]), f64(vx[:, :, T8:]),
                                           sel_np)
    ex = bf16_excess(out_f64(out), ref)
    assert ex <= 0, (ex, max_abs(out_f64(out), ref))
