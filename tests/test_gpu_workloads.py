"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

Integer outputs (INT8 codes, scales, selected blocks) are compared exactly over
every unit.  Attention outputs are compared in full where the oracle can afford
it (the INT8 decode, the bf16 full-attention decode layer, the 8192-token
prefill with the workload's heads) and otherwise on seeded samples the oracle
computes one by one: 512 query rows x all 64 heads of the 131072-token prefill,
256 whole (head, query block) tiles of the block-sparse prefill.  Inputs come
from the same seeded generators as every other test.  The oracle runs on a
thread pool (one task per head or unit, BLAS held to one thread each).
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

import hybrid_swa_kv_amd as hsk
import oracle
from hybrid_swa_kv_amd import synth
from tests.helpers import announce, bf16_excess, gpu_bf16, max_abs, out_f64
from tests.test_gpu_blocksparse import check_selection
from tests.test_gpu_sparse_decode import check_rows

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

WORKERS = max(1, min(16, os.cpu_count() or 1))


def pmap(fn, items):
    """fn over items on a thread pool (numpy releases the GIL in its loops); prints
    a progress line at every quarter."""
    items = list(items)
    out = []
    with threadpool_limits(1), ThreadPoolExecutor(WORKERS) as ex:
        for i, r in enumerate(ex.map(fn, items), 1):
            out.append(r)
            if i * 4 // len(items) != (i - 1) * 4 // len(items):
                print(f"[oracle] {i} of {len(items)}", flush=True)
    return out


def prefill_rows(L, n, seed):
    """n distinct query rows: the tile and window edges, then seeded random rows."""
    fixed = [0, 1, 2, 63, 64, 127, 128, 1022, 1023, 1024, 1025, 2047, 2048, 4159, 4160, L // 2, L - 2, L - 1]
    rng = np.random.default_rng(seed)
    rows = set(fixed)
    while len(rows) < n:
        rows.update(int(x) for x in rng.integers(0, L, size=n - len(rows)))
    return np.array(sorted(rows), dtype=np.int64)


def prefill_oracle_by_head(qf, kf, vf, W, rows=None):
    """oracle.swa_prefill one query head at a time (same definition, head-sliced)."""
    L, Hq, D = qf.shape
    Hkv = kf.shape[1]
    G = Hq // Hkv
    window_only = 0 < W < L
    # a window's keys sit right before each row: one row per oracle block keeps
    # the key span at W for scattered rows
    rb = 1 if (window_only and rows is not None) else 64

    def one(h):
        g = h // G
        return oracle.swa_prefill(qf[:, h:h + 1], kf[:, g:g + 1], vf[:, g:g + 1], W, rows=rows,
                                  row_block=rb)[:, 0]

    return np.stack(pmap(one, range(Hq)), axis=1)


@pytest.fixture(scope="module")
def prefill_inputs():
    L, Hq, Hkv, D = 131072, 64, 8, 128
    q = synth.token_major(3, synth.Q, L, Hq, D)
    k = synth.token_major(3, synth.K, L, Hkv, D)
    v = synth.token_major(3, synth.V, L, Hkv, D)
    return q, k, v


@pytest.mark.parametrize("W", [1024, 0])
def test_prefill_131072_512_rows_all_heads(prefill_inputs, W):
    """L 131072, 64/8 heads, D 128 (window 1024, then full causal): 512 rows x 64 heads."""
    q, k, v = prefill_inputs
    L = q.shape[0]
    announce("prefill_full_size", L=L, W=W)
    out = hsk.swa_prefill(gpu_bf16(q), gpu_bf16(k), gpu_bf16(v), W)
    rows = prefill_rows(L, 512, 7 + W)
    got = synth.from_torch_bf16(out[torch.from_numpy(rows).cuda()]).astype(np.float64)
    del out
    ref = prefill_oracle_by_head(synth.bf16_bits_to_f32(q), synth.bf16_bits_to_f32(k),
                                 synth.bf16_bits_to_f32(v), W, rows=rows)
    ex = bf16_excess(got, ref, f"prefill W={W}")
    assert ex <= 0, (ex, max_abs(got, ref))


@pytest.mark.parametrize("W", [1024, 0])
def test_prefill_8192_full_tensor_workload_heads(W):
    """The prefill workload's heads, head_dim and window at L 8192: every output."""
    L, Hq, Hkv, D = 8192, 64, 8, 128
    announce("prefill_8192_full_tensor", L=L, Hq=Hq, W=W)
    q = synth.token_major(33, synth.Q, L, Hq, D)
    k = synth.token_major(33, synth.K, L, Hkv, D)
    v = synth.token_major(33, synth.V, L, Hkv, D)
    out = hsk.swa_prefill(gpu_bf16(q), gpu_bf16(k), gpu_bf16(v), W)
    got = out_f64(out)
    ref = prefill_oracle_by_head(synth.bf16_bits_to_f32(q), synth.bf16_bits_to_f32(k),
                                 synth.bf16_bits_to_f32(v), W)
    ex = bf16_excess(got, ref, f"prefill 8192 W={W}")
    assert ex <= 0, (ex, max_abs(got, ref))


def test_int8_decode_65536_every_unit():
    """Batch 16, context 65536 (63488 INT8 + 2048 bf16), 32/8 heads: codes and
    scales of all 128 (sequence, KV head) units bit-exact, all 16 x 32 outputs."""
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
    del dk, dv
    kc, ks, vc, vs = (t.cpu().numpy() for t in (kc, ks, vc, vs))

    def unit(bg):
        b, g = bg
        okc, oks = oracle.kv_quant_int8_b32(synth.bf16_bits_to_f32(kx[b, g, :T8]))
        ovc, ovs = oracle.kv_quant_int8_b32(synth.bf16_bits_to_f32(vx[b, g, :T8]))
        exact = (np.array_equal(kc[b, g], okc) and np.array_equal(vc[b, g], ovc)
                 and np.array_equal(ks[b, g].view(np.uint32), oks.view(np.uint32))
                 and np.array_equal(vs[b, g].view(np.uint32), ovs.view(np.uint32)))
        hs = slice(g * G, (g + 1) * G)
        ref = oracle.attn_decode_int8kv(
            synth.bf16_bits_to_f32(q[b:b + 1, hs]).astype(np.float64),
            okc[None, None], oks[None, None], ovc[None, None], ovs[None, None],
            synth.bf16_bits_to_f32(kx[b:b + 1, g:g + 1, T8:]), synth.bf16_bits_to_f32(vx[b:b + 1, g:g + 1, T8:]))
        return exact, ref[0]

    units = [(b, g) for b in range(B) for g in range(Hkv)]
    res = pmap(unit, units)
    bad = [u for u, (exact, _) in zip(units, res) if not exact]
    assert not bad, ("INT8 codes or scales differ", bad)
    ref = np.empty((B, Hq, D))
    for (b, g), (_, r) in zip(units, res):
        ref[b, g * G:(g + 1) * G] = r
    ex = bf16_excess(got, ref, "int8 decode")
    assert ex <= 0, (ex, max_abs(got, ref))


def test_full_layer_decode_32768():
    """The bf16 full-attention layer of the 70-layer decode step: batch 32, context
    32768 (the INT8 decode with no INT8 region: 8 splits of 4096 per unit), 32/8
    heads, every output."""
    B, Hq, Hkv, D, ctx = 32, 32, 8, 128, 32768
    G = Hq // Hkv
    announce("full_layer_decode", B=B, ctx=ctx)
    kx = synth.head_major(14, synth.K, B, Hkv, ctx, D)
    vx = synth.head_major(14, synth.V, B, Hkv, ctx, D)
    q = synth.normal(14, synth.Q, (B, Hq, D), 1)
    out = hsk.attn_decode_int8kv(gpu_bf16(q), None, None, None, None, gpu_bf16(kx), gpu_bf16(vx))
    got = out_f64(out)
    qf = synth.bf16_bits_to_f32(q).astype(np.float64)

    def unit(bg):
        b, g = bg
        hs = slice(g * G, (g + 1) * G)
        return oracle.swa_decode(qf[b:b + 1, hs], synth.bf16_bits_to_f32(kx[b:b + 1, g:g + 1]),
                                 synth.bf16_bits_to_f32(vx[b:b + 1, g:g + 1]), [0], [ctx - 1], 0)[0]

    units = [(b, g) for b in range(B) for g in range(Hkv)]
    ref = np.empty((B, Hq, D))
    for (b, g), r in zip(units, pmap(unit, units)):
        ref[b, g * G:(g + 1) * G] = r
    ex = bf16_excess(got, ref, "full layer decode")
    assert ex <= 0, (ex, max_abs(got, ref))


def blocksparse_tiles(Hq, nb, n, seed):
    """n distinct (head, query block) pairs: the listed blocks on several heads,
    then seeded random pairs."""
    fixed_qb = [0, 1, 16, 17, 63, 64, 65, nb - 1]
    pairs = {(h, qb) for qb in fixed_qb for h in (0, Hq // 3, Hq // 2 + 1, Hq - 1)}
    rng = np.random.default_rng(seed)
    while len(pairs) < n:
        pairs.add((int(rng.integers(0, Hq)), int(rng.integers(0, nb))))
    return sorted(pairs)


def test_blocksparse_131072():
    """L 131072, 32/8 heads, 64-token blocks, top-64, window 1024: every selection
    exact (near-ties counted), 256 whole (head, query block) output tiles."""
    L, Hq, Hkv, D, block, topk, W = 131072, 32, 8, 128, 64, 64, 1024
    G = Hq // Hkv
    announce("blocksparse_full_size", L=L)
    q = synth.token_major(5, synth.Q, L, Hq, D)
    k = synth.token_major(5, synth.K, L, Hkv, D)
    v = synth.token_major(5, synth.V, L, Hkv, D)
    out, sel = hsk.blocksparse_select_attend(gpu_bf16(q), gpu_bf16(k), gpu_bf16(v), block, topk, W)
    sel_np = sel.cpu().numpy()
    got_all = out_f64(out)
    del out
    qf, kf, vf = synth.bf16_bits_to_f32(q), synth.bf16_bits_to_f32(k), synth.bf16_bits_to_f32(v)
    check_selection(sel_np, qf, kf, block, topk)          # every (head, query block)
    tiles = blocksparse_tiles(Hq, L // block, 256, 11)
    assert len(tiles) == 256

    def tile(hq):
        h, qb = hq
        g = h // G
        rows = np.arange(qb * block, (qb + 1) * block)
        return oracle.blocksparse_attend(qf[:, h:h + 1], kf[:, g:g + 1], vf[:, g:g + 1], sel_np[h:h + 1],
                                         block, W, rows=rows)[:, 0]

    ref = np.stack(pmap(tile, tiles))
    got = np.stack([got_all[qb * block:(qb + 1) * block, h] for h, qb in tiles])
    ex = bf16_excess(got, ref, "blocksparse tiles")
    assert ex <= 0, (ex, max_abs(got, ref))


def test_sparse_decode_int8_workload_every_row():
    """Batch 16, context 65536 (63488 INT8 + 2048 bf16), 32/8 heads, top-64 INT8
    blocks: means of every unit bit-exact, every (sequence, head) selection, every
    output."""
    announce("sparse_decode_workload")
    B, Hq, Hkv, D, T8, Th, topk = 16, 32, 8, 128, 63488, 2048, 64
    G = Hq // Hkv
    q = synth.normal_gpu(1300, synth.Q, (B, Hq, D))
    kx = synth.normal_gpu(1300, synth.K, (B, Hkv, T8 + Th, D), outlier_p=0.01)
    vx = synth.normal_gpu(1300, synth.V, (B, Hkv, T8 + Th, D), outlier_p=0.01)
    kc, ks = hsk.kv_quant_int8_b32(kx[:, :, :T8].contiguous())
    vc, vs = hsk.kv_quant_int8_b32(vx[:, :, :T8].contiguous())
    km = hsk.kv_block_means_int8(kc, ks)
    out, sel = hsk.attn_decode_int8kv_sparse(q, kc, ks, vc, vs, km, kx[:, :, T8:].contiguous(),
                                             vx[:, :, T8:].contiguous(), topk=topk)
    torch.cuda.synchronize()
    sel_np = sel.cpu().numpy()
    got = out.float().cpu().numpy().astype(np.float64)
    qh = q.float().cpu().numpy().astype(np.float64)
    kc, ks, vc, vs, km = (t.cpu().numpy() for t in (kc, ks, vc, vs, km))
    kh = kx[:, :, T8:].float().cpu().numpy()
    vh = vx[:, :, T8:].float().cpu().numpy()
    del kx, vx

    def unit(bg):
        b, g = bg
        hs = slice(g * G, (g + 1) * G)
        u = (slice(b, b + 1), slice(g, g + 1))
        means = oracle.int8_block_means(kc[u], ks[u])
        means_exact = np.array_equal(km[u], means.transpose(0, 1, 3, 2))
        _, scores = oracle.sparse_select(qh[b:b + 1, hs], means, topk, return_scores=True)
        ref = oracle.attn_decode_int8kv_sparse(qh[b:b + 1, hs], kc[u], ks[u], vc[u], vs[u],
                                               kh[u].astype(np.float64), vh[u].astype(np.float64),
                                               sel_np[b:b + 1, hs])
        return means_exact, scores[0], ref[0]

    units = [(b, g) for b in range(B) for g in range(Hkv)]
    res = pmap(unit, units)
    assert all(r[0] for r in res), "block means differ"
    scores = np.empty((B, Hq, T8 // 32))
    ref = np.empty((B, Hq, D))
    for (b, g), (_, sc, r) in zip(units, res):
        scores[b, g * G:(g + 1) * G] = sc
        ref[b, g * G:(g + 1) * G] = r
    check_rows(sel_np, scores, topk, [(b, h) for b in range(B) for h in range(Hq)])
    ex = bf16_excess(got, ref, "sparse decode")
    assert ex <= 0, (ex, max_abs(got, ref))
