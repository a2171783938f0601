"""attn_decode_int8kv_noalloc against attn_decode_int8kv, through the C ABI.

Two calls in a row on the library's static device array, the second with a
smaller input, each compared bit for bit with the workspace entry point on the
same inputs (same kernels and split plan, so the outputs must be identical), and
with the oracle at the bf16 bar.
"""

import numpy as np
import pytest
import torch

import hybrid_swa_kv_amd as hsk
import oracle
from hybrid_swa_kv_amd import synth
from tests.helpers import announce, bf16_excess, f64, gpu_bf16, max_abs, out_f64

pytestmark = pytest.mark.gpu


def _case(seed, B, Hq, Hkv, D, T8, Th):
    kx = synth.head_major(seed, synth.K, B, Hkv, T8 + Th, D, outlier_p=0.01)
    vx = synth.head_major(seed, synth.V, B, Hkv, T8 + Th, D, outlier_p=0.01)
    q = synth.normal(seed, synth.Q, (B, Hq, D), 1)
    kc, ks = hsk.kv_quant_int8_b32(gpu_bf16(np.ascontiguousarray(kx[:, :, :T8])))
    vc, vs = hsk.kv_quant_int8_b32(gpu_bf16(np.ascontiguousarray(vx[:, :, :T8])))
    kh = gpu_bf16(np.ascontiguousarray(kx[:, :, T8:]))
    vh = gpu_bf16(np.ascontiguousarray(vx[:, :, T8:]))
    okc, oks = oracle.kv_quant_int8_b32(synth.bf16_bits_to_f32(kx[:, :, :T8]))
    ovc, ovs = oracle.kv_quant_int8_b32(synth.bf16_bits_to_f32(vx[:, :, :T8]))
    ref = oracle.attn_decode_int8kv(f64(q), okc, oks, ovc, ovs, f64(kx[:, :, T8:]), f64(vx[:, :, T8:]))
    return gpu_bf16(q), kc, ks, vc, vs, kh, vh, ref


def test_noalloc_matches_workspace_entry_point_twice():
    # the second call is smaller (fewer units, splits and heads) and reuses the
    # same static array right after the first
    for seed, shape in ((501, (4, 32, 8, 128, 8192, 512)), (502, (2, 8, 2, 64, 1024, 33))):
        B, Hq, Hkv, D, T8, Th = shape
        announce("noalloc", seed=seed, B=B, Hq=Hq, Hkv=Hkv, D=D, T8=T8, Th=Th)
        q, kc, ks, vc, vs, kh, vh, ref = _case(seed, *shape)
        got = hsk.attn_decode_int8kv_noalloc(q, kc, ks, vc, vs, kh, vh)
        want = hsk.attn_decode_int8kv(q, kc, ks, vc, vs, kh, vh)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), seed
        ex = bf16_excess(out_f64(got), ref, "noalloc")
        assert ex <= 0, (seed, ex, max_abs(out_f64(got), ref))


def test_noalloc_workload_size_and_no_int8_region():
    """The INT8 decode workload's shape (batch 16, 63488 + 2048 tokens, 32/8 heads)
    and an all-bf16 context, each bit-identical to the workspace entry point."""
    B, Hq, Hkv, D, T8, Th = 16, 32, 8, 128, 63488, 2048
    announce("noalloc_workload", B=B, T8=T8, Th=Th)
    q = synth.normal_gpu(77, synth.Q, (B, Hq, D))
    kx = synth.normal_gpu(77, synth.K, (B, Hkv, T8 + Th, D), outlier_p=0.01)
    vx = synth.normal_gpu(77, synth.V, (B, Hkv, T8 + Th, D), outlier_p=0.01)
    kc, ks = hsk.kv_quant_int8_b32(kx[:, :, :T8].contiguous())
    vc, vs = hsk.kv_quant_int8_b32(vx[:, :, :T8].contiguous())
    kh, vh = kx[:, :, T8:].contiguous(), vx[:, :, T8:].contiguous()
    got = hsk.attn_decode_int8kv_noalloc(q, kc, ks, vc, vs, kh, vh)
    want = hsk.attn_decode_int8kv(q, kc, ks, vc, vs, kh, vh)
    got2 = hsk.attn_decode_int8kv_noalloc(q, None, None, None, None, kh, vh)
    want2 = hsk.attn_decode_int8kv(q, None, None, None, None, kh, vh)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    assert torch.equal(got2.view(torch.int16), want2.view(torch.int16))


def test_noalloc_rejects_sizes_beyond_its_array():
    # 4096 units x 16 heads x 130 floats: beyond the 32 MiB array; refused on the host
    B, Hq, Hkv, D, T8, Th = 512, 128, 8, 128, 0, 64
    need = hsk.attn_decode_int8kv_workspace_size(B, Hq, Hkv, D, T8, Th)
    assert need > 32 << 20
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    kh = torch.zeros((B, Hkv, Th, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="workspace"):
        hsk.attn_decode_int8kv_noalloc(q, None, None, None, None, kh, kh)
