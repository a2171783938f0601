"""GPU parity: kv_quant_int8_b32 (bit-exact codes and scales) and attn_decode_int8kv."""

import numpy as np
import pytest
import torch

import hybrid_swa_kv_amd as hsk
import oracle
from hybrid_swa_kv_amd import synth
from tests.helpers import bf16_excess, announce, f64, gpu_bf16, max_abs, out_f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,Hkv,T,D", [(1, 1, 32, 128), (2, 3, 96, 64), (3, 2, 1024, 128)])
def test_quant_bit_exact(B, Hkv, T, D):
    announce("quant", B=B, Hkv=Hkv, T=T, D=D)
    x = synth.head_major(60 + T, synth.K, B, Hkv, T, D, outlier_p=0.01)
    x = x.copy()
    x[0, 0, :32] = 0                                        # an all-zero block
    if T >= 64:
        x[-1, -1, 32:64] = synth.f32_to_bf16_bits(np.full((32, D), 2.0 ** -30, np.float32))
        x[-1, -1, 40, 3] = synth.f32_to_bf16_bits(np.array([-2.0 ** -29], np.float32))[0]
    codes, scales = hsk.kv_quant_int8_b32(gpu_bf16(x))
    ref_c, ref_s = oracle.kv_quant_int8_b32(synth.bf16_bits_to_f32(x))
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), ref_c)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))


def _decode_case(seed, B, Hq, Hkv, D, T8, Th, outlier_p=0.01):
    T = T8 + Th
    kx = synth.head_major(seed, synth.K, B, Hkv, T, D, outlier_p=outlier_p)
    vx = synth.head_major(seed, synth.V, B, Hkv, T, D, outlier_p=outlier_p)
    q = synth.normal(seed, synth.Q, (B, Hq, D), 1)
    kc, ks = oracle.kv_quant_int8_b32(synth.bf16_bits_to_f32(kx[:, :, :T8]))
    vc, vs = oracle.kv_quant_int8_b32(synth.bf16_bits_to_f32(vx[:, :, :T8]))
    kh = np.ascontiguousarray(kx[:, :, T8:])
    vh = np.ascontiguousarray(vx[:, :, T8:])
    ref = oracle.attn_decode_int8kv(f64(q), kc, ks, vc, vs, f64(kh), f64(vh))
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    out = hsk.attn_decode_int8kv(gpu_bf16(q), t(kc) if T8 else None, t(ks) if T8 else None,
                                 t(vc) if T8 else None, t(vs) if T8 else None, gpu_bf16(kh), gpu_bf16(vh))
    return out_f64(out), ref


@pytest.mark.parametrize("B,Hq,Hkv,D,T8,Th", [
    (2, 8, 2, 128, 0, 1), (2, 8, 2, 128, 32, 17), (1, 4, 4, 64, 96, 64), (3, 16, 1, 128, 2048, 100),
    (2, 4, 1, 128, 4096, 2048), (1, 2, 2, 64, 128, 33), (2, 12, 4, 128, 1024, 1)])
def test_int8_decode_parity(B, Hq, Hkv, D, T8, Th):
    announce("int8_decode", B=B, Hq=Hq, Hkv=Hkv, D=D, T8=T8, Th=Th)
    got, ref = _decode_case(70 + T8 + Th, B, Hq, Hkv, D, T8, Th)
    ex = bf16_excess(got, ref)
    assert ex <= 0, (ex, max_abs(got, ref))


def test_int8_pipeline_on_gpu_codes():
    # GPU quantiser feeding the GPU decode equals the oracle's quantise + decode
    B, Hq, Hkv, D, T8, Th = 2, 8, 2, 128, 2048, 256
    announce("int8_pipeline")
    seed = 80
    T = T8 + Th
    kx = synth.head_major(seed, synth.K, B, Hkv, T, D, outlier_p=0.01)
    vx = synth.head_major(seed, synth.V, B, Hkv, T, D, outlier_p=0.01)
    q = synth.normal(seed, synth.Q, (B, Hq, D), 1)
    dk, dv = gpu_bf16(kx), gpu_bf16(vx)
    kc, ks = hsk.kv_quant_int8_b32(dk[:, :, :T8].contiguous())
    vc, vs = hsk.kv_quant_int8_b32(dv[:, :, :T8].contiguous())
    out = hsk.attn_decode_int8kv(gpu_bf16(q), kc, ks, vc, vs, dk[:, :, T8:].contiguous(), dv[:, :, T8:].contiguous())
    okc, oks = oracle.kv_quant_int8_b32(synth.bf16_bits_to_f32(kx[:, :, :T8]))
    ovc, ovs = oracle.kv_quant_int8_b32(synth.bf16_bits_to_f32(vx[:, :, :T8]))
    ref = oracle.attn_decode_int8kv(f64(q), okc, oks, ovc, ovs, f64(kx[:, :, T8:]), f64(vx[:, :, T8:]))
    assert bf16_excess(out_f64(out), ref) <= 0
    a = hsk.attn_decode_int8kv(gpu_bf16(q), kc, ks, vc, vs, dk[:, :, T8:].contiguous(), dv[:, :, T8:].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), out.view(torch.int16))   # deterministic split merge
