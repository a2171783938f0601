"""The Python binding refuses every mis-shaped tensor before the C call (CPU only).

Each case hands the binding CPU tensors whose shapes agree except for one
argument.  The mismatch must raise ValueError naming that argument; with every
shape right the binding gets as far as the device check ("must be a GPU
tensor"), which shows the shape checks passed and nothing reached the library.
"""

import pytest
import torch

import hybrid_swa_kv_amd as hsk

bf, i8, f32, i32 = torch.bfloat16, torch.int8, torch.float32, torch.int32


def z(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def expect(fn, name):
    with pytest.raises(ValueError) as e:
        fn()
    msg = str(e.value)
    assert msg.startswith(name + " "), msg
    return msg


def reaches_device_check(fn):
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        fn()


def test_prefill_shapes():
    B, L, Hq, Hkv, D = 2, 64, 4, 2, 64
    q, k, v = z(B, L, Hq, D), z(B, L, Hkv, D), z(B, L, Hkv, D)
    rk, rv = z(B, Hkv, 32, D), z(B, Hkv, 32, D)
    reaches_device_check(lambda: hsk.swa_prefill(q, k, v, 16, ring_k=rk, ring_v=rv))
    reaches_device_check(lambda: hsk.swa_prefill(q[0], k[0], v[0], 16))
    expect(lambda: hsk.swa_prefill(q, z(B, L - 1, Hkv, D), v, 16), "k")
    expect(lambda: hsk.swa_prefill(q, k, z(B, L, Hkv, D // 2), 16), "v")
    expect(lambda: hsk.swa_prefill(q, z(1, L, Hkv, D), z(1, L, Hkv, D), 16), "k")
    expect(lambda: hsk.swa_prefill(q, k, v, 16, ring_k=rk, ring_v=z(B, Hkv, 16, D)), "ring_v")
    expect(lambda: hsk.swa_prefill(q, k, v, 16, ring_k=z(B, Hkv + 1, 32, D), ring_v=rv), "ring_k")
    expect(lambda: hsk.swa_prefill(q, k.float(), v, 16), "k")


def test_decode_ring_shapes():
    B, Hq, Hkv, D, W = 3, 8, 2, 128, 16
    q, kn, vn = z(B, Hq, D), z(B, Hkv, D), z(B, Hkv, D)
    rk, rv, pos = z(B, Hkv, W, D), z(B, Hkv, W, D), z(B, dtype=i32)
    reaches_device_check(lambda: hsk.swa_decode_ring(q, kn, vn, rk, rv, pos))
    expect(lambda: hsk.swa_decode_ring(q, kn, vn, rk, z(B, Hkv, W - 1, D), pos), "ring_v")
    expect(lambda: hsk.swa_decode_ring(q, kn, vn, z(B - 1, Hkv, W, D), rv, pos), "ring_k")
    expect(lambda: hsk.swa_decode_ring(q, z(B, Hkv, D // 2), vn, rk, rv, pos), "k_new")
    expect(lambda: hsk.swa_decode_ring(q, kn, z(B, Hkv + 1, D), rk, rv, pos), "v_new")
    expect(lambda: hsk.swa_decode_ring(q, kn, vn, rk, rv, z(B - 1, dtype=i32)), "pos")
    expect(lambda: hsk.swa_decode_ring(q, kn, vn, rk, rv, z(B, dtype=torch.int64)), "pos")


def test_quant_shapes():
    reaches_device_check(lambda: hsk.kv_quant_int8_b32(z(1, 2, 64, 128)))
    expect(lambda: hsk.kv_quant_int8_b32(z(1, 2, 40, 128)), "x")
    expect(lambda: hsk.kv_quant_int8_b32(z(1, 2, 64, 128, dtype=f32)), "x")


def _pool(B=2, Hq=8, Hkv=2, D=128, T8=64, Th=16):
    return dict(q=z(B, Hq, D), k_codes=z(B, Hkv, T8, D, dtype=i8), k_scales=z(B, Hkv, T8 // 32, dtype=f32),
                v_codes=z(B, Hkv, T8, D, dtype=i8), v_scales=z(B, Hkv, T8 // 32, dtype=f32),
                k_hot=z(B, Hkv, Th, D), v_hot=z(B, Hkv, Th, D))


@pytest.mark.parametrize("sparse", [False, True])
def test_int8_decode_shapes(sparse):
    B, Hkv, D, T8 = 2, 2, 128, 64
    means = z(B, Hkv, D, T8 // 32, dtype=f32)

    def call(**over):
        a = _pool()
        a.update(over)
        if sparse:
            m = over.pop("k_means", means)
            return lambda: hsk.attn_decode_int8kv_sparse(a["q"], a["k_codes"], a["k_scales"], a["v_codes"],
                                                         a["v_scales"], m, a["k_hot"], a["v_hot"], topk=1)
        a.pop("k_means", None)
        return lambda: hsk.attn_decode_int8kv(**a)

    reaches_device_check(call())
    reaches_device_check(call(k_codes=None, k_scales=None, v_codes=None, v_scales=None))
    expect(call(v_hot=z(B, Hkv, 15, D)), "v_hot")
    expect(call(v_codes=z(B, Hkv, T8 - 32, D, dtype=i8)), "v_codes")
    expect(call(k_codes=z(B, Hkv, T8, D // 2, dtype=i8)), "k_codes")
    expect(call(k_scales=z(B, Hkv, T8 // 32 + 1, dtype=f32)), "k_scales")
    expect(call(v_scales=z(B, Hkv, T8 // 32, dtype=torch.float64)), "v_scales")
    expect(call(k_codes=z(B, Hkv, 48, D, dtype=i8)), "k_codes")
    expect(call(k_hot=z(B, Hkv + 2, 16, D), v_hot=z(B, Hkv + 2, 16, D)), "k_codes")
    if sparse:
        expect(call(k_means=z(B, Hkv, T8 // 32, D, dtype=f32)), "k_means")


def test_blocksparse_shapes():
    L, Hq, Hkv, D = 256, 4, 2, 128
    q, k, v = z(L, Hq, D), z(L, Hkv, D), z(L, Hkv, D)
    reaches_device_check(lambda: hsk.blocksparse_select_attend(q, k, v, 64, 2, 64))
    expect(lambda: hsk.blocksparse_select_attend(q, z(L - 64, Hkv, D), v, 64, 2, 64), "k")
    expect(lambda: hsk.blocksparse_select_attend(q, k, z(L, Hkv, 64), 64, 2, 64), "v")
    with pytest.raises(ValueError, match="multiple of block"):
        hsk.blocksparse_select_attend(z(L - 1, Hq, D), z(L - 1, Hkv, D), z(L - 1, Hkv, D), 64, 2, 64)


def test_chunk_and_means_and_prefix_shapes():
    B, C, Hq, Hkv, D, W = 1, 128, 4, 2, 128, 64
    q, k, v = z(B, C, Hq, D), z(B, C, Hkv, D), z(B, C, Hkv, D)
    rk, rv = z(B, Hkv, W, D), z(B, Hkv, W, D)
    reaches_device_check(lambda: hsk.swa_prefill_chunk(q, k, v, rk, rv, 0))
    expect(lambda: hsk.swa_prefill_chunk(q, z(B, C, Hkv, 64), v, rk, rv, 0), "k")
    expect(lambda: hsk.swa_prefill_chunk(q, k, v, rk, z(B, Hkv, W + 64, D), 0), "ring_v")
    codes, scales = z(2, 2, 64, 128, dtype=i8), z(2, 2, 2, dtype=f32)
    reaches_device_check(lambda: hsk.kv_block_means_int8(codes, scales))
    expect(lambda: hsk.kv_block_means_int8(codes, z(2, 2, 3, dtype=f32)), "scales")
    reaches_device_check(lambda: hsk.swa_window_safe_len(z(3, 8, dtype=i32), z(3, dtype=i32)))
    expect(lambda: hsk.swa_window_safe_len(z(3, 8, dtype=i32), z(2, dtype=i32)), "match_len")


def test_tensors_and_stream_must_share_one_gpu():
    """Pointers from two GPUs in one call would be read by kernels on one of them:
    the binding refuses mixed devices, and a stream of another device."""
    from types import SimpleNamespace

    from hybrid_swa_kv_amd import api

    def on(dev):
        return SimpleNamespace(is_cuda=True, device=torch.device(dev))

    assert api._device(None, "a", on("cuda:0"), "b", on("cuda:0"), "c") == torch.device("cuda:0")
    with pytest.raises(ValueError, match="c is on cuda:1"):
        api._device(on("cuda:0"), "a", None, "b", on("cuda:1"), "c")
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        api._device(on("cuda:0"), "a", SimpleNamespace(is_cuda=False, device=torch.device("cpu")), "b")
    with pytest.raises(ValueError, match="out is on cuda:1"):
        api._same_device(torch.device("cuda:0"), on("cuda:1"), "out")
    with pytest.raises(ValueError, match="stream is on cuda:1"):
        api._stream(SimpleNamespace(device=torch.device("cuda:1"), cuda_stream=0), torch.device("cuda:0"))
