"""C ABI checks that need no GPU: the library loads, exports every declared symbol,
and rejects bad arguments on the host with the documented status codes.

Every call below fails validation before anything is enqueued (the pointers are
fake and never dereferenced).
"""

import os
import re

import pytest

from hybrid_swa_kv_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "hybrid_swa_kv.h")
OK, NULL, SHAPE, UNSUP, ALIGN, WS = 0, 1, 2, 3, 4, 5
P = 4096          # a fake, 16-byte aligned "device pointer"
MIS = 4100        # misaligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from hybrid_swa_kv_amd import build

        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert getattr(lib, n) is not None
    assert lib.hsk_abi_version() >= 1
    for code in range(7):
        assert lib.hsk_strerror(code)


def test_prefill_validation(lib):
    f = lib.swa_prefill
    #        q  k  v  out B  L  Hq Hkv D  win scale dtype rk rv rw stream
    assert f(None, P, P, P, 1, 8, 2, 2, 128, 0, 1.0, 1, None, None, 0, None) == NULL
    assert f(P, P, P, P, 1, 8, 2, 2, 128, 0, 1.0, 1, P, None, 4, None) == NULL
    assert f(P, P, P, P, 0, 8, 2, 2, 128, 0, 1.0, 1, None, None, 0, None) == SHAPE
    assert f(P, P, P, P, 1, 0, 2, 2, 128, 0, 1.0, 1, None, None, 0, None) == SHAPE
    assert f(P, P, P, P, 1, 8, 3, 2, 128, 0, 1.0, 1, None, None, 0, None) == SHAPE
    assert f(P, P, P, P, 1, 8, 2, 2, 96, 0, 1.0, 1, None, None, 0, None) == UNSUP
    assert f(P, P, P, P, 1, 8, 2, 2, 128, 0, 1.0, 7, None, None, 0, None) == UNSUP
    assert f(P, P, P, P, 1, 8, 2, 2, 128, 0, float("nan"), 1, None, None, 0, None) == SHAPE
    assert f(P, P, P, P, 1, 8, 2, 2, 128, 0, -1.0, 1, None, None, 0, None) == SHAPE
    assert f(P, P, P, P, 1, 8, 2, 2, 128, 0, 1.0, 1, P, P, 0, None) == SHAPE
    assert f(P, MIS, P, P, 1, 8, 2, 2, 128, 0, 1.0, 1, None, None, 0, None) == ALIGN
    assert f(P, P, P, P, 1, 1 << 20, 128, 8, 64, 0, 1.0, 0, None, None, 0, None) == UNSUP  # fp32: > 2^26 rows x heads


def test_decode_ring_validation(lib):
    f = lib.swa_decode_ring
    #        q  kn vn rk rv pos out slot B Hq Hkv D W scale stream
    assert f(P, P, P, P, P, None, P, None, 2, 8, 2, 128, 128, 1.0, None) == NULL
    assert f(P, P, P, P, P, P, P, None, 2, 8, 2, 128, 0, 1.0, None) == SHAPE
    assert f(P, P, P, P, P, P, P, None, 2, 8, 2, 128, 70000, 1.0, None) == SHAPE
    assert f(P, P, P, P, P, P, P, None, 2, 8, 3, 128, 128, 1.0, None) == SHAPE
    assert f(P, P, P, P, P, P, P, None, 2, 8, 2, 32, 128, 1.0, None) == UNSUP
    assert f(P, P, P, P, P, P, P, None, 2, 40, 2, 128, 128, 1.0, None) == UNSUP
    assert f(P, P, P, P, P, P, P, None, 65536, 8, 2, 128, 128, 1.0, None) == UNSUP
    assert f(P, P, P, MIS, P, P, P, None, 2, 8, 2, 128, 128, 1.0, None) == ALIGN
    assert f(P, P, P, P, P, P + 2, P, None, 2, 8, 2, 128, 128, 1.0, None) == ALIGN


def test_quant_validation(lib):
    f = lib.kv_quant_int8_b32
    assert f(P, None, P, 1, 1, 32, 128, None) == NULL
    assert f(P, P, P, 1, 1, 33, 128, None) == SHAPE
    assert f(P, P, P, 0, 1, 32, 128, None) == SHAPE
    assert f(P, P, P, 1, 1, 32, 256, None) == UNSUP
    assert f(P, MIS, P, 1, 1, 32, 128, None) == ALIGN
    assert f(P, P, P, 1, 1, 0, 128, None) == OK          # empty region: nothing to do
    assert f(P, P, P, 1 << 16, 1 << 10, 1 << 20, 128, None) == UNSUP  # 2^41 blocks


def test_block_means_validation(lib):
    f = lib.kv_block_means_int8
    #        codes scales means B Hkv T8 D stream
    assert f(P, P, P, 0, 1, 32, 128, None) == SHAPE
    assert f(P, P, P, 1, 1, 33, 128, None) == SHAPE
    assert f(P, P, P, 1, 1, 32, 96, None) == UNSUP
    assert f(P, P, P, 1 << 16, 1 << 10, 1 << 20, 128, None) == UNSUP
    assert f(None, None, None, 1, 1, 0, 128, None) == OK     # empty region: nothing to do
    assert f(None, P, P, 1, 1, 32, 128, None) == NULL
    assert f(P, P, P + 2, 1, 1, 32, 128, None) == ALIGN


def test_int8_decode_validation(lib):
    f = lib.attn_decode_int8kv
    need = lib.attn_decode_int8kv_workspace_size(16, 32, 8, 128, 63488, 2048)
    assert need > 0
    assert lib.attn_decode_int8kv_workspace_size(16, 32, 8, 128, 63488, 0) == 0
    assert lib.attn_decode_int8kv_workspace_size(1, 4, 1, 128, 0, 1 << 30) == 0  # weights past 2^31
    #        q kc ks vc vs kh vh out B Hq Hkv D T8 Th scale ws wsb stream
    assert f(P, None, P, P, P, P, P, P, 16, 32, 8, 128, 64, 8, 1.0, P, need, None) == NULL
    assert f(P, P, P, P, P, P, P, P, 16, 32, 8, 128, 48, 8, 1.0, P, need, None) == SHAPE
    assert f(P, P, P, P, P, P, P, P, 16, 32, 8, 128, 64, 0, 1.0, P, need, None) == SHAPE
    assert f(P, P, P, P, P, P, P, P, 1, 34, 2, 128, 64, 8, 1.0, P, need, None) == UNSUP
    assert f(P, P, P, P, P, P, P, P, 1, 4, 1, 128, 0, 1 << 30, 1.0, P, need, None) == UNSUP
    assert f(P, P, P, P, P, P, P, P, 16, 32, 8, 128, 63488, 2048, 1.0, P, need - 1, None) == WS
    assert f(P, P, P, P, P, P, P, P, 16, 32, 8, 128, 63488, 2048, 1.0, None, need, None) == WS
    assert f(P, P, P, P, P, MIS, P, P, 16, 32, 8, 128, 63488, 2048, 1.0, P, need, None) == ALIGN


def test_int8_decode_noalloc_validation(lib):
    """Errors of the static-array variant come back before any HIP call (no GPU
    needed): argument errors as the workspace entry point's, sizes beyond its
    32 MiB array as a workspace error."""
    f = lib.attn_decode_int8kv_noalloc
    #        q kc ks vc vs kh vh out B Hq Hkv D T8 Th scale stream
    assert f(P, None, P, P, P, P, P, P, 16, 32, 8, 128, 64, 8, 1.0, None) == NULL
    assert f(P, P, P, P, P, P, P, P, 16, 32, 8, 128, 48, 8, 1.0, None) == SHAPE
    assert f(P, P, P, P, P, P, P, P, 16, 32, 8, 128, 64, 0, 1.0, None) == SHAPE
    assert f(P, P, P, P, P, P, P, P, 1, 34, 2, 128, 64, 8, 1.0, None) == UNSUP
    assert lib.attn_decode_int8kv_workspace_size(512, 128, 8, 128, 0, 64) > 32 << 20
    assert f(P, None, None, None, None, P, P, P, 512, 128, 8, 128, 0, 64, 1.0, None) == WS


def test_blocksparse_validation(lib):
    f = lib.blocksparse_select_attend
    need = lib.blocksparse_workspace_size(131072, 32, 8, 128, 64, 64)
    # fp64 block sums of Q and K ([H][D][nb], nb = 2048 already a multiple of 64)
    # plus the per-head lower triangle of block scores
    assert need == ((32 + 8) * 2048 * 128 + 32 * (2048 * 2047 // 2)) * 8
    # block counts are padded to a multiple of 64 in the sums
    assert lib.blocksparse_workspace_size(64 * 100, 4, 1, 64, 64, 4) == ((4 + 1) * 128 * 64 + 4 * (100 * 99 // 2)) * 8
    #        q k v out sel L Hq Hkv D block topk win scale ws wsb stream
    assert f(P, P, P, P, None, 1024, 4, 1, 128, 64, 4, 128, 1.0, P, need, None) == NULL
    assert f(P, P, P, P, P, 1000, 4, 1, 128, 64, 4, 128, 1.0, P, need, None) == SHAPE
    assert f(P, P, P, P, P, 1024, 4, 1, 128, 32, 4, 128, 1.0, P, need, None) == UNSUP
    assert f(P, P, P, P, P, 1024, 4, 1, 128, 64, 300, 128, 1.0, P, need, None) == UNSUP
    assert f(P, P, P, P, P, 1024, 4, 1, 128, 64, 4, 0, 1.0, P, need, None) == SHAPE
    assert f(P, P, P, P, P, 64 * 5000, 4, 1, 128, 64, 4, 128, 1.0, P, 1 << 40, None) == UNSUP
    assert f(P, P, P, P, P, 1024, 4, 1, 128, 64, 4, 128, 1.0, P, 10, None) == WS
    assert f(P, P, P, MIS, P, 1024, 4, 1, 128, 64, 4, 128, 1.0, P, need, None) == ALIGN


def test_window_safe_validation(lib):
    f = lib.swa_window_safe_len
    MIS2 = 4098      # 2-byte aligned only
    #        slot_pos match out B  W  stream
    assert f(None, P, P, 4, 8, None) == NULL
    assert f(P, P, None, 4, 8, None) == NULL
    assert f(None, None, None, 0, 8, None) == 0  # empty batch
    assert f(None, None, None, -1, 8, None) == SHAPE
    assert f(P, P, P, -1, 8, None) == SHAPE
    assert f(P, P, P, 4, 0, None) == SHAPE
    assert f(P, P, P, 4, 65537, None) == SHAPE
    assert f(MIS2, P, P, 4, 8, None) == ALIGN
    assert f(P, P, P, 0, 8, None) == 0          # empty batch: nothing enqueued


def test_prefill_chunk_validation(lib):
    f = lib.swa_prefill_chunk
    #        q k v out rk rv B C  Hq Hkv D  W   pos0 scale stream
    assert f(P, P, P, P, None, P, 1, 64, 8, 2, 128, 128, 0, 1.0, None) == NULL
    assert f(P, P, P, P, P, P, 0, 64, 8, 2, 128, 128, 0, 1.0, None) == SHAPE
    assert f(P, P, P, P, P, P, 1, 64, 8, 2, 128, 128, -64, 1.0, None) == SHAPE
    assert f(P, P, P, P, P, P, 1, 64, 8, 2, 128, 100, 0, 1.0, None) == UNSUP     # W % 64
    assert f(P, P, P, P, P, P, 1, 64, 8, 2, 128, 128, 32, 1.0, None) == UNSUP    # pos0 % 64
    assert f(P, P, P, P, P, P, 1, 64, 8, 2, 96, 128, 0, 1.0, None) == UNSUP      # head_dim
    assert f(P, P, P, P, P, P, 1, 64, 8, 2, 128, 128, 0, 0.0, None) == SHAPE
    assert f(P, P, P, MIS, P, P, 1, 64, 8, 2, 128, 128, 0, 1.0, None) == ALIGN


def test_sparse_decode_validation(lib):
    f = lib.attn_decode_int8kv_sparse
    need = lib.attn_decode_int8kv_sparse_workspace_size(16, 32, 8, 128, 63488, 2048, 64)
    assert need > 0
    assert lib.attn_decode_int8kv_sparse_workspace_size(16, 32, 8, 128, 63488, 2048, -1) == 0
    #        q  kc ks vc vs km kh vh out sel B  Hq Hkv D  T8  Th topk scale ws wsb stream
    assert f(P, P, P, P, P, P, P, P, P, None, 2, 8, 2, 128, 64, 16, 4, 1.0, P, need, None) == NULL
    assert f(P, P, P, P, P, None, P, P, P, P, 2, 8, 2, 128, 64, 16, 4, 1.0, P, need, None) == NULL
    assert f(P, P, P, P, P, P, P, P, P, P, 2, 8, 2, 128, 48, 16, 4, 1.0, P, need, None) == SHAPE
    assert f(P, P, P, P, P, P, P, P, P, P, 2, 8, 2, 128, 64, 16, 300, 1.0, P, need, None) == UNSUP
    assert f(P, P, P, P, P, P, P, P, P, P, 2, 64, 2, 128, 64, 16, 4, 1.0, P, need, None) == UNSUP
    assert f(P, P, P, P, P, P, P, P, P, P, 2, 8, 2, 128, 64, 16, 4, 1.0, P, 0, None) == WS
    g = lib.kv_block_means_int8
    assert g(P, P, P, 2, 2, 48, 128, None) == SHAPE
    assert g(None, None, None, 2, 2, 0, 128, None) == 0
    assert g(None, P, P, 2, 2, 64, 128, None) == NULL
    assert g(P, P, P, 2, 2, 64, 96, None) == UNSUP
