"""INT8 block-wise KV encoder, step by step in IEEE fp32.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

[K25-arch] section 2.2 "direction one": the warm KV region is stored as INT8
with block-wise quantisation; section 2.3: one scale is calibrated per group of
32 tokens.  The pages give neither the scale rule nor the rounding; the reading
taken here (symmetric absmax scaling) is:

  for each (sequence, KV head, 32-token block) and separately for K and V:
    X = the block's 32 x D values as fp32 (exact from bf16)
    a = max |X|
    a == 0  ->  scale 0, every code 0
    else    ->  s = fl32(a / 127)                  (correctly rounded division)
                c = clamp(rint(fl32(X / s)), -127, 127)   rint = half to even
  dequantised value = c * s

Blocks are aligned to token 0 and span all of head_dim (section 3.3 of the same
page evicts whole quantisation blocks, so the region is a whole number of
blocks).  -128 is never produced.
"""

from __future__ import annotations

import numpy as np


def kv_quant_int8_b32(x, block: int = 32):
    """Encode x [..., T, D] (values exactly representable in fp32) block-wise.

    Returns (codes int8 [..., T, D], scales float32 [..., T/block]).
    """
    xf = np.asarray(x, dtype=np.float32)
    *lead, T, D = xf.shape
    if T % block != 0:
        raise ValueError("token count must be a multiple of the block size")
    xb = xf.reshape(*lead, T // block, block, D)
    a = np.abs(xb).max(axis=(-2, -1))                       # exact in fp32
    nonzero = a != np.float32(0)
    s = np.where(nonzero, a / np.float32(127), np.float32(0)).astype(np.float32)
    s_div = np.where(nonzero, s, np.float32(1)).astype(np.float32)[..., None, None]
    quot = (xb / s_div).astype(np.float32)                  # fl32(x / s)
    c = np.clip(np.rint(quot), -127, 127)
    c = np.where(nonzero[..., None, None], c, 0).astype(np.int8)
    return c.reshape(*lead, T, D), s


def dequant_int8_b32(codes, scales, block: int = 32) -> np.ndarray:
    """code * scale per element, in fp64 (exact: an 8-bit integer times an fp32)."""
    c = np.asarray(codes, dtype=np.float64)
    s = np.asarray(scales, dtype=np.float64)
    *lead, T, D = c.shape
    return (c.reshape(*lead, T // block, block, D) * s[..., None, None]).reshape(*lead, T, D)
