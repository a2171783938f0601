"""Seeded synthetic inputs shared by the tests, the bench and the CPU oracle.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the attention, ring, quantisation or selection arithmetic.

Every tensor is generated slice by slice from
``numpy.random.Generator(PCG64(SeedSequence((workload, tensor_id, slice_id))))``
as float32 N(0, 1) and rounded to bfloat16 with round-to-nearest-even, so the
same bytes come out on any host, in any order, and no slice needs the others.
Slices are drawn on a thread pool.

Outliers (the INT8 decode workload): each element independently, with
probability p, is multiplied by a factor before the bf16 rounding (a power of
two keeps the rounding exact).  Outlier positions come from their own stream,
as gaps between hits drawn from the geometric distribution, which is the same
law as independent Bernoulli(p) draws per element.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# tensor ids inside a workload's seed tuple
Q, K, V, OUTLIER, K_NEW, V_NEW, POS, MISC = 0, 1, 2, 3, 4, 5, 6, 7

_THREADS = max(1, min(16, os.cpu_count() or 1))


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(tuple(int(x) for x in key))))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 -> bfloat16 (nearest, ties to even); returns uint16 bit patterns.

    Inputs here are finite; NaN handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    lsb = (u >> 16) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= np.uint32(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _slice_normal(workload: int, tensor_id: int, slice_id: int, n: int,
                  outlier_p: float, outlier_mult: float) -> np.ndarray:
    x = _rng(workload, tensor_id, slice_id).standard_normal(n, dtype=np.float32)
    if outlier_p > 0.0:
        g = _rng(workload, OUTLIER, tensor_id, slice_id)
        idx = []
        cur = -1
        while True:
            gaps = g.geometric(outlier_p, size=max(64, int(n * outlier_p * 1.2) + 64))
            pos = cur + np.cumsum(gaps)
            keep = pos[pos < n]
            idx.append(keep)
            if len(keep) < len(pos):
                break
            cur = int(pos[-1])
        idx = np.concatenate(idx)
        x[idx] *= np.float32(outlier_mult)
    return x


def normal(workload: int, tensor_id: int, shape, slice_axes: int, dtype: str = "bf16",
           outlier_p: float = 0.0, outlier_mult: float = 8.0) -> np.ndarray:
    """N(0,1) tensor of ``shape``; the first ``slice_axes`` axes index the slices.

    Slice ids are the row-major flattening of the leading ``slice_axes`` indices.
    dtype "bf16" returns uint16 bit patterns, "f32" float32 values.
    """
    shape = tuple(int(s) for s in shape)
    lead = shape[:slice_axes]
    n_slices = int(np.prod(lead)) if lead else 1
    per = int(np.prod(shape[slice_axes:]))
    out = np.empty((n_slices, per), dtype=np.uint16 if dtype == "bf16" else np.float32)

    def work(s: int) -> None:
        x = _slice_normal(workload, tensor_id, s, per, outlier_p, outlier_mult)
        out[s] = f32_to_bf16_bits(x) if dtype == "bf16" else x

    if n_slices == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(work, range(n_slices)))
    return out.reshape(shape)


def token_major(workload: int, tensor_id: int, L: int, H: int, D: int,
                dtype: str = "bf16", B: int | None = None) -> np.ndarray:
    """Prefill tensor [L, H, D] (or [B, L, H, D]); one slice per (batch, head)."""
    if B is None:
        x = normal(workload, tensor_id, (H, L, D), 1, dtype)
        return np.ascontiguousarray(x.transpose(1, 0, 2))
    x = normal(workload, tensor_id, (B, H, L, D), 2, dtype)
    return np.ascontiguousarray(x.transpose(0, 2, 1, 3))


def head_major(workload: int, tensor_id: int, B: int, H: int, T: int, D: int,
               dtype: str = "bf16", outlier_p: float = 0.0, outlier_mult: float = 8.0) -> np.ndarray:
    """Cache tensor [B, H, T, D]; one slice per (batch, head)."""
    return normal(workload, tensor_id, (B, H, T, D), 2, dtype, outlier_p, outlier_mult)


def integers(workload: int, tensor_id: int, shape, low: int, high: int) -> np.ndarray:
    """Uniform int64 in [low, high) (e.g. decode positions)."""
    return _rng(workload, tensor_id, 0).integers(low, high, size=shape, dtype=np.int64)


def to_torch(x: np.ndarray, device="cpu"):
    """uint16 bf16 bit patterns -> torch.bfloat16; other dtypes map directly."""
    import torch

    if x.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device)


def from_torch_bf16(t) -> np.ndarray:
    """torch.bfloat16 tensor -> float32 numpy values (exact)."""
    import torch

    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return bf16_bits_to_f32(bits)


def normal_gpu(workload: int, tensor_id: int, shape, outlier_p: float = 0.0, outlier_mult: float = 8.0,
               device="cuda"):
    """Seeded N(0,1) bf16 tensor drawn on the GPU (torch's Philox generator).

    Same distribution as ``normal`` (float32 draw, optional outliers, one
    round-to-nearest-even to bf16) but not the same values; used where only the
    distribution matters (throughput runs), since drawing gigabytes on the host
    is slow.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(workload) * 1_000_003 + int(tensor_id) * 7919 + 12345)
    x = torch.randn(tuple(int(s) for s in shape), generator=g, device=device, dtype=torch.float32)
    if outlier_p > 0.0:
        hit = torch.rand(x.shape, generator=g, device=device) < outlier_p
        x = torch.where(hit, x * outlier_mult, x)
        del hit
    return x.to(torch.bfloat16)
