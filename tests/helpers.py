"""Shared helpers for the GPU parity tests (inputs from synth, outputs to numpy)."""

from __future__ import annotations

import numpy as np
import torch

from hybrid_swa_kv_amd import synth

BF16_TOL = 2e-2   # max-abs tolerance for bf16 outputs (see bf16_excess)
BF16_REL = 2.0 ** -7  # above |ref| = 2.56 the bf16 format itself cannot hold 2e-2
F32_TOL = 1e-5    # max-abs tolerance for fp32 outputs


def dev():
    return torch.device("cuda:0")


def gpu_bf16(bits: np.ndarray):
    return synth.to_torch(bits, dev())


def f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 values (exact)."""
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def out_f64(t) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return synth.from_torch_bf16(t).astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)))) if np.size(a) else 0.0


def bf16_excess(got, ref) -> float:
    """Largest |got - ref| - max(2e-2, 2^-7 |ref|) over all elements (<= 0 passes).

    A bf16 output is itself rounded by up to half an ulp, 2^-9 |x|, which exceeds
    2e-2 once |x| >= 8; the absolute bar therefore turns into a relative bar of
    2^-7 (one to two bf16 ulps) where 2^-7 |ref| > 2e-2, i.e. for |ref| > 2.56.
    """
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if got.size == 0:
        return -1.0
    allowed = np.maximum(BF16_TOL, BF16_REL * np.abs(ref))
    return float(np.max(np.abs(got - ref) - allowed))


def announce(name: str, **kw) -> None:
    print(f"[case] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)
