"""Shared helpers for the GPU parity tests (inputs from synth, outputs to numpy)."""

from __future__ import annotations

import numpy as np
import torch

from hybrid_swa_kv_amd import synth

BF16_TOL = 2e-2   # max-abs tolerance of the arithmetic for bf16 outputs (see bf16_excess)
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


def half_ulp_bf16(x) -> np.ndarray:
    """Half a bf16 unit in the last place of |x| (the largest rounding error of a
    bf16 result near x): 2^(e - 9) for |x| = m 2^e, m in [0.5, 1); 2^-134 (half
    the smallest subnormal step) below the normal range."""
    a = np.abs(np.asarray(x, np.float64))
    _, e = np.frexp(a)
    return np.where(a >= 2.0 ** -126, np.ldexp(1.0, e - 9), 2.0 ** -134)


def bf16_excess(got, ref, label: str = "") -> float:
    """Largest |got - ref| - (2e-2 + half_ulp_bf16(ref)) over all elements (<= 0 passes).

    2e-2 bounds the error of the arithmetic; a bf16 output also carries its own
    final rounding, up to half an ulp of the value, which is between 2^-9 |x| and
    2^-8 |x| and exceeds 2e-2 from |x| >= 8 on (the x8 outliers of the INT8
    workload produce such outputs).  The number of elements whose error is above
    2e-2, i.e. that needed the half-ulp term, is printed.
    """
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if got.size == 0:
        return -1.0
    err = np.abs(got - ref)
    n_extra = int(np.count_nonzero(err > BF16_TOL))
    if n_extra:
        print(f"[bf16] {label} {n_extra} of {err.size} elements above 2e-2 (within 2e-2 + half ulp: "
              f"{int(np.count_nonzero(err <= BF16_TOL + half_ulp_bf16(ref)))})", flush=True)
    return float(np.max(err - (BF16_TOL + half_ulp_bf16(ref))))


def announce(name: str, **kw) -> None:
    print(f"[case] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)
