"""The bf16 tolerance helper against torch's own bf16 rounding (CPU only)."""

import numpy as np
import torch

from tests.helpers import BF16_TOL, bf16_excess, half_ulp_bf16


def test_half_ulp_bounds_the_rounding_of_bf16():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(200000) * 10.0 ** rng.integers(-6, 6, 200000),
                        [1.0, 2.0, 7.999, 8.0, 15.9, 16.0, -8.0, 1e-38, -3e-39]])
    r = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    err = np.abs(r - x.astype(np.float32).astype(np.float64))
    assert np.all(err <= half_ulp_bf16(x) * (1 + 1e-12))
    # the bound is reached: a value half-way between two bf16 neighbours
    for v in (1.0, 8.0, 12.0, 1024.0):
        h = half_ulp_bf16(v)
        mid = v + float(h)
        assert torch.tensor(mid, dtype=torch.float32).to(torch.bfloat16).item() in (v, v + 2 * float(h))


def test_half_ulp_values():
    assert half_ulp_bf16(1.0) == 2.0 ** -8
    assert half_ulp_bf16(1.99) == 2.0 ** -8
    assert half_ulp_bf16(7.99) == 2.0 ** -6
    assert half_ulp_bf16(8.0) == 2.0 ** -5     # 2^-5 > 2e-2 from |x| = 8 on
    assert half_ulp_bf16(-0.5) == 2.0 ** -9


def test_excess_bar():
    ref = np.array([0.1, 9.0])
    assert bf16_excess(ref + BF16_TOL, ref) <= 0
    assert bf16_excess(ref + np.array([BF16_TOL + 2 * half_ulp_bf16(0.1), 0.0]), ref) > 0
    # at |ref| = 9 the bar is 2e-2 + 2^-5
    assert bf16_excess(np.array([0.1, 9.0 + 0.05]), ref) <= 0
    assert bf16_excess(np.array([0.1, 9.0 + 0.052]), ref) > 0
