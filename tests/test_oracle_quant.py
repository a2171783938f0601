"""Pins for the INT8 block encoder oracle (CPU only).

Independent routes to the same codes: exact rational arithmetic with
fractions.Fraction (correctly rounded to fp32 through fp64, which is innocuous
for a single division since 53 >= 2*24 + 2), Python's round() (half to even)
and decimal's ROUND_HALF_EVEN; hand-made half-way cases; the error bound of the
encoding.
"""

import decimal
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from hybrid_swa_kv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32(x):
    return float(np.float32(x))


def exact_encode_block(block):
    """Encode one [32, D] block with exact rationals."""
    vals = [float(x) for x in np.asarray(block, dtype=np.float32).ravel()]
    a = max(abs(x) for x in vals)
    if a == 0.0:
        return [0] * len(vals), 0.0
    s = _f32(float(Fraction(a) / 127))
    codes = []
    for x in vals:
        quot = _f32(float(Fraction(x) / Fraction(s)))
        c1 = round(quot)                                        # banker's rounding
        c2 = int(decimal.Decimal(quot).to_integral_value(rounding=decimal.ROUND_HALF_EVEN))
        assert c1 == c2
        codes.append(max(-127, min(127, c1)))
    return codes, s


def test_golden_halfway_cases():
    with open(os.path.join(GOLDEN, "int8_halfway_cases.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        x = np.zeros((32, 4), dtype=np.float32)
        vals = np.array(case["x"], dtype=np.float32)
        x.ravel()[: len(vals)] = vals
        codes, scales = oracle.kv_quant_int8_b32(x[None])
        assert float(scales[0, 0]) == case["scale"]
        assert codes.ravel()[: len(vals)].tolist() == case["codes"]


def test_zero_block_and_absmax():
    x = np.zeros((2, 64, 8), dtype=np.float32)
    x[1, 40, 3] = -3.25
    x[1, 33, 0] = 1.0
    codes, scales = oracle.kv_quant_int8_b32(x)
    assert scales.shape == (2, 2)
    assert scales[0, 0] == 0 and scales[0, 1] == 0 and scales[1, 0] == 0
    assert not codes[0].any() and not codes[1, :32].any()
    assert codes[1, 40, 3] == -127
    assert scales[1, 1] == np.float32(3.25) / np.float32(127)
    assert codes.min() >= -127


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_exact_rational_encoder(seed):
    bits = synth.head_major(40 + seed, synth.K, 1, 1, 96, 16, outlier_p=0.02)
    x = synth.bf16_bits_to_f32(bits)[0, 0]
    x[5:37, :] *= np.float32(2.0 ** -20)                    # a block of tiny values
    codes, scales = oracle.kv_quant_int8_b32(x)
    for n in range(3):
        ref_codes, ref_s = exact_encode_block(x[32 * n: 32 * n + 32])
        assert float(scales[n]) == ref_s
        assert codes[32 * n: 32 * n + 32].ravel().tolist() == ref_codes


def test_roundtrip_bound():
    bits = synth.head_major(50, synth.V, 2, 3, 256, 32, outlier_p=0.01)
    x = synth.bf16_bits_to_f32(bits)
    codes, scales = oracle.kv_quant_int8_b32(x)
    deq = oracle.dequant_int8_b32(codes, scales)
    s = np.repeat(scales.astype(np.float64), 32, axis=-1)[..., None]
    err = np.abs(x.astype(np.float64) - deq)
    assert np.all(err <= s * (0.5 + 2.0 ** -18))
    # every block reaches +-127 at its absmax element
    blk = np.abs(codes.reshape(2, 3, 8, 32 * 32)).max(axis=-1)
    assert np.all(blk == 127)


def test_dequant_exact():
    c = np.array([[[-127, 3], [5, 127]]], dtype=np.int8).repeat(16, axis=1)  # [1, 32, 2]
    s = np.array([[0.1]], dtype=np.float32)
    d = oracle.dequant_int8_b32(c, s)
    assert d[0, 0, 0] == -127 * float(np.float32(0.1))
    assert d[0, 16, 1] == 127 * float(np.float32(0.1))
    assert d[0, 1, 1] == 3 * float(np.float32(0.1))
