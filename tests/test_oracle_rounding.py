"""Pins of the oracle's fp64 -> bf16 / fp16 roundings (CPU)."""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle.rounding import (f64_to_bf16_bits, bf16_bits_to_f64,
                             f64_to_fp16_bits, fp16_bits_to_f64)


def _all_bf16_values():
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    vals = bf16_bits_to_f64(bits)
    keep = np.isfinite(vals)
    return bits[keep], vals[keep]


def _nearest_by_table(x, table_bits, table_vals, mant_mask):
    """Exact nearest representable value, ties to even significand (brute force)."""
    fx = Fraction(x)
    i = np.searchsorted(table_vals, x)
    best = None
    for j in (i - 2, i - 1, i, i + 1):
        if 0 <= j < len(table_vals):
            d = abs(Fraction(float(table_vals[j])) - fx)
            even = (int(table_bits[j]) & 1) == 0
            key = (d, 0 if even else 1)
            if best is None or key < best[0]:
                best = (key, table_bits[j], table_vals[j])
    return best[2]


@pytest.fixture(scope="module")
def bf16_table():
    bits, vals = _all_bf16_values()
    order = np.argsort(vals, kind="stable")
    bits, vals = bits[order], vals[order]
    # drop -0 duplicate so the table is strictly increasing
    keep = np.concatenate([[True], np.diff(vals) > 0])
    return bits[keep], vals[keep]


def test_bf16_matches_torch_on_fp32_inputs():
    # For inputs exactly representable in fp32, torch's fp32 -> bf16 cast is a
    # single RNE rounding, so it must agree with the fp64 path bit for bit.
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200_000) * np.exp2(rng.integers(-140, 120, 200_000))).astype(np.float32)
    x[:8] = [0.0, -0.0, 1.0, -2.5, 1e-45, 3.3e38, -1e-40, 65504.0]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = f64_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_exact_nearest_brute_force(bf16_table):
    bits_t, vals_t = bf16_table
    rng = np.random.default_rng(1)
    x = rng.standard_normal(3000) * np.exp2(rng.integers(-135, 126, 3000).astype(np.float64))
    got = bf16_bits_to_f64(f64_to_bf16_bits(x))
    for xi, gi in zip(x, got):
        assert gi == _nearest_by_table(xi, bits_t, vals_t, 0x7F)


@pytest.mark.parametrize("x, expect", [
    (1.0 + 2.0 ** -8, 1.0),                         # exact tie -> even (down)
    (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),         # exact tie -> even (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 1.0 + 2.0 ** -7),  # just above tie (fp32 would round twice)
    (1.0 + 2.0 ** -8 - 2.0 ** -40, 1.0),
    (-(1.0 + 2.0 ** -8 + 2.0 ** -40), -(1.0 + 2.0 ** -7)),
    (2.0 ** -133, 2.0 ** -133),                     # smallest subnormal
    (2.0 ** -134, 0.0),                             # tie to even -> 0
    (2.0 ** -134 + 2.0 ** -160, 2.0 ** -133),
    (3 * 2.0 ** -134, 2.0 ** -132),                 # subnormal tie -> even
    (2.0 ** -126 - 2.0 ** -134, 2.0 ** -126),       # rounds up into the normals
    (3.3895313892515355e38, 3.3895313892515355e38),  # max bf16
    (3.4e38, float("inf")),
])
def test_bf16_constructed_cases(x, expect):
    got = bf16_bits_to_f64(f64_to_bf16_bits(np.array([x])))[0]
    assert got == expect and np.signbit(got) == np.signbit(expect)


def test_fp16_exact_nearest_brute_force():
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    vals = fp16_bits_to_f64(bits)
    keep = np.isfinite(vals)
    bits, vals = bits[keep], vals[keep]
    order = np.argsort(vals, kind="stable")
    bits, vals = bits[order], vals[order]
    k = np.concatenate([[True], np.diff(vals) > 0])
    bits, vals = bits[k], vals[k]
    rng = np.random.default_rng(2)
    x = rng.standard_normal(3000) * np.exp2(rng.integers(-26, 15, 3000).astype(np.float64))
    got = fp16_bits_to_f64(f64_to_fp16_bits(x))
    for xi, gi in zip(x, got):
        assert gi == _nearest_by_table(xi, bits, vals, 0x3FF)


@pytest.mark.parametrize("x, expect", [
    (1.0 + 2.0 ** -11, 1.0),                         # tie -> even
    (1.0 + 2.0 ** -11 + 2.0 ** -40, 1.0 + 2.0 ** -10),  # single rounding (fp32 path gives 1.0)
    (1.0 + 2.0 ** -11 - 2.0 ** -40, 1.0),
    (2.0 ** -25, 0.0),                               # subnormal tie -> 0
    (2.0 ** -25 + 2.0 ** -60, 2.0 ** -24),
    (65519.99, 65504.0),
    (65520.0, float("inf")),                         # tie above max -> inf
])
def test_fp16_constructed_cases(x, expect):
    assert fp16_bits_to_f64(f64_to_fp16_bits(np.array([x])))[0] == expect
