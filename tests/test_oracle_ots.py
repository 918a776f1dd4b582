"""Pins of O7, the OScaR variant (``oracle/ots.py``): the KIVI per-channel
formulas, Omni-Token Scaling, exact codes, error bounds and the storage
figure the OScaR notes give."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import ots, rotate
from oracle.rounding import bf16_bits_to_f64, f64_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _b(x):
    return f64_to_bf16_bits(np.asarray(x, np.float64))


def test_worked_example_block_range():
    # OScaR notes: a block spanning [-3, 3] at 2 bits has Delta = 2 and error
    # bound Delta / 2 = 1; per channel, z = -min / Delta = 1.5 and the four
    # levels Delta (Q - z) are -3, -1, 1, 3
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    lo, hi = g["range"]
    col = np.array([lo, -2.0, -1.0, 0.0, 0.5, 1.0, 2.0, hi])
    codes, d16, z16 = ots.channel_quantize(_b(col[:, None]))
    assert bf16_bits_to_f64(d16)[0] == g["delta"] and bf16_bits_to_f64(z16)[0] == 1.5
    # v = u / 2 + 1.5: -3 -> 0, -2 -> 0.5 (tie, even 0), -1 -> 1, 0 -> 1.5 (tie, even 2),
    # 0.5 -> 1.75, 1 -> 2, 2 -> 2.5 (tie, even 2), 3 -> 3
    assert codes[:, 0].tolist() == [0, 0, 1, 2, 2, 2, 2, 3]
    rec = ots.channel_dequant(codes, d16, z16)[:, 0]
    assert rec.tolist() == [-3.0, -3.0, -1.0, 1.0, 1.0, 1.0, 1.0, 3.0]
    assert np.abs(rec - col).max() <= g["error_bound"]


def test_per_channel_blocks_are_independent():
    # each channel has its own range; scaling one channel leaves the others' codes
    rng = np.random.default_rng(2)
    u = rng.standard_normal((32, 128)) * 0.1
    c1, d1, z1 = ots.channel_quantize(_b(u))
    u2 = u.copy()
    u2[:, 7] *= 8.0
    c2, d2, z2 = ots.channel_quantize(_b(u2))
    keep = np.arange(128) != 7
    assert np.array_equal(c1[:, keep], c2[:, keep]) and np.array_equal(d1[keep], d2[keep])
    assert bf16_bits_to_f64(d2)[7] == bf16_bits_to_f64(f64_to_bf16_bits(
        np.array([(bf16_bits_to_f64(_b(u2[:, 7])).max() - bf16_bits_to_f64(_b(u2[:, 7])).min()) / 3])))[0]


def test_codes_equal_exact_rational_rounding():
    # Q = clamp(rne(u / Delta16 + z16), 0, 3) in exact rationals
    rng = np.random.default_rng(4)
    u16 = _b(rng.standard_normal((16, 24)) * np.exp(rng.uniform(-2, 2, (1, 24))))
    codes, d16, z16 = ots.channel_quantize(u16)
    u = bf16_bits_to_f64(u16)
    dl, z = bf16_bits_to_f64(d16), bf16_bits_to_f64(z16)
    for j in range(24):
        for i in range(16):
            v = Fraction(u[i, j]) / Fraction(dl[j]) + Fraction(z[j])
            fl = v.numerator // v.denominator
            r = v - fl
            q = fl + (1 if r > Fraction(1, 2) or (r == Fraction(1, 2) and fl % 2 == 1) else 0)
            assert codes[i, j] == min(3, max(0, q)), (i, j)


def test_constant_channel_decodes_to_its_value():
    u = np.tile(np.array([[0.25, -1.5, 3.0]]), (8, 1))
    codes, d16, z16 = ots.channel_quantize(_b(u))
    assert np.all(bf16_bits_to_f64(d16) == 0) and np.all(codes == 0)
    assert np.array_equal(ots.channel_dequant(codes, d16, z16), u)


def test_ots_unit_norm_and_uniform_row():
    # a rotated row c (+-1, ..., +-1) has norm c sqrt(d): s = c sqrt(128), u = +-1/sqrt(128)
    row = np.where(np.arange(128) % 3 == 0, -0.5, 0.5)[None, :]
    s16, u16 = ots.ots_scale(_b(row))
    assert bf16_bits_to_f64(s16)[0] == bf16_bits_to_f64(_b([0.5 * np.sqrt(128)]))[0]
    rng = np.random.default_rng(6)
    k = _b(rng.standard_normal((64, 128)) * np.exp(rng.uniform(-4, 4, (64, 1))))
    s16, u16 = ots.ots_scale(k)
    norms = np.sqrt((bf16_bits_to_f64(u16) ** 2).sum(axis=1))
    assert np.all(np.abs(norms - 1.0) < 2 ** -7)           # bf16 rounding of s and of u
    s, z = ots.ots_scale(np.zeros((1, 128), np.uint16))
    assert s[0] == 0 and np.all(z == 0)


def test_ots_keys_error_bound_and_token_norm_imbalance():
    # tokens whose norms differ by 2^8 (the token norm imbalance OTS removes):
    # every decoded key is within s_t * Delta_j / 2 of its rotated row
    rng = np.random.default_rng(8)
    G = 32
    k = rng.standard_normal((2 * G, 128)) * np.exp(rng.uniform(-4, 4, (2 * G, 1)))
    kb = _b(k)
    dec = ots.ots_keys(kb, G, bitrev=True)
    k_rot = rotate.hadamard_rotate_to_bf16(kb, True)
    s16, u16 = ots.ots_scale(k_rot)
    s = bf16_bits_to_f64(s16)
    for b0 in (0, G):
        _, d16, _ = ots.channel_quantize(u16[b0:b0 + G])
        bound = s[b0:b0 + G, None] * bf16_bits_to_f64(d16)[None, :] * 0.5
        err = np.abs(dec[b0:b0 + G] - s[b0:b0 + G, None] * bf16_bits_to_f64(u16[b0:b0 + G]))
        # the stored z16 is a rounded -min / Delta: allow one bf16 ulp of z times Delta
        slack = s[b0:b0 + G, None] * bf16_bits_to_f64(d16)[None, :] * 2 ** -6
        assert np.all(err <= bound + slack + 1e-12)


def test_storage_figure():
    # "32 + 2 = 34 bytes" per INT2 key token-head with OTS at d = 128
    assert ots.key_bytes_per_token_head(128) == 34


def test_norm_independent_of_channel_order():
    # rows whose squares span more than 53 bits (so a running fp64 sum would
    # depend on the order): the token scale and the normalized row are the
    # same for every permutation of the channels (reading 1: one rounding of
    # the exact sum), and the scale is bf16(sqrt) of the exact rational sum
    rng = np.random.default_rng(5)
    for _ in range(20):
        row = rng.standard_normal(128) * 2.0 ** rng.integers(-30, 30, 128)
        k = _b(row[None, :])
        s16, u16 = ots.ots_scale(k)
        exact = sum(Fraction(float(x)) ** 2 for x in bf16_bits_to_f64(k[0]))
        assert s16[0] == _b(np.sqrt(np.float64(float(exact))))[0]
        for _ in range(3):
            p = rng.permutation(128)
            s2, u2 = ots.ots_scale(k[:, p])
            assert s2[0] == s16[0] and np.array_equal(u2[0], u16[0, p])


def test_zero_extreme_is_positive_zero():
    # a channel whose block minimum is zero, held once as -0 and once as +0:
    # both give the same parameters (reading 6)
    base = np.linspace(0.0, 0.75, 32)
    a = _b(base[:, None])
    b = a.copy()
    b[0, 0] = 0x8000                     # -0 in place of +0
    ca, da, za = ots.channel_quantize(a)
    cb, db, zb = ots.channel_quantize(b)
    assert np.array_equal(ca, cb) and np.array_equal(da, db) and np.array_equal(za, zb)
    assert za[0] == 0x8000               # bf16(-(+0) / Delta) = -0
