"""Pins of the oracle's quantizer, dequantizer and page packing (CPU)."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import quant, layout
from oracle.rounding import fp16_bits_to_f64, bf16_bits_to_f64
from synth import bf16_from_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_rows(rng, shape, scale=1.0):
    return bf16_bits_to_f64(bf16_from_f32((rng.standard_normal(shape) * scale).astype(np.float32)))


@pytest.mark.parametrize("g", [32, 64, 128])
def test_quantile_matches_numpy(g):
    # library routine: np.quantile's default ("linear", Hyndman-Fan type 7)
    rng = np.random.default_rng(10 + g)
    x = _bf16_rows(rng, (4000, g))
    kap = rng.uniform(0.5, 1.0, 4000).astype(np.float32)
    srt = np.sort(x, axis=-1)
    hi = quant.quantile_type7(srt, kap.astype(np.float64))
    lo = quant.quantile_type7(srt, 1.0 - kap.astype(np.float64))
    ref_hi = np.array([np.quantile(r, float(k)) for r, k in zip(x, kap)])
    ref_lo = np.array([np.quantile(r, 1.0 - float(k)) for r, k in zip(x, kap)])
    assert np.array_equal(hi, ref_hi)
    assert np.array_equal(lo, ref_lo)


def test_kappa_one_is_min_max():
    rng = np.random.default_rng(3)
    x = _bf16_rows(rng, (500, 64))
    lo, hi = quant.clip_range(x, np.float32(1.0))
    assert np.array_equal(lo, x.min(-1)) and np.array_equal(hi, x.max(-1))


def test_worked_example_delta_and_bound():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    lo, hi = ex["range"]
    # a group spanning exactly [lo, hi] (bf16 and fp16 representable points)
    x = np.linspace(lo, hi, 128)
    x = bf16_bits_to_f64(bf16_from_f32(x.astype(np.float32)))
    x[0], x[-1] = lo, hi
    codes, s16, z16 = quant.quantize_rows(x[None, :], np.float32(1.0), 128)
    s = fp16_bits_to_f64(s16)[0, 0]
    z = fp16_bits_to_f64(z16)[0, 0]
    assert s == ex["delta"] == (hi - lo) / (2 ** ex["bits"] - 1)
    assert z == lo
    xh = quant.dequant_rows(codes, s16, z16, 128)[0]
    assert np.abs(xh - x).max() <= ex["error_bound"] == s / 2


def _exact_code(x, s, z):
    """Nearest grid point k in {0..3} to (x - z)/s in exact rationals, ties to even."""
    if s == 0:
        return 0
    t = (Fraction(x) - Fraction(z)) / Fraction(s)
    best = None
    for k in range(4):
        key = (abs(t - k), k % 2)
        if best is None or key < best[0]:
            best = (key, k)
    return best[1]


@pytest.mark.parametrize("g", [32, 64, 128])
def test_codes_exact_rational_brute_force(g):
    rng = np.random.default_rng(20 + g)
    x = _bf16_rows(rng, (60, g), scale=3.0)
    codes, s16, z16 = quant.quantize_rows(x, np.float32(0.9), g)
    s = fp16_bits_to_f64(s16)[:, 0]
    z = fp16_bits_to_f64(z16)[:, 0]
    for r in range(x.shape[0]):
        for j in range(g):
            assert codes[r, j] == _exact_code(x[r, j], s[r], z[r])


def test_codes_at_exact_ties_round_half_even():
    # x exactly on the thresholds z + s/2, z + 3s/2, z + 5s/2 -> codes 0, 2, 2
    s = np.array([[0.5]])
    z = np.array([[-1.0]])
    xg = np.array([[[-0.75, -0.25, 0.25, -0.7, 0.3, 5.0, -9.0]]])
    c = quant.codes_from_params(xg, s, z)[0, 0]
    assert c.tolist() == [0, 2, 2, 1, 3, 3, 0]


@pytest.mark.parametrize("v", [1.5, -0.375, 0.0, 7.0, -1024.0])
@pytest.mark.parametrize("kappa", [0.5, 0.9, 1.0])
def test_all_equal_group_round_trips(v, kappa):
    x = np.full((3, 128), v)
    for g in (32, 64, 128):
        c, s16, z16 = quant.quantize_rows(x, np.float32(kappa), g)
        assert np.array_equal(quant.dequant_rows(c, s16, z16, g), x)
        assert (fp16_bits_to_f64(s16) == 0).all() and (c == 0).all()


@pytest.mark.parametrize("g", [32, 64, 128])
def test_error_bound_inside_clip_range(g):
    rng = np.random.default_rng(30 + g)
    x = _bf16_rows(rng, (3000, 128), scale=2.0)
    kap = np.float32(0.92)
    codes, s16, z16 = quant.quantize_rows(x, kap, g)
    xh = quant.dequant_rows(codes, s16, z16, g)
    xg = x.reshape(3000, -1, g)
    hg = xh.reshape(3000, -1, g)
    lo, hi = quant.clip_range(xg, kap)
    s = fp16_bits_to_f64(s16)
    z = fp16_bits_to_f64(z16)
    pre = (np.abs(z - lo) <= s / 2) & (np.abs(z + 3 * s - hi) <= s / 2)
    assert pre.mean() > 0.999              # fp16 rounding of s, z is tiny here
    err = np.abs(xg - hg)
    inside = (xg >= lo[..., None]) & (xg <= hi[..., None]) & pre[..., None]
    assert (err[inside] <= np.broadcast_to(s[..., None], err.shape)[inside] / 2).all()
    # outside the clip range the value is clamped to the nearest end level
    above = (xg > z[..., None] + 2.5 * s[..., None])
    assert np.allclose(hg[above], np.broadcast_to((z + 3 * s)[..., None], hg.shape)[above])
    below = (xg <= z[..., None] + 0.5 * s[..., None])
    assert np.array_equal(hg[below], np.broadcast_to(z[..., None], hg.shape)[below])


def test_dequant_is_exact_affine():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 4, (50, 128)).astype(np.uint8)
    s16 = np.full((50, 2), np.float16(0.3).view(np.uint16))
    z16 = np.full((50, 2), np.float16(-0.7).view(np.uint16))
    xh = quant.dequant_rows(codes, s16, z16, 64)
    exp = [[Fraction(float(np.float16(0.3))) * int(c) + Fraction(float(np.float16(-0.7)))
            for c in row] for row in codes[:3]]
    assert [[Fraction(v) for v in row] for row in xh[:3]] == exp


def test_pack_repeating_codes_gives_e4():
    c = np.tile(np.arange(4, dtype=np.uint8), (16, 32))     # code = channel % 4
    assert (layout.pack_k_codes(c) == 0xE4E4E4E4).all()
    assert (layout.pack_v_codes(c) == 0xE4E4E4E4).all()


def test_pack_bit_positions():
    c = np.zeros((16, 128), np.uint8)
    c[5, 37] = 3          # K: slot 5, channel 37 -> word 5*8 + 2, bits 10..11
    kw = layout.pack_k_codes(c)
    assert kw[5 * 8 + 2] == 3 << 10 and np.count_nonzero(kw) == 1
    vw = layout.pack_v_codes(c)   # V: slot 5 = 4*1 + 2*0 + 1, channel 37 = 8*4 + 5
    assert vw[2 * (16 * 1 + 4) + 0] == 3 << (16 + 10) and np.count_nonzero(vw) == 1


@pytest.mark.parametrize("g", [32, 64, 128])
def test_page_pack_round_trip(g):
    rng = np.random.default_rng(40 + g)
    ng = 128 // g
    kc = rng.integers(0, 4, (16, 128)).astype(np.uint8)
    vc = rng.integers(0, 4, (16, 128)).astype(np.uint8)
    ps = [rng.integers(0, 1 << 16, (16, ng)).astype(np.uint16) for _ in range(4)]
    blk = layout.pack_page_head(kc, vc, *ps, g)
    assert blk.size == layout.page_head_bytes(g) == 1024 + 128 * ng
    out = layout.unpack_page_head(blk, g)
    for a, b in zip(out, (kc, vc, *ps)):
        assert np.array_equal(a, b)


def test_window_block_round_trip_and_permutation():
    idx = layout.v_window_index(np.arange(16)[:, None], np.arange(128)[None, :])
    assert np.array_equal(np.sort(idx.ravel()), np.arange(2048))
    rng = np.random.default_rng(5)
    k = rng.integers(0, 1 << 16, (16, 128)).astype(np.uint16)
    v = rng.integers(0, 1 << 16, (16, 128)).astype(np.uint16)
    k2, v2 = layout.unpack_window_block(layout.pack_window_block(k, v))
    assert np.array_equal(k, k2) and np.array_equal(v, v2)


def test_bytes_per_token_head_match_pages():
    mb = json.load(open(os.path.join(GOLDEN, "memory_bytes.json")))
    bf16 = mb["bf16_bytes_per_token_head"]
    assert bf16 == 128 * 2 * 2
    per_tok = {g: layout.page_head_bytes(g) / 16 for g in (128, 64, 32)}
    assert per_tok == {128: 72.0, 64: 80.0, 32: 96.0}
    assert round(bf16 / per_tok[32], 1) == mb["int2_ratio_g32"]
    assert per_tok[128] * 8 / 2 / 128 == mb["int2_bits_per_element_g128_without_windows"]


def test_signed_zero_order_statistic_is_plus_zero():
    # kappa = 1: lo is the group minimum; a group whose minimum is zero, held
    # as -0 in some channels and +0 in others, stores the zero point +0
    g = 32
    x = np.abs(np.linspace(0.0, 3.0, g))
    x[[0, 5, 9]] = -0.0
    x[[1, 2]] = 0.0
    lo, hi = quant.clip_range(x[None, :], 1.0)
    assert lo[0] == 0.0 and not np.signbit(lo[0]) and hi[0] == 3.0
    _, s, z = quant.quantize_rows(x[None, :], 1.0, g)
    assert int(z[0, 0]) == 0x0000
    # kappa < 1 whose lower quantile interpolates between -0 and +0 is +0 too
    y = np.concatenate([[-1.0], [-0.0] * 10, [0.0] * 10, np.linspace(0.5, 2.0, g - 21)])
    lo2, _ = quant.clip_range(y[None, :], 0.9)
    assert lo2[0] == 0.0 and not np.signbit(lo2[0])
