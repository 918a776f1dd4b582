"""The kernels' fp64 -> bf16 / fp16 rounding routines (the same source,
compiled for the host and exported as oscar_round_f64_host) against the
oracle's independent single roundings, on crafted ties, near-ties, carries
into the exponent, the bf16 / fp16 normal-range edges, subnormals, overflow
and special values.  No GPU needed."""

import ctypes
import os

import numpy as np
import pytest

from oracle.rounding import f64_to_bf16_bits, f64_to_fp16_bits
from ultra_bit_kv_amd import _lib


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("liboscar_kv.so not built")
    return _lib.lib()


def run(L, target, x):
    x = np.ascontiguousarray(x, np.float64)
    out = np.zeros(x.shape, np.uint16)
    st = L.oscar_round_f64_host(target, x.ctypes.data_as(ctypes.c_void_p),
                                out.ctypes.data_as(ctypes.c_void_p), x.size)
    assert st == 0
    return out


def crafted(mant_bits, emin, emax, rng):
    """Ties, near-ties and carries of a short float with `mant_bits` explicit
    significand bits and normal exponents emin .. emax, plus range edges."""
    xs = []
    k = rng.integers(0, 1 << mant_bits, 3000)
    e = rng.integers(emin - mant_bits - 2, emax + 2, 3000)
    base = (np.float64(1 << mant_bits) + k) * np.ldexp(1.0, e - mant_bits)
    half = np.ldexp(1.0, e - mant_bits - 1)
    for v in (base + half, base - half, np.nextafter(base + half, np.inf),
              np.nextafter(base + half, -np.inf), base):
        xs.append(v)
    # all-ones significands rounding up into the next binade
    top = (np.float64((1 << (mant_bits + 1)) - 1) + 0.5) * np.ldexp(1.0, np.arange(emin, emax + 1) - mant_bits)
    xs += [top, np.nextafter(top, 0.0)]
    edges = [np.ldexp(1.0, emin), np.nextafter(np.ldexp(1.0, emin), 0), np.ldexp(1.0, emin - 1),
             np.ldexp(1.0, emin - mant_bits), np.ldexp(1.0, emin - mant_bits - 1),
             np.nextafter(np.ldexp(1.0, emin - mant_bits - 1), 1.0),
             np.ldexp(1.0, emax), (2 - np.ldexp(1.0, -mant_bits)) * np.ldexp(1.0, emax),
             (2 - np.ldexp(1.0, -mant_bits - 1)) * np.ldexp(1.0, emax),
             np.nextafter((2 - np.ldexp(1.0, -mant_bits - 1)) * np.ldexp(1.0, emax), 0),
             np.ldexp(1.0, emax + 1), 1e300, 5e-324, 2.2250738585072014e-308, 0.0, np.inf]
    xs.append(np.array(edges))
    xs.append(rng.standard_normal(5000) * np.exp(rng.uniform(-80, 80, 5000)))
    x = np.concatenate(xs)
    return np.concatenate([x, -x])


def test_bf16_general_and_bit_pattern_routines(L):
    x = crafted(7, -126, 127, np.random.default_rng(11))
    want = f64_to_bf16_bits(x)
    assert np.array_equal(run(L, 0, x), want)
    assert np.array_equal(run(L, 2, x), want)


def test_fp16_routine(L):
    x = crafted(10, -14, 15, np.random.default_rng(12))
    assert np.array_equal(run(L, 1, x), f64_to_fp16_bits(x))
    # numpy's own fp64 -> fp16 cast is a single rounding too
    with np.errstate(over="ignore"):
        assert np.array_equal(run(L, 1, x), x.astype(np.float16).view(np.uint16))


def test_nan_and_argument_checks(L):
    out = run(L, 0, np.array([np.nan]))
    assert out[0] & 0x7F80 == 0x7F80 and out[0] & 0x7F != 0
    out = run(L, 1, np.array([np.nan]))
    assert out[0] & 0x7C00 == 0x7C00 and out[0] & 0x3FF != 0
    assert L.oscar_round_f64_host(3, None, None, 0) == -1
    buf = np.zeros(1)
    p = buf.ctypes.data_as(ctypes.c_void_p)
    assert L.oscar_round_f64_host(3, p, p, 1) == -10
    assert L.oscar_round_f64_host(0, p, p, -1) == -10
