"""fp64 -> bf16 and fp64 -> fp16, each a single round-to-nearest-even.

Test infrastructure (see ``oracle/__init__.py``).

The cache stores rotated rows as bf16 and the quantizer's scale and zero-point
as fp16 (OSCAR summary page, section 4 "KV Cache Layout / KV Cache Update";
the fp16 storage precision is this build's reading, listed in the design notes).
Both roundings here go straight from the fp64 value to the short format, so no
intermediate fp32 rounding can move a value across a tie.

* bf16: done on the integer bit pattern of the float64 (numpy has no bf16).
* fp16: numpy's own float64 -> float16 cast, which rounds once.
"""

import numpy as np

_U64 = np.uint64


def f64_to_bf16_bits(x):
    """Round float64 values to bf16 (RNE, subnormals kept), return uint16 bits.

    bf16 = 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.  A finite
    non-zero input is sig * 2**(e - 52) with a 53-bit integer significand
    ``sig``.  The bf16 quantum at exponent e is 2**(e - 7) for normal results
    (e >= -126) and 2**-133 below that, so the result's integer significand is
    sig / 2**shift rounded to nearest, ties to even, with shift = 45 for normal
    results and shift = -81 - e for subnormal ones.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    b = x.view(np.uint64)
    sign = ((b >> _U64(63)) & _U64(1)).astype(np.uint32) << 15
    expf = ((b >> _U64(52)) & _U64(0x7FF)).astype(np.int64)
    frac = b & _U64((1 << 52) - 1)

    normal64 = expf != 0
    sig = np.where(normal64, frac | _U64(1 << 52), frac)
    e = np.where(normal64, expf - 1023, -1022)
    # fp64 subnormals are < 2**-1022, far below half the smallest bf16.
    sub = e < -126
    shift = np.where(sub, -81 - e, 45)
    too_small = shift > 60
    shift_c = np.clip(shift, 1, 60).astype(np.uint64)

    q = sig >> shift_c
    rem = sig & ((_U64(1) << shift_c) - _U64(1))
    half = _U64(1) << (shift_c - _U64(1))
    up = (rem > half) | ((rem == half) & ((q & _U64(1)) == _U64(1)))
    q = (q + up.astype(np.uint64)).astype(np.int64)
    q = np.where(too_small, 0, q)

    # normal result: q in [128, 256]; q == 256 carries into the exponent.
    carry = (~sub) & (q == 256)
    e_n = np.where(carry, e + 1, e)
    q_n = np.where(carry, 128, q)
    bits_normal = ((e_n + 127) << 7) | (q_n - 128)
    bits_normal = np.where(e_n + 127 >= 255, 0x7F80, bits_normal)
    # subnormal result: q in [0, 128]; q == 128 is exactly the smallest normal.
    bits = np.where(sub, q, bits_normal)

    special = expf == 0x7FF
    is_nan = special & (frac != _U64(0))
    bits = np.where(special, np.where(is_nan, 0x7FC0, 0x7F80), bits)
    return (bits.astype(np.uint32) | sign).astype(np.uint16)


def bf16_bits_to_f64(bits):
    """Exact widening of bf16 bit patterns to float64."""
    bits = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return bits.view(np.float32).astype(np.float64)


def f64_to_fp16_bits(x):
    """Round float64 values to IEEE fp16 (RNE, subnormals kept); uint16 bits.

    numpy converts double -> half directly (one rounding), unlike a path
    through fp32, which can round twice.
    """
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x.astype(np.float16).view(np.uint16)


def fp16_bits_to_f64(bits):
    """Exact widening of fp16 bit patterns to float64."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
