"""O1: fixed per-head rotation of keys, values and queries.

Test infrastructure (see ``oracle/__init__.py``).

Sources:
* OSCAR summary page, section 5 "Rotation Analysis": one fixed composed
  rotation R = U . H_Had . P_br per layer and head; section 4: keys and values
  are rotated before the cache write, and the value rotation can be absorbed
  into the projections.
* OScaR notes, "Hadamard transform" / "Canalized Rotation": an orthogonal
  transform applied to both q and k leaves q.k unchanged.
* WUSH-KV notes, "method step details": the key transform is applied online,
  after RoPE, to each new key and each new query.

Convention (row vectors): x' = x . R, x' of a query uses the R_K of its KV head
(query head hq belongs to KV head hq // g).  The rotated row is rounded once to
bf16.  ``rotate_to_bf16`` returns the correctly rounded bf16 of the *exact*
product: the fp64 product is used when it provably rounds the same way, and
the rare element whose error bound straddles a bf16 rounding boundary is
recomputed in exact rational arithmetic.
"""

from fractions import Fraction

import numpy as np

from .rounding import f64_to_bf16_bits, bf16_bits_to_f64

_U = 2.0 ** -53


def rotate_f64(x, r):
    """Unrounded x . R in fp64 for float64 rows x [N, D] and R [D, D]."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(r, dtype=np.float64)


def _ordinal(bits):
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def _from_ordinal(o):
    o = np.asarray(o, dtype=np.int64)
    return np.where(o < 0, (-o) | 0x8000, o).astype(np.uint16)


def _round_fraction_to_bf16(v):
    """Correctly rounded (RNE) bf16 bits of an exact rational v."""
    guess = _ordinal(f64_to_bf16_bits(np.array([float(v)])))[0]
    best = None
    for o in (guess - 1, guess, guess + 1):
        bits = _from_ordinal(np.array([o]))[0]
        val = Fraction(float(bf16_bits_to_f64(np.array([bits]))[0]))
        dist = abs(val - v)
        even = (int(bits) & 1) == 0
        key = (dist, 0 if even else 1)
        if best is None or key < best[0]:
            best = (key, bits)
    return best[1]


def exact_row_dot_bf16(x_row, r_col):
    """bf16 bits of the exact dot product of two float64 vectors (rationals)."""
    acc = Fraction(0)
    for a, b in zip(x_row.tolist(), r_col.tolist()):
        acc += Fraction(a) * Fraction(b)
    return _round_fraction_to_bf16(acc)


def rotate_to_bf16(x_bits, r):
    """bf16 bits of x . R for bf16 rows ``x_bits`` [N, D] and fp32 R [D, D].

    Each product x_i R_ij (8-bit times 24-bit significands) is exact in fp64,
    so the fp64 result differs from the exact sum by at most
    bound = 2 D u sum_i |x_i R_ij|.  When [y - bound, y + bound] stays strictly
    between the two bf16 rounding boundaries around bf16(y), bf16(y) is the
    correctly rounded value; otherwise the element is recomputed exactly.
    """
    x = bf16_bits_to_f64(x_bits)
    rd = np.asarray(r, dtype=np.float32).astype(np.float64)
    d = rd.shape[0]
    y = x @ rd
    bound = 2.0 * d * _U * (np.abs(x) @ np.abs(rd)) + 2.0 ** -1070
    out = f64_to_bf16_bits(y)
    o = _ordinal(out)
    v = bf16_bits_to_f64(out)
    v_lo = bf16_bits_to_f64(_from_ordinal(o - 1))
    v_hi = bf16_bits_to_f64(_from_ordinal(o + 1))
    mid_lo = (v + v_lo) * 0.5
    mid_hi = (v + v_hi) * 0.5
    safe = (y - bound > mid_lo) & (y + bound < mid_hi)
    bad = np.argwhere(~safe)
    for i, j in bad:
        out[i, j] = exact_row_dot_bf16(x[i], rd[:, j])
    return out


def rotate_heads_to_bf16(x_bits, r_heads, g=1):
    """Rotate rows [N, H, D] where head h uses r_heads[h // g]; bf16 bits out."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    n, h, d = x_bits.shape
    out = np.empty_like(x_bits)
    for hh in range(h):
        out[:, hh, :] = rotate_to_bf16(x_bits[:, hh, :], r_heads[hh // g])
    return out
