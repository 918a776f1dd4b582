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
* OScaR notes, step one "Canalized Rotation": the normalized Hadamard matrix
  (entries +-1/sqrt(d), H H^T = I) applied to q and k; the OSCAR summary
  page, section 5, composes it with a bit-reversal permutation P_br.  The
  structured rotation ``Hadamard`` is R = H / sqrt(d) or R = H P_br / sqrt(d)
  with Sylvester's H[i][k] = (-1)^popcount(i & k).

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


def bit_reverse(i, bits):
    """i with its ``bits`` low bits in reverse order."""
    r = 0
    for b in range(bits):
        r |= ((i >> b) & 1) << (bits - 1 - b)
    return r


_SIGNS = {}


def hadamard_signs(d, bitrev=False):
    """Integer matrix sqrt(d) R of the structured rotation: entry (i, k) is
    (-1)^popcount(i & c), c = bit_reverse(k) with ``bitrev`` (the column
    permutation P_br applied after Sylvester's H), else c = k."""
    if (d, bitrev) in _SIGNS:
        return _SIGNS[(d, bitrev)].copy()
    bits = d.bit_length() - 1
    assert d == 1 << bits
    col = [bit_reverse(k, bits) if bitrev else k for k in range(d)]
    m = np.empty((d, d), dtype=np.int64)
    for i in range(d):
        for k in range(d):
            m[i, k] = -1 if bin(i & col[k]).count("1") % 2 else 1
    _SIGNS[(d, bitrev)] = m
    return m.copy()


class Hadamard:
    """The structured rotation R = H / sqrt(d) (``bitrev`` False) or
    R = H P_br / sqrt(d) (``bitrev`` True), the same for every head."""

    def __init__(self, d=128, bitrev=False):
        self.d, self.bitrev = d, bitrev

    def signs(self):
        return hadamard_signs(self.d, self.bitrev)

    def matrix(self):
        """fp64 R (entries +-1/sqrt(d))."""
        return self.signs().astype(np.float64) / np.sqrt(self.d)


def _cmp_scaled(s, d, m):
    """Sign of s / sqrt(d) - m for rationals s, m, exactly."""
    a_neg, b_neg = s < 0, m < 0
    if a_neg != b_neg:
        return -1 if a_neg else 1
    if s == 0 and m == 0:
        return 0
    lhs, rhs = s * s, d * m * m          # |s / sqrt(d)|^2 vs |m|^2, both >= 0
    c = (lhs > rhs) - (lhs < rhs)
    return -c if a_neg else c


def round_scaled_to_bf16(s, d):
    """Correctly rounded (RNE) bf16 bits of s / sqrt(d) for a rational s."""
    guess = _ordinal(f64_to_bf16_bits(np.array([float(s) / np.sqrt(d)])))[0]

    def val(o):
        return Fraction(float(bf16_bits_to_f64(_from_ordinal(np.array([o])))[0]))

    o = guess
    while _cmp_scaled(s, d, (val(o) + val(o - 1)) / 2) < 0:
        o -= 1
    while _cmp_scaled(s, d, (val(o) + val(o + 1)) / 2) > 0:
        o += 1
    # now the value lies within [mid(o - 1, o), mid(o, o + 1)]; a tie goes to
    # the even significand
    if _cmp_scaled(s, d, (val(o) + val(o - 1)) / 2) == 0 and int(_from_ordinal(np.array([o]))[0]) & 1:
        o -= 1
    elif _cmp_scaled(s, d, (val(o) + val(o + 1)) / 2) == 0 and int(_from_ordinal(np.array([o]))[0]) & 1:
        o += 1
    return _from_ordinal(np.array([o]))[0]


def hadamard_rotate_to_bf16(x_bits, bitrev=False):
    """bf16 bits of x . H (P_br) / sqrt(d) for bf16 rows ``x_bits`` [N, d],
    correctly rounded from the exact value.

    s = x . (sqrt(d) R) is a signed sum of the row's values; its fp64 value
    errs by less than 2 d u sum|x_i|, so y = s / sqrt(d) in fp64 errs by less
    than that over sqrt(d) plus 4u|y|.  Elements whose bound straddles a bf16
    rounding boundary are recomputed from the exact rational s.
    """
    x = bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))
    d = x.shape[1]
    sg = hadamard_signs(d, bitrev)
    s = x @ sg.astype(np.float64)
    y = s / np.sqrt(d)
    bound = (2.0 * d * _U * (np.abs(x).sum(axis=1, keepdims=True)) / np.sqrt(d)
             + 4.0 * _U * np.abs(y) + 2.0 ** -1070)
    out = f64_to_bf16_bits(y)
    o = _ordinal(out)
    v = bf16_bits_to_f64(out)
    mid_lo = (v + bf16_bits_to_f64(_from_ordinal(o - 1))) * 0.5
    mid_hi = (v + bf16_bits_to_f64(_from_ordinal(o + 1))) * 0.5
    safe = (y - bound > mid_lo) & (y + bound < mid_hi)
    for i, j in np.argwhere(~safe):
        exact = sum((Fraction(a) * int(b) for a, b in zip(x[i].tolist(), sg[:, j].tolist())),
                    Fraction(0))
        out[i, j] = round_scaled_to_bf16(exact, d)
    return out


def rotate_rows_to_bf16(x_bits, r):
    """bf16 rows x . R for a dense fp32 R [D, D] or a ``Hadamard``."""
    if isinstance(r, Hadamard):
        return hadamard_rotate_to_bf16(x_bits, r.bitrev)
    return rotate_to_bf16(x_bits, r)


def as_matrix(r):
    """fp64 matrix of a dense R or a ``Hadamard``."""
    if isinstance(r, Hadamard):
        return r.matrix()
    return np.asarray(r, dtype=np.float64)


def rotate_heads_to_bf16(x_bits, r_heads, g=1):
    """Rotate rows [N, H, D] where head h uses r_heads[h // g]; bf16 bits out."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    n, h, d = x_bits.shape
    out = np.empty_like(x_bits)
    for hh in range(h):
        out[:, hh, :] = rotate_rows_to_bf16(x_bits[:, hh, :], r_heads[hh // g])
    return out
