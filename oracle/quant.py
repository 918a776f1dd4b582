"""O3 / O4: clipped asymmetric INT2 quantizer and its dequantizer.

Test infrastructure (see ``oracle/__init__.py``).

Sources:
* OScaR notes, "integer quantization basics": Q(x) = clamp(round(x/Delta + z),
  0, 2^b - 1), x_hat = Delta (Q(x) - z), |x - x_hat| <= Delta/2, and the
  min-max step Delta = (max - min) / (2^b - 1).
* OSCAR summary page, section 3 "Scale Determination and Clipping": affine
  asymmetric INT2 with scale and zero point for keys and values,
  percentile-based clipping; appendix A.5: per-token, per-group scales.
* WUSH-KV notes, "background: quantization groups and clipped quantizers": the
  OSCAR-style quantizer clips at the kappa-quantile (affine, with zero point).

Readings taken (all in the design notes):
1. Clip range of a group = [Q(1 - kappa), Q(kappa)], two-sided quantiles of
   the group's values, linear interpolation between order statistics (type 7).
   kappa = 1 is plain min-max.
2. Delta = (hi - lo) / 3, stored as fp16 ``s``; the zero point is stored as the
   fp16 *value* ``z`` = lo, so x_hat = s * code + z (the same affine map as
   Delta (Q - z') with z' = -lo / Delta, defined also when Delta = 0).
3. A zero order statistic is +0 (-0 and +0 are the same value; the stored
   zero point of a group whose lower clip limit is zero is then +0).
4. Codes are taken from the stored fp16 s and z: round-half-to-even of
   (x - z) / s clamped to [0, 3], which equals
   [x > z + s/2] + [x >= z + 3s/2] + [x > z + 5s/2] exactly.  s = 0 gives code 0.
"""

import numpy as np

from .rounding import f64_to_fp16_bits, fp16_bits_to_f64


def quantile_type7(sorted_groups, q):
    """Linear-interpolated quantile of each ascending-sorted group (last axis).

    h = (G - 1) q; i = floor(h); value = s[i] + (h - i) * (s[i+1] - s[i]),
    every operation one IEEE fp64 rounding, in this order.
    """
    s = np.asarray(sorted_groups, dtype=np.float64)
    g = s.shape[-1]
    q = np.asarray(q, dtype=np.float64)
    h = (g - 1) * q
    i = np.floor(h)
    f = h - i
    i = i.astype(np.int64)
    i1 = np.minimum(i + 1, g - 1)
    a = np.take_along_axis(s, np.broadcast_to(i[..., None], s.shape[:-1] + (1,)), -1)[..., 0]
    b = np.take_along_axis(s, np.broadcast_to(i1[..., None], s.shape[:-1] + (1,)), -1)[..., 0]
    return a + f * (b - a)


def clip_range(groups, kappa):
    """(lo, hi) clip limits of each group: Q(1 - kappa) and Q(kappa)."""
    # -0 and +0 are one value: a zero order statistic is taken as +0 (x + 0.0
    # maps -0 to +0 and leaves every other value unchanged)
    srt = np.sort(np.asarray(groups, dtype=np.float64), axis=-1) + 0.0
    kap = np.asarray(kappa, dtype=np.float32).astype(np.float64)
    hi = quantile_type7(srt, kap)
    lo = quantile_type7(srt, 1.0 - kap)
    return lo, hi


def quantize_rows(x, kappa, group):
    """Quantize rows of bf16-valued float64 ``x`` [..., D] in groups of ``group``.

    ``kappa`` broadcasts against x.shape[:-1] (one clip ratio per row).
    Returns (codes uint8 [..., D], s16 uint16 [..., D/G], z16 uint16 [..., D/G]).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % group == 0
    xg = x.reshape(x.shape[:-1] + (d // group, group))
    kap = np.broadcast_to(np.asarray(kappa, dtype=np.float32), x.shape[:-1])[..., None]
    lo, hi = clip_range(xg, kap)
    delta = (hi - lo) / 3.0
    s16 = f64_to_fp16_bits(delta)
    z16 = f64_to_fp16_bits(lo)
    codes = codes_from_params(xg, fp16_bits_to_f64(s16), fp16_bits_to_f64(z16))
    return codes.reshape(x.shape).astype(np.uint8), s16, z16


def codes_from_params(xg, s, z):
    """Codes of grouped values xg [..., ng, G] given fp16-valued s, z [..., ng]."""
    s = s[..., None]
    z = z[..., None]
    t1 = z + 0.5 * s
    t2 = z + 1.5 * s
    t3 = z + 2.5 * s
    c = (xg > t1).astype(np.int64) + (xg >= t2) + (xg > t3)
    c = np.where(s == 0.0, 0, c)
    return c


def dequant_rows(codes, s16, z16, group):
    """x_hat = s * code + z, exact in fp64 (returned as float64)."""
    codes = np.asarray(codes)
    d = codes.shape[-1]
    cg = codes.reshape(codes.shape[:-1] + (d // group, group)).astype(np.float64)
    s = fp16_bits_to_f64(s16)[..., None]
    z = fp16_bits_to_f64(z16)[..., None]
    return (s * cg + z).reshape(codes.shape)
