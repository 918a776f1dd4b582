"""O7 (the OScaR variant): Hadamard-rotated keys scaled to unit norm per token
(Omni-Token Scaling) and quantized per channel over blocks of G tokens.

Test infrastructure (see ``oracle/__init__.py``): what the variant computes,
against which the library's OScaR key mode is checked.

Sources:
* OScaR notes, background "KIVI and the per-channel paradigm": keys are
  quantized per channel in blocks of G tokens, values per token; for channel j
  and block g, Delta = (max - min) / (2^b - 1), z = -min / Delta,
  Q = clamp(round(K / Delta + z), 0, 2^b - 1), K^ = Delta (Q - z); the newest
  R = 128 tokens stay in a BF16 residual buffer that is quantized when full.
* OScaR notes, step one "Canalized Rotation" (k~ = H k, normalized H) and step
  two "Omni-Token Scaling": s_t = ||H k_t||_2, the quantized row is
  H k_t / s_t, s_t is stored beside the codes as one BF16 scalar per token,
  and k^ = s_t Delta_{j,g} (Q - z_{j,g}); the storage analysis puts a key
  token-head at 32 B of codes + 2 B of scale.
* OScaR notes, the algorithm listing (normalized keys enter the BF16
  residual buffer; a full buffer is quantized per channel) and the cache
  layout figure (codes, Delta and z in BF16, s per token in BF16).

Readings (the notes leave these open):
1. Rounding: k~ is the bf16 rounding of x . H / sqrt(d) (``rotate.Hadamard``);
   s16 = bf16(sqrt(S)) with S the sum of the squared bf16 entries rounded
   once to fp64 (exactly rounded, so independent of the summation order; the
   squares of bf16 values are exact in fp64, and whenever their bits span at
   most 53 positions S itself is exact) and sqrt the correctly rounded fp64
   square root; the buffered row is u16 = bf16(k~ / s16) from the correctly
   rounded fp64 quotient.  Blocks are quantized from u16.
2. Delta16 = bf16((max - min) / 3) and z16 = bf16(-min / Delta16) (for
   Delta16 = 0 see 4); codes come
   from the stored Delta16, z16: Q = clamp(rne(u / Delta16 + z16), 0, 3), taken
   exactly as [v > 1/2] + [v >= 3/2] + [v > 5/2] with v = u / Delta16 + z16.
3. Parameter count: one (Delta, z) per channel per block of G tokens; the
   layout figure's "(S/G) x (d/G)" is read as a garble of (S/G) x d.
4. A constant channel (max = min) has Delta16 = 0; it decodes to min, kept as
   z16 = bf16(min) with Delta16 = 0 (K^ = z16 when Delta16 = 0).
5. Dequantized key: k^ = s16 * Delta16 * (Q - z16) in fp64.
6. A zero extreme of a channel's block (min or max) is taken as +0: -0 and
   +0 are the same value, and the stored z of a block whose minimum is zero
   is then bf16(-0 / Delta) = -0 whichever zero the block held.
"""

import math

import numpy as np

from . import rotate
from .rounding import f64_to_bf16_bits, bf16_bits_to_f64


def ots_scale(k_rot_bits):
    """(s16, u16) bits for bf16 rotated key rows [N, d]: s16 = bf16(||k~||_2),
    u16 = bf16(k~ / s16)."""
    k = bf16_bits_to_f64(np.asarray(k_rot_bits, np.uint16))
    sq = np.array([math.fsum(row) for row in (k * k)], np.float64).reshape(k.shape[0])
    s16 = f64_to_bf16_bits(np.sqrt(sq))
    s = bf16_bits_to_f64(s16)
    with np.errstate(invalid="ignore", divide="ignore"):
        u = np.where(s[:, None] > 0, k / np.where(s > 0, s, 1.0)[:, None], 0.0)
    return s16, f64_to_bf16_bits(u)


def channel_quantize(u_bits):
    """Per-channel INT2 of one block of G tokens, u16 rows [G, d]:
    (codes uint8 [G, d], delta16 [d], z16 [d]) as bf16 bits."""
    u = bf16_bits_to_f64(np.asarray(u_bits, np.uint16))
    mn, mx = u.min(axis=0) + 0.0, u.max(axis=0) + 0.0   # a zero extreme is +0 (reading 6)
    d16 = f64_to_bf16_bits((mx - mn) / 3.0)
    dl = bf16_bits_to_f64(d16)
    const = dl == 0
    with np.errstate(invalid="ignore", divide="ignore"):
        z16 = np.where(const, f64_to_bf16_bits(mn), f64_to_bf16_bits(-mn / np.where(const, 1.0, dl)))
    z = bf16_bits_to_f64(z16)
    # v > t  <=>  u > Delta (t - z): Delta (8-bit) times t - z (exact in fp64)
    # is exact, so each threshold comparison is exact
    codes = np.zeros(u.shape, np.uint8)
    for t, strict in ((0.5, True), (1.5, False), (2.5, True)):
        thr = dl * (t - z)
        hit = u > thr if strict else u >= thr
        codes += np.where(const[None, :], False, hit).astype(np.uint8)
    return codes, d16, z16


def channel_dequant(codes, d16, z16):
    """Normalized rows u^ [G, d] of a block (before the per-token scale)."""
    dl = bf16_bits_to_f64(d16)
    z = bf16_bits_to_f64(z16)
    q = np.asarray(codes, np.float64)
    return np.where(dl[None, :] == 0, z[None, :], dl[None, :] * (q - z[None, :]))


def ots_keys(k_bits, group, bitrev=False):
    """Decoded keys [N, d] (rotated basis) of N post-RoPE bf16 key rows of one
    head, N a multiple of ``group``: rotate, scale, quantize each block of
    ``group`` consecutive tokens per channel, dequantize, rescale."""
    k_bits = np.asarray(k_bits, np.uint16)
    n = k_bits.shape[0]
    assert n % group == 0
    k_rot = rotate.hadamard_rotate_to_bf16(k_bits, bitrev)
    s16, u16 = ots_scale(k_rot)
    s = bf16_bits_to_f64(s16)
    out = np.empty(k_bits.shape, np.float64)
    for b in range(0, n, group):
        c, d16, z16 = channel_quantize(u16[b:b + group])
        out[b:b + group] = s[b:b + group, None] * channel_dequant(c, d16, z16)
    return out


def key_bytes_per_token_head(d=128, bits=2):
    """Bytes of one key token-head in the OTS layout besides the per-block
    parameters: packed codes plus the BF16 scale."""
    return d * bits // 8 + 2


# ---------------------------------------------------------------------------
# The OScaR variant as a whole cache (one sequence, one KV head).
#
# Placement, windows and values are those of the OSCAR cache (``cache.py``):
# the BF16 sink and recent windows hold the rotated rows, values are quantized
# per token over channel groups of G (O3, with the head's value clip ratio;
# OScaR's per-token value quantizer is its min-max case kappa = 1).  Keys of
# the INT2 segment take the OScaR path: Omni-Token Scaling, then per-channel
# INT2 over blocks of G consecutive INT2 tokens (the segment starts at S_sink
# and grows by S_flush, a multiple of G, so blocks never straddle a flush).
#
# Reading taken (beyond readings 1-5 above): the residual BF16 buffer holds the
# rotated key row itself; the per-token norm and the normalized row are taken
# when the row is quantized.  Normalizing on entry and storing s_t beside the
# buffered row would quantize the same bits (s16 and u16 are functions of the
# bf16 row); the BF16 window is then read back as the rotated row, not as
# s16 * u16.
# ---------------------------------------------------------------------------

D = 128
PAGE = 16


class OtsHeadCache:
    """OScaR cache of one sequence, one KV head, after ``length`` tokens.

    k_bits, v_bits: post-RoPE bf16 bits [length, D]; r_k, r_v: fp32 [D, D] or
    ``rotate.Hadamard``; kappa_v: the value clip ratio; group: G (key block
    length in tokens and value group width in channels).
    """

    def __init__(self, k_bits, v_bits, r_k, r_v, kappa_v, group, s_sink, s_keep, s_flush):
        from . import placement, quant
        assert s_flush % group == 0, "key blocks must not straddle a flush"
        self.length = k_bits.shape[0]
        self.group = group
        self.s_sink, self.s_keep, self.s_flush = s_sink, s_keep, s_flush
        self.k_rot = rotate.rotate_rows_to_bf16(k_bits, r_k)
        self.v_rot = rotate.rotate_rows_to_bf16(v_bits, r_v)
        self.sink, self.int2, self.recent = placement.segments(self.length, s_sink, s_keep, s_flush)
        a, b = self.int2
        nq = b - a
        assert nq % group == 0
        # keys: per-token scale and normalized rows, then one (Delta, z) per
        # channel per block of `group` tokens
        self.ks16, u16 = ots_scale(self.k_rot[a:b]) if nq else (np.zeros(0, np.uint16),
                                                                np.zeros((0, D), np.uint16))
        nb = nq // group
        self.kc = np.zeros((nq, D), np.uint8)
        self.kd16 = np.zeros((nb, D), np.uint16)
        self.kz16 = np.zeros((nb, D), np.uint16)
        for blk in range(nb):
            r = slice(blk * group, (blk + 1) * group)
            self.kc[r], self.kd16[blk], self.kz16[blk] = channel_quantize(u16[r])
        # values: per token, groups of `group` channels (O3)
        self.vc, self.vs, self.vz = quant.quantize_rows(bf16_bits_to_f64(self.v_rot[a:b]), kappa_v,
                                                        group)
        k_dec = bf16_bits_to_f64(self.k_rot)
        v_dec = bf16_bits_to_f64(self.v_rot)
        if nq:
            s = bf16_bits_to_f64(self.ks16)
            for blk in range(nb):
                r = slice(blk * group, (blk + 1) * group)
                k_dec[a + blk * group:a + (blk + 1) * group] = (
                    s[r, None] * channel_dequant(self.kc[r], self.kd16[blk], self.kz16[blk]))
            v_dec[a:b] = quant.dequant_rows(self.vc, self.vs, self.vz, group)
        self.k_dec, self.v_dec = k_dec, v_dec

    def dequant_f32(self):
        """Decoded rows as fp32 (one rounding of the fp64 values) [length, D]."""
        return self.k_dec.astype(np.float32), self.v_dec.astype(np.float32)

    def page_block(self, m):
        """Expected OTS page-head block of logical INT2 page m, and its valid slots."""
        from . import layout
        a, b = self.int2
        p0 = self.s_sink + PAGE * m
        n_valid = max(0, min(PAGE, b - p0))
        r = slice(p0 - a, p0 - a + n_valid)
        ng = D // self.group
        kc = np.zeros((PAGE, D), np.uint8)
        vc = np.zeros((PAGE, D), np.uint8)
        ks = np.zeros(PAGE, np.uint16)
        vs = np.zeros((PAGE, ng), np.uint16)
        vz = np.zeros_like(vs)
        kc[:n_valid], vc[:n_valid], ks[:n_valid] = self.kc[r], self.vc[r], self.ks16[r]
        vs[:n_valid], vz[:n_valid] = self.vs[r], self.vz[r]
        blk = (PAGE * m) // self.group                       # key block of this page
        half = ((PAGE * m) % self.group) // PAGE             # which channel half it stores
        ch = slice(64 * half, 64 * half + 64)
        return layout.pack_ots_page_head(kc, vc, ks, self.kd16[blk, ch], self.kz16[blk, ch], vs, vz,
                                         self.group), n_valid

    def window_rows(self):
        """{(block, slot): position} of every valid window slot."""
        from . import placement
        sb = -(-self.s_sink // PAGE)
        cap = placement.ring_capacity(self.s_keep, self.s_flush)
        out = {}
        for p in range(*self.sink):
            out[(p // PAGE, p % PAGE)] = p
        for p in range(*self.recent):
            r = (p - self.s_sink) % cap
            out[(sb + r // PAGE, r % PAGE)] = p
        return out
