"""Whole-sequence cache state: rotate, place, quantize, decode (O1-O4).

Test infrastructure (see ``oracle/__init__.py``).

The cache content is a function of the token stream alone: every quantized
row is the bf16 rotated row of its token, whether it reached INT2 through a
prefill chunk or through a flush of the recent window (OSCAR summary page,
section 4 "KV Cache Update": the same clip-quantize step is reused during
demotion).  So the state after ``length`` tokens is built directly from the
placement rule, without replaying appends.
"""

import numpy as np

from . import placement, quant, rotate, layout
from .rounding import bf16_bits_to_f64

D = 128
PAGE = 16


class HeadCache:
    """Cache of one sequence, one KV head, after ``length`` tokens.

    k_bits, v_bits: post-RoPE bf16 bits [length, D]; r_k, r_v: fp32 [D, D] or
    ``rotate.Hadamard``;
    kappa_k, kappa_v: fp32 clip ratios of this head.
    """

    def __init__(self, k_bits, v_bits, r_k, r_v, kappa_k, kappa_v, group,
                 s_sink, s_keep, s_flush):
        self.length = n = k_bits.shape[0]
        self.group = group
        self.s_sink, self.s_keep, self.s_flush = s_sink, s_keep, s_flush
        self.k_rot = rotate.rotate_rows_to_bf16(k_bits, r_k)
        self.v_rot = rotate.rotate_rows_to_bf16(v_bits, r_v)
        self.sink, self.int2, self.recent = placement.segments(n, s_sink, s_keep, s_flush)
        a, b = self.int2
        self.kc, self.ks, self.kz = quant.quantize_rows(bf16_bits_to_f64(self.k_rot[a:b]), kappa_k, group)
        self.vc, self.vs, self.vz = quant.quantize_rows(bf16_bits_to_f64(self.v_rot[a:b]), kappa_v, group)
        k_dec = bf16_bits_to_f64(self.k_rot)
        v_dec = bf16_bits_to_f64(self.v_rot)
        if b > a:
            k_dec[a:b] = quant.dequant_rows(self.kc, self.ks, self.kz, group)
            v_dec[a:b] = quant.dequant_rows(self.vc, self.vs, self.vz, group)
        self.k_dec, self.v_dec = k_dec, v_dec

    def dequant_f32(self):
        """What the dequant call returns for this head: fp32 rows [length, D]."""
        return self.k_dec.astype(np.float32), self.v_dec.astype(np.float32)

    def page_block(self, m):
        """Expected page-head block of logical INT2 page m, and the valid-slot mask."""
        a, b = self.int2
        p0 = self.s_sink + PAGE * m
        n_valid = max(0, min(PAGE, b - p0))
        kc = np.zeros((PAGE, D), np.uint8)
        vc = np.zeros((PAGE, D), np.uint8)
        ng = D // self.group
        ks = np.zeros((PAGE, ng), np.uint16)
        kz = np.zeros_like(ks)
        vs = np.zeros_like(ks)
        vz = np.zeros_like(ks)
        r = slice(p0 - a, p0 - a + n_valid)
        kc[:n_valid], vc[:n_valid] = self.kc[r], self.vc[r]
        ks[:n_valid], kz[:n_valid] = self.ks[r], self.kz[r]
        vs[:n_valid], vz[:n_valid] = self.vs[r], self.vz[r]
        blk = layout.pack_page_head(kc, vc, ks, kz, vs, vz, self.group)
        return blk, n_valid

    def window_rows(self):
        """{(block, slot): position} of every valid window slot."""
        sb = -(-self.s_sink // PAGE)
        cap = placement.ring_capacity(self.s_keep, self.s_flush)
        out = {}
        for p in range(*self.sink):
            out[(p // PAGE, p % PAGE)] = p
        for p in range(*self.recent):
            r = (p - self.s_sink) % cap
            out[(sb + r // PAGE, r % PAGE)] = p
        return out
