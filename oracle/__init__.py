"""Plain, slow CPU oracle for the OSCAR-style INT2 KV-cache hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the ``ultra_bit_kv_amd``
package, its C ABI library or its kernels) may import, call or link anything in
this package.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.

Everything here is written from the three source pages:

* "OSCAR: Offline Spectral Covariance-Aware Rotation for 2-bit KV Cache
  Quantization" (paperlayer.ai summary) -- the subject: fixed per-head rotation,
  clipped asymmetric INT2, BF16 sink/recent windows, mixed BF16/INT2 decode.
* "OScaR reading notes" (zhongzhuzhou.org blog) -- the uniform quantizer and
  dequantizer formulas, the worked example, orthogonality preserving q.k.
* "WUSH-KV notes" (paper.rainbus.top) -- the S_sink / S_keep / S_flush / S_quant
  flush rule and the kappa-quantile clipped affine quantizer.

Arithmetic is fp64 unless a step names a rounding.  Modules:

* ``rounding``  -- fp64 -> bf16 / fp16 single round-to-nearest-even.
* ``rotate``    -- O1: x' = x . R, rounded once to bf16 (with an exactness guard),
  for a dense R or the structured R = H (P_br) / sqrt(d).
* ``placement`` -- O2: S_quant closed form, segments, ring slots, pages.
* ``quant``     -- O3/O4: kappa-quantile clip, scale/zero, codes, dequant.
* ``layout``    -- the documented on-HBM packing of pages and window blocks.
* ``attention`` -- O5: decode attention over the decoded cache, split + merge.
* ``cache``     -- builds the whole decoded cache state of a sequence.
* ``prefill``   -- O6: causal attention of a new chunk over the mixed cache.
* ``ots``       -- O7: the OScaR variant (per-token key scale, per-channel INT2
  keys over blocks of G tokens); not yet on the GPU path.
"""

from . import rounding, rotate, placement, quant, layout, attention, cache, prefill, ots  # noqa: F401
