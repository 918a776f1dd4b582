"""O6: chunked-prefill attention of a new chunk over the mixed cache, fp64.

Test infrastructure (see ``oracle/__init__.py``).

Sources:
* WUSH-KV notes, "method step details", inference (Algorithm 2): the key
  transform is applied to every new key and query of a chunk, the chunk's
  rows join the cache at full precision, grouped-query attention runs over
  the mixed-precision cache, and the S_flush-aligned segments beyond the
  S_sink / S_keep windows are quantized.
* OSCAR summary page, section 4 "KV Cache Update": during prefill the fused
  kernel clips, quantizes and packs the rows written to the cache;
  "KV Cache Layout": BF16 sink, INT2 middle, BF16 recent window.
* OSCAR summary page, section 2 "Attention and KV cache": softmax(Q K^T /
  sqrt(d)) row by row, outputs are weighted sums of value rows.

Reading taken (the pages do not fix the order of the chunk's own flush and
its attention for an API that appends first): the call follows the chunk's
append, as a decode step follows its token's append.  The query at chunk
position p attends to positions 0 .. p (causal):
* positions below len_before as the cache holds them after the append
  (bf16 window rows, INT2 rows as scale * code + zero; the append's flush may
  already have moved some previously recent rows to INT2);
* the chunk's own rows len_before .. p at their bf16 rotated values, whether
  or not the append quantized them (Algorithm 2 attends to the new rows at
  full precision).
"""

import numpy as np

from . import attention
from .rounding import bf16_bits_to_f64


def context_rows(hc, len_before, p):
    """Key and value rows [p + 1, D] (rotated basis) seen by the query at
    position p of a chunk that starts at ``len_before``; ``hc`` is the
    ``cache.HeadCache`` of the row after the chunk's append."""
    assert 0 <= len_before <= p < hc.length
    k = np.concatenate([hc.k_dec[:len_before], bf16_bits_to_f64(hc.k_rot[len_before:p + 1])])
    v = np.concatenate([hc.v_dec[:len_before], bf16_bits_to_f64(hc.v_rot[len_before:p + 1])])
    return k, v


def prefill_head(q_rot, hc, len_before, r_v=None, rows=None):
    """Outputs of the chunk queries of one KV head.

    q_rot: fp64 [n_new, g, D], the rotated queries of chunk positions
    len_before .. len_before + n_new - 1; hc: the head's cache after the
    append (its length is len_before + n_new).  Returns [n_new, g, D] in the
    original basis (o' . R_V^T), or in the rotated basis when r_v is None.
    ``rows`` restricts the work to the listed chunk indices (the others stay
    NaN)."""
    q_rot = np.asarray(q_rot, dtype=np.float64)
    n_new = q_rot.shape[0]
    assert hc.length == len_before + n_new
    out = np.full(q_rot.shape, np.nan)
    for j in (range(n_new) if rows is None else rows):
        k, v = context_rows(hc, len_before, len_before + j)
        o = attention.attend(q_rot[j], k, v)
        out[j] = o if r_v is None else attention.unrotate(o, r_v)
    return out
