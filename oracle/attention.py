"""O5: decode attention over the decoded mixed BF16 / INT2 cache, fp64.

Test infrastructure (see ``oracle/__init__.py``).

Sources:
* OSCAR summary page, section 2 "Attention and KV cache": row-wise scores
  softmax(Q K^T / sqrt(d)); outputs are weighted sums of value rows.
* OSCAR summary page, section 4 "Decoding Attention Kernel": BF16 and INT2
  segments are unpacked and accumulated in floating point; existing decoders
  process sequence segments in separate launches and merge them.
* OScaR notes, "KV cache" background: Attention(q, K, V) = softmax(q K^T /
  sqrt(d_k)) V for the newest query against all cached rows.
* OSCAR summary page, section 4: the value rotation is undone on the output
  (or absorbed into W_O); here o = o' . R_V^T explicitly.

The decoded rows are whatever the cache holds: bf16 rows in the windows and
s * code + z in the INT2 middle, all in the rotated basis.  The just-appended
token is part of the context.  No mask, soft-cap or bias.
"""

import numpy as np

from . import rotate

D = 128


def attend(q, k, v):
    """Plain softmax(q k^T / sqrt(D)) v for q [g, D], k, v [T, D] (fp64)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    logits = q @ k.T / np.sqrt(D)
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    return (p @ v) / p.sum(axis=1, keepdims=True)


def partial(q, k, v):
    """Un-normalized partial state of one context slice: (m [g], l [g], o [g, D])."""
    q = np.asarray(q, dtype=np.float64)
    logits = q @ np.asarray(k, dtype=np.float64).T / np.sqrt(D)
    m = logits.max(axis=1)
    p = np.exp(logits - m[:, None])
    return m, p.sum(axis=1), p @ np.asarray(v, dtype=np.float64)


def merge(parts):
    """Log-sum-exp merge of partial states -> normalized output [g, D]."""
    ms = np.stack([p[0] for p in parts])          # [S, g]
    ls = np.stack([p[1] for p in parts])
    os_ = np.stack([p[2] for p in parts])         # [S, g, D]
    m = ms.max(axis=0)
    w = np.exp(ms - m[None, :])
    l = (w * ls).sum(axis=0)
    return (w[:, :, None] * os_).sum(axis=0) / l[:, None]


def attend_split(q, k, v, cuts):
    """Same result as ``attend`` computed over context slices cut at ``cuts``."""
    bounds = [0] + list(cuts) + [len(k)]
    parts = [partial(q, k[a:b], v[a:b]) for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
    return merge(parts)


def unrotate(o_rot, r_v):
    """o = o' . R_V^T (row vectors)."""
    return np.asarray(o_rot, dtype=np.float64) @ rotate.as_matrix(r_v).T


def decode_head(q_rot, k_dec, v_dec, r_v):
    """Output [g, D] (original basis) of the g query heads of one KV head."""
    return unrotate(attend(q_rot, k_dec, v_dec), r_v)
