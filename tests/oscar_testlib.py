"""Shared helpers for the GPU parity tests: build the library's cache and the
oracle's expectation from the same seeded workload inputs.

The oracle side only ever sees the synthetic inputs (never a GPU output)."""

import numpy as np

from oracle import placement, rotate, attention
from oracle.cache import HeadCache
from oracle.rounding import bf16_bits_to_f64

D = 128


def page_needs(w, lens):
    return [max(1, placement.n_int2_pages(int(L), w.s_sink, w.s_keep, w.s_flush)) for L in lens]


def make_cache(w, lens, identity=False, spare_pages=0, max_seqs=None, out_rotated=False,
               rotation=0, key_mode=0):
    """An empty OscarKVCache sized for sequences growing to ``lens``
    (``rotation`` 1 / 2: the structured R = H / sqrt(128) / H P_br / sqrt(128))."""
    from ultra_bit_kv_amd import OscarKVCache
    if rotation:
        had = [rotate.Hadamard(D, bitrev=rotation == 2)] * w.hkv
        r_k = r_v = None
    elif identity:
        eye = np.broadcast_to(np.eye(D, dtype=np.float32), (w.hkv, D, D)).copy()
        r_k = r_v = eye
    else:
        r_k, r_v = w.rotations()
    kk, kv = w.kappas()
    need = [n + spare_pages for n in page_needs(w, lens)]
    bt, total = w.page_pool(need)
    cache = OscarKVCache(num_q_heads=w.hq, num_kv_heads=w.hkv, group_size=w.group,
                         s_sink=w.s_sink, s_keep=w.s_keep, s_flush=w.s_flush,
                         max_seqs=max_seqs or len(lens), max_pages_per_seq=bt.shape[1],
                         num_pages=total, clip_k=kk, clip_v=kv, r_k=r_k, r_v=r_v,
                         block_table=bt, out_rotated=out_rotated, rotation=rotation,
                         key_mode=key_mode)
    cache.host_block_table = bt
    cache.host_r = (had, had) if rotation else (r_k, r_v)
    return cache


def fill(cache, w, lens, chunk=4096, seqs=None, max_tokens=1 << 18, last_step=True):
    """Append positions [0, L - 1) of every sequence in chunks of up to
    ``chunk`` tokens (at most ``max_tokens`` per call), then (``last_step``)
    the last token of each with its query (a decode step).  Returns the
    step's q_rot (None without the last step)."""
    import torch
    seqs = list(range(len(lens))) if seqs is None else seqs
    lens = [int(x) for x in lens]
    done = [0] * len(lens)
    while True:
        idx, n_new, budget = [], [], max_tokens
        for i in range(len(lens)):
            n = min(chunk, lens[i] - 1 - done[i], budget)
            if n > 0:
                idx.append(i)
                n_new.append(n)
                budget -= n
            if budget == 0:
                break
        if not idx:
            break
        k = np.concatenate([w.keys(seqs[i], done[i], done[i] + n) for i, n in zip(idx, n_new)])
        v = np.concatenate([w.values(seqs[i], done[i], done[i] + n) for i, n in zip(idx, n_new)])
        cache.append_tokens(idx, [done[i] for i in idx], n_new, k, v)
        for i, n in zip(idx, n_new):
            done[i] += n
    if not last_step:
        torch.cuda.synchronize()
        return None
    all_i = list(range(len(lens)))
    k = np.concatenate([w.keys(seqs[i], lens[i] - 1, lens[i]) for i in all_i])
    v = np.concatenate([w.values(seqs[i], lens[i] - 1, lens[i]) for i in all_i])
    q = np.concatenate([w.queries(seqs[i], lens[i] - 1, lens[i]) for i in all_i])
    q_rot, _, _ = cache.append_tokens(all_i, [L - 1 for L in lens], [1] * len(lens), k, v, q)
    torch.cuda.synchronize()
    return q_rot


def oracle_ots_head(w, seq, h, L, r_k, r_v):
    """The OScaR key mode's oracle cache of one (sequence, KV head)."""
    from oracle.ots import OtsHeadCache
    _, kv = w.kappas()
    return OtsHeadCache(w.keys(seq, 0, L)[:, h], w.values(seq, 0, L)[:, h], r_k[h], r_v[h], kv[h],
                        w.group, w.s_sink, w.s_keep, w.s_flush)


def oracle_head(w, seq, h, L, r_k, r_v):
    kk, kv = w.kappas()
    k = w.keys(seq, 0, L)[:, h]
    v = w.values(seq, 0, L)[:, h]
    return HeadCache(k, v, r_k[h], r_v[h], kk[h], kv[h], w.group, w.s_sink, w.s_keep, w.s_flush)


def oracle_q_rot(w, seq, L, r_k):
    q = w.queries(seq, L - 1, L)          # [1, Hq, D]
    return rotate.rotate_heads_to_bf16(q, r_k, g=w.g)[0]   # [Hq, D] bf16 bits


def oracle_decode(w, seq, h, L, r_k, r_v, hc=None):
    """fp64 output [g, D] of the g query heads of KV head h (original basis)."""
    hc = hc or oracle_head(w, seq, h, L, r_k, r_v)
    qr = bf16_bits_to_f64(oracle_q_rot(w, seq, L, r_k)[h * w.g:(h + 1) * w.g])
    return attention.decode_head(qr, hc.k_dec, hc.v_dec, r_v[h])


def compare_attention(got, want, tol_abs=2e-3, tol_rel=1e-3):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want).max()
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
    return err, rel, (err <= tol_abs and rel <= tol_rel)
