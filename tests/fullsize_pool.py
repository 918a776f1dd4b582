"""Oracle expectations of whole caches, computed in worker processes.

Test infrastructure.  Each task regenerates one sequence's inputs from the
seeded workload (``synth``, NumPy only) and runs the fp64 oracle for some of
its KV heads: the expected INT2 page-head blocks (codes, fp16 scales and zero
points in the documented layout), the expected BF16 window rows, the rotated
query row and the decode output.  The workers import neither torch nor the
library and never touch the GPU; the main test process compares their
results with the cache the library built.
"""

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

D = 128
PAGE = 16

_ROT = {}


def _rotations(w, rotation):
    from oracle import rotate
    key = (w.name, w.index, w.hkv, rotation)
    if key not in _ROT:
        if rotation:
            had = rotate.Hadamard(D, bitrev=rotation == 2)
            _ROT[key] = ([had] * w.hkv, [had] * w.hkv)
        else:
            _ROT[key] = w.rotations()
    return _ROT[key]


def head_expectations(w, seq, L, heads, rotation=0, want_out=True):
    """Oracle view of sequence ``seq`` after L tokens, for the KV heads listed."""
    from oracle import attention, layout, placement, rotate
    from oracle.cache import HeadCache
    from oracle.rounding import bf16_bits_to_f64
    r_k, r_v = _rotations(w, rotation)
    kk, kv = w.kappas()
    k = w.keys(seq, 0, L)
    v = w.values(seq, 0, L)
    q_rot = rotate.rotate_heads_to_bf16(w.queries(seq, L - 1, L), r_k, g=w.g)[0]
    n_pages = placement.n_int2_pages(L, w.s_sink, w.s_keep, w.s_flush)
    ng = D // w.group
    out = []
    for h in heads:
        hc = HeadCache(k[:, h], v[:, h], r_k[h], r_v[h], kk[h], kv[h], w.group, w.s_sink,
                       w.s_keep, w.s_flush)
        a, b = hc.int2
        nq = b - a
        # codes and params of the INT2 positions, padded to whole pages
        pad = n_pages * PAGE
        def padded(x, shape):
            y = np.zeros((pad,) + shape, x.dtype)
            y[:nq] = x
            return y.reshape((n_pages, PAGE) + shape)
        pages = layout.pack_page_heads(
            padded(hc.kc, (D,)), padded(hc.vc, (D,)), padded(hc.ks, (ng,)), padded(hc.kz, (ng,)),
            padded(hc.vs, (ng,)), padded(hc.vz, (ng,)), w.group) if n_pages else None
        wr = hc.window_rows()
        keys = sorted(wr)
        pos = np.array([wr[x] for x in keys], np.int64)
        rec = {"h": h, "pages": pages, "n_int2": nq,
               "win_blk": np.array([x[0] for x in keys], np.int64),
               "win_t": np.array([x[1] for x in keys], np.int64),
               "win_k": hc.k_rot[pos] if len(pos) else np.zeros((0, D), np.uint16),
               "win_v": hc.v_rot[pos] if len(pos) else np.zeros((0, D), np.uint16)}
        if want_out:
            qr = bf16_bits_to_f64(q_rot[h * w.g:(h + 1) * w.g])
            rec["out"] = attention.decode_head(qr, hc.k_dec, hc.v_dec, r_v[h])
        out.append(rec)
    return {"seq": seq, "L": L, "q_rot": q_rot, "heads": out}


def _init_worker():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)          # one BLAS thread per worker process


def make_pool(max_workers=16):
    """Worker processes (spawned, one BLAS thread each), at most the box's
    CPU share."""
    n = max(1, min(max_workers, os.cpu_count() or 1))
    return ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"),
                               initializer=_init_worker)


def tasks_for(w, lens, seqs, rotation=0, want_out=True, split_len=16384):
    """(function, args) per task: one task per sequence, or one per (sequence,
    KV head) for sequences of at least ``split_len`` tokens."""
    out = []
    for i in seqs:
        L = int(lens[i])
        if L >= split_len:
            out += [(w, i, L, [h], rotation, want_out) for h in range(w.hkv)]
        else:
            out.append((w, i, L, list(range(w.hkv)), rotation, want_out))
    return out


_SLOTS = {}


def page_byte_slots(group):
    """Slot (0..15) of every byte of a page-head block, from the layout's own
    packer: a block with one slot's codes and parameters all ones."""
    from oracle import layout
    if group not in _SLOTS:
        ng = D // group
        pb = layout.page_head_bytes(group)
        slot = np.full(pb, -1, np.int64)
        for t in range(PAGE):
            c = np.zeros((PAGE, D), np.uint8)
            c[t] = 3
            p = np.zeros((PAGE, ng), np.uint16)
            p[t] = 0xFFFF
            blk = layout.pack_page_head(c, c, p, p, p, p, group)
            hit = blk != 0
            assert (slot[hit] == -1).all()
            slot[hit] = t
        assert (slot >= 0).all()
        _SLOTS[group] = slot
    return _SLOTS[group]
