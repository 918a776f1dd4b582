"""Parity at the workloads' full sizes, through the C ABI, in the launch
configuration the benchmark times.  Whole caches are built on the GPU and
decoded; for EVERY (sequence, KV head) of the bs1 32K / 128K, bs64 and
serving-step workloads:

* every INT2 page-head block (codes, fp16 scales, fp16 zero points) and every
  BF16 window row is compared bit for bit with the fp64 oracle's cache,
* the rotated query row is compared bit for bit,
* the decode output is compared with the oracle's (max-abs 2e-3, rel-L2 1e-3),

and the dequantized rows of sampled sequences bit for bit.  The oracle runs in
worker processes (``tests/fullsize_pool.py``) while the GPU builds the cache."""
from concurrent.futures import as_completed

import numpy as np
import pytest
import torch

from oracle.layout import v_window_index
from synth import get
from tests import fullsize_pool
from tests.oscar_testlib import compare_attention, fill, make_cache, oracle_head

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module")
def pool():
    ex = fullsize_pool.make_pool()
    yield ex
    ex.shutdown()


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _submit(pool, w, lens, seqs, rotation, want_out=True):
    return [pool.submit(fullsize_pool.head_expectations, *t)
            for t in fullsize_pool.tasks_for(w, lens, seqs, rotation, want_out)]


def _host_views(cache):
    c = cache.cfg
    pb = cache.page_head_bytes
    pages = cache.pages.cpu().numpy()[:c.num_pages * c.num_kv_heads * pb]
    pages = pages.reshape(c.num_pages, c.num_kv_heads, pb)
    nb = -(-c.s_sink // 16) + cache.ring_capacity // 16
    win = cache.win.cpu().numpy().view(np.uint16).reshape(c.max_seqs, c.num_kv_heads, nb, 2 * 16 * D)
    return pages, win


def _verify(w, cache, futures, q_rot, out, label):
    """Compare the cache (and decode outputs where the oracle computed them)
    with the oracle's, sequence by sequence as the workers finish."""
    pages, win = _host_views(cache)
    bt = cache.host_block_table
    slot_of = fullsize_pool.page_byte_slots(w.group)
    qr = q_rot.contiguous().view(torch.int16).cpu().numpy().view(np.uint16) if q_rot is not None else None
    ch = np.arange(D)[None, :]
    n_heads = n_pages_seen = n_rows = 0
    worst = (0.0, 0.0)
    for f in as_completed(futures):
        r = f.result()
        i = r["seq"]
        for hr in r["heads"]:
            h = hr["h"]
            exp = hr["pages"]
            if exp is not None:
                npg = exp.shape[0]
                got = pages[bt[i, :npg], h]
                n_last = hr["n_int2"] - 16 * (npg - 1)
                if n_last == 16:
                    same = np.array_equal(got, exp)
                else:
                    keep = slot_of < n_last
                    same = (np.array_equal(got[:-1], exp[:-1]) and
                            np.array_equal(got[-1][keep], exp[-1][keep]))
                if not same:
                    bad = [m for m in range(npg) if not np.array_equal(got[m], exp[m])]
                    raise AssertionError(f"{label}: seq {i} head {h}: INT2 page-heads differ at "
                                         f"logical pages {bad[:8]} of {npg}")
                n_pages_seen += npg
            blk, t = hr["win_blk"], hr["win_t"]
            if len(blk):
                wb = win[i, h]
                gk = wb[blk[:, None], D * t[:, None] + ch]
                gv = wb[blk[:, None], 16 * D + v_window_index(t[:, None], ch)]
                assert np.array_equal(gk, hr["win_k"]), (label, i, h, "window K rows")
                assert np.array_equal(gv, hr["win_v"]), (label, i, h, "window V rows")
                n_rows += len(blk)
            if "out" in hr:
                assert np.array_equal(qr[i, h * w.g:(h + 1) * w.g],
                                      r["q_rot"][h * w.g:(h + 1) * w.g]), (label, i, h, "q_rot")
                err, rel, ok = compare_attention(out[i, h * w.g:(h + 1) * w.g], hr["out"])
                worst = (max(worst[0], err), max(worst[1], rel))
                assert ok, (label, i, h, err, rel)
            n_heads += 1
    _case(f"{label}: {n_heads} (sequence, KV head) pairs, {n_pages_seen} INT2 page-heads and "
          f"{n_rows} window rows bit-exact; decode max_abs={worst[0]:.3e} rel_l2={worst[1]:.3e}")
    return n_heads


def _check_dequant(w, cache, i, L, heads):
    """Dequantized rows of one sequence, bit for bit (in-process oracle)."""
    r_k, r_v = cache.host_r
    kd, vd = cache.dequant(i, L, 0, L)
    kd, vd = kd.cpu().numpy(), vd.cpu().numpy()
    for h in heads:
        ek, ev = oracle_head(w, i, h, L, r_k, r_v).dequant_f32()
        assert np.array_equal(kd[:, h].view(np.uint32), ek.view(np.uint32)), (w.name, i, h)
        assert np.array_equal(vd[:, h].view(np.uint32), ev.view(np.uint32)), (w.name, i, h)
    _case(f"{w.name}: dequantized rows of sequence {i} ({L} tokens, heads {list(heads)}) bit-exact")


@pytest.mark.parametrize("name,rotation", [
    ("c2_qwen3_8b_bs1", 0),
    ("c2_qwen3_8b_bs1", 1),        # structured H / sqrt(128): two-level merge un-rotation
    ("c4_long_bs1", 0),
])
def test_fullsize_long_context(pool, name, rotation):
    from ultra_bit_kv_amd import SeqBatch
    w = get(name)
    lens = [int(x) for x in w.lengths_after()]
    _case(f"{name} full size, lens {lens}, rotation {rotation}: all {w.hkv} KV heads")
    futures = _submit(pool, w, lens, [0], rotation)
    cache = make_cache(w, lens, rotation=rotation)
    q_rot = fill(cache, w, lens, chunk=8192)
    out = cache.decode(SeqBatch(range(len(lens)), lens), q_rot).cpu().numpy()
    assert _verify(w, cache, futures, q_rot, out, f"{name} rot {rotation}") == w.hkv
    if name == "c2_qwen3_8b_bs1" and rotation == 0:
        _check_dequant(w, cache, 0, lens[0], [0, 7])


@pytest.mark.parametrize("rotation", [0, 2])
def test_fullsize_bs64(pool, rotation):
    """The benchmark's workload and launch plan: 64 sequences, U[4096, 8192];
    with the dense per-head rotation and the structured H P_br / sqrt(128)."""
    from ultra_bit_kv_amd import SeqBatch
    w = get("c3_bs64")
    lens = [int(x) for x in w.lengths_after()]
    _case(f"c3_bs64 full size, {len(lens)} sequences, rotation {rotation}: every sequence and head")
    futures = _submit(pool, w, lens, range(len(lens)), rotation)
    cache = make_cache(w, lens, max_seqs=len(lens), rotation=rotation)
    q_rot = fill(cache, w, lens, chunk=8192)
    out = cache.decode(SeqBatch(range(len(lens)), lens), q_rot).cpu().numpy()
    assert _verify(w, cache, futures, q_rot, out, f"c3 rot {rotation}") == len(lens) * w.hkv
    if rotation == 0:
        _check_dequant(w, cache, int(np.argmax(lens)), max(lens), range(w.hkv))


def test_fullsize_serving_step(pool):
    """The Qwen3-32B-shaped serving step: one append call carrying 256 decode
    tokens (8 of them trigger a 256-token flush) and 16 fresh 2048-token
    prefill chunks, then the decode of the 256 sequences.  Every decode
    sequence's cache and output and every prefilled sequence's cache."""
    from ultra_bit_kv_amd import SeqBatch
    w = get("c5_qwen3_32b_step")
    lens = [int(x) for x in w.lengths_after()]                # after the step
    n_dec, n_pre, plen = len(lens), w.prefill_chunks, w.prefill_len
    _case(f"c5 full size: {n_dec} decode sequences + {n_pre} x {plen} prefill, every head")
    all_lens = lens + [plen] * n_pre
    futures = (_submit(pool, w, all_lens, range(n_dec), 0) +
               _submit(pool, w, all_lens, range(n_dec, n_dec + n_pre), 0, want_out=False))
    cache = make_cache(w, all_lens, max_seqs=n_dec + n_pre)
    fill(cache, w, lens, chunk=4096, last_step=False)          # positions [0, L - 1)
    # the step: decode tokens of sequences 0..255, prefill of sequences 256..271
    slots = list(range(n_dec + n_pre))
    before = [L - 1 for L in lens] + [0] * n_pre
    n_new = [1] * n_dec + [plen] * n_pre
    k = np.concatenate([w.keys(i, b, b + n) for i, b, n in zip(slots, before, n_new)])
    v = np.concatenate([w.values(i, b, b + n) for i, b, n in zip(slots, before, n_new)])
    q = np.concatenate([w.queries(i, b, b + n) for i, b, n in zip(slots, before, n_new)])
    q_rot, _, _ = cache.append_tokens(slots, before, n_new, k, v, q)
    torch.cuda.synchronize()
    flushing = [i for i, L in enumerate(lens) if L == w.lengths[3]]
    assert len(flushing) == 8
    out = cache.decode(SeqBatch(range(n_dec), lens), q_rot[:n_dec].contiguous()).cpu().numpy()
    assert _verify(w, cache, futures, q_rot[:n_dec], out, "c5 step") == (n_dec + n_pre) * w.hkv
    _check_dequant(w, cache, n_dec + 7, plen, [2])
    _check_dequant(w, cache, flushing[0], lens[flushing[0]], [1])
