"""GPU parity of the plain BF16 paged decode (oscar_bf16_paged_decode_attn,
the uncompressed comparison kernel) against the oracle's plain attention.

The oracle sees the same bf16 keys, values and queries the cache holds,
widened to fp64, and computes softmax(q K^T / sqrt(128)) V per query head
(oracle.attention.attend).  Bar: max-abs <= 2e-3 and rel-L2 <= 1e-3.
"""

import numpy as np
import pytest

from oracle import attention
from oracle.rounding import bf16_bits_to_f64
from synth import get
from tests.oscar_testlib import compare_attention

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ultra_bit_kv_amd import lib
    lib()


def build(w, lens, holes=()):
    """A BF16 paged cache holding positions [0, L) of every row (keys and
    values straight from the workload, no rotation), its block table, and
    the list of (row, logical page) entries replaced by invalid ids."""
    from ultra_bit_kv_amd import BF16PagedCache
    need = [max(1, -(-int(L) // 16)) for L in lens]
    bt, total = w.page_pool(need)
    bt = bt.copy()
    for k, (i, m) in enumerate(holes):
        bt[i, m] = -1 if k % 2 == 0 else total + 5   # both kinds of invalid id
    cache = BF16PagedCache(num_q_heads=w.hq, num_kv_heads=w.hkv, max_seqs=len(lens),
                           max_pages_per_seq=bt.shape[1], num_pages=total, block_table=bt)
    for i, L in enumerate(lens):
        L = int(L)
        npg = need[i]
        for part, rows in ((0, w.keys(i, 0, L)), (1, w.values(i, 0, L))):
            buf = np.zeros((npg * 16, w.hkv, 128), np.uint16)
            buf[:L] = rows
            t = torch.from_numpy(buf.reshape(npg, 16, w.hkv, 128).transpose(0, 2, 1, 3).copy()
                                 .view(np.int16)).view(torch.bfloat16).cuda()
            ids = torch.from_numpy(np.asarray(bt[i, :npg], np.int64))
            ok = (ids >= 0) & (ids < total)
            cache.pages[ids[ok].cuda(), :, part] = t[ok.cuda()]
    return cache, bt


def queries(w, lens):
    return np.stack([w.queries(i, int(L) - 1, int(L))[0] for i, L in enumerate(lens)])


def run(w, lens, holes=()):
    from ultra_bit_kv_amd import SeqBatch, as_bf16
    cache, bt = build(w, lens, holes)
    q = queries(w, lens)
    out = cache.decode(SeqBatch(np.arange(len(lens)), lens), as_bf16(q))
    torch.cuda.synchronize()
    return out.cpu().numpy(), q, bt


def expected(w, i, L, q, holes=(), heads=None):
    """Oracle output [Hq, 128] (or the listed KV heads only) of row i."""
    g = w.hq // w.hkv
    keep = np.ones(L, bool)
    for (ii, m) in holes:
        if ii == i:
            keep[16 * m:16 * (m + 1)] = False
    k = bf16_bits_to_f64(w.keys(i, 0, L))[keep]
    v = bf16_bits_to_f64(w.values(i, 0, L))[keep]
    qf = bf16_bits_to_f64(q[i])
    out = {}
    for h in (range(w.hkv) if heads is None else heads):
        out[h] = attention.attend(qf[g * h:g * (h + 1)], k[:, h], v[:, h])
    return out


def check(name, w, lens, holes=(), rows=None, heads=None):
    got, q, _ = run(w, lens, holes)
    g = w.hq // w.hkv
    gs, ws = [], []
    for i in (range(len(lens)) if rows is None else rows):
        for h, want in expected(w, i, int(lens[i]), q, holes, heads).items():
            gs.append(got[i, g * h:g * (h + 1)])
            ws.append(want)
    err, rel, ok = compare_attention(np.stack(gs), np.stack(ws))
    print(f"[case] bf16 {name} max_abs={err:.3e} rel_l2={rel:.3e}", flush=True)
    assert ok, (name, err, rel)


def test_bf16_tiny():
    w = get("c1_tiny")
    check("c1", w, [1024])


def test_bf16_ragged_lengths():
    # one token, a partial page, a full page, one past it, an odd page count
    lens = [1, 15, 16, 17, 1000]
    w = get("c3_bs64").scaled(n_seqs=len(lens), lengths=("list", tuple(lens)))
    check("ragged", w, lens)


@pytest.mark.parametrize("hq, hkv, lens", [
    (2, 2, [33, 250]),          # g = 1: one head per pass, two KV heads per work-group
    (64, 2, [100, 517]),        # g = 32: two passes of 16 heads
    (12, 3, [70, 300, 2]),      # odd KV head count: one wave per work-group
    (40, 8, [260, 31]),         # g = 5: a partial pass of 8 heads
])
def test_bf16_head_shapes(hq, hkv, lens):
    w = get("c3_bs64").scaled(n_seqs=len(lens), hq=hq, hkv=hkv, lengths=("list", tuple(lens)))
    check(f"hq{hq}_hkv{hkv}", w, lens)


def test_bf16_invalid_block_table_entries_are_skipped():
    lens = [200, 90]
    w = get("c3_bs64").scaled(n_seqs=2, lengths=("list", tuple(lens)))
    check("holes", w, lens, holes=[(0, 3), (0, 7), (1, 0)])


def test_bf16_long_context_many_splits():
    # one row: the planner gives it far more than 32 splits (chunked merge)
    w = get("c2_qwen3_8b_bs1").scaled(lengths=("list", (20000,)))
    check("long20000", w, [20000])


def test_bf16_more_rows_than_one_launch():
    # 2100 rows: two launches of at most 2048 sequences
    rng = np.random.default_rng(7)
    lens = [int(x) for x in rng.integers(1, 40, 2100)]
    w = get("c1_tiny").scaled(n_seqs=len(lens), lengths=("list", tuple(lens)))
    check("rows2100", w, lens, rows=[0, 1, 2047, 2048, 2099])


def test_bf16_bs64_workload_sampled():
    # the bs64 workload at full size; four rows and two KV heads against the oracle
    w = get("c3_bs64")
    lens = [int(x) for x in w.lengths_after()]
    check("c3_full_sampled", w, lens, rows=[0, 17, 40, 63], heads=[0, 5])
