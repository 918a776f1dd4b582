"""GPU parity: liboscar_kv (through the C ABI) against the CPU oracle.

Bars (fixed by the method's contract):
* rotated rows (q_rot, window rows), INT2 codes, fp16 scales / zero points and
  dequantized rows: bit-exact;
* decode attention: max-abs <= 2e-3 and rel-L2 <= 1e-3 (fp32 accumulation).
"""

import numpy as np
import pytest

from oracle import layout, placement
from oracle.rounding import bf16_bits_to_f64
from synth import get
from tests.oscar_testlib import (make_cache, fill, oracle_head, oracle_q_rot, oracle_decode,
                                 compare_attention)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ultra_bit_kv_amd import lib
    lib()


def small(name):
    """Reduced-size variants of the five workloads (ragged, several tiles)."""
    if name == "c1":
        return get("c1_tiny"), [1024]
    if name == "c2s":
        return get("c2_qwen3_8b_bs1").scaled(lengths=("list", (1500,))), [1500]
    if name == "c3s":
        w = get("c3_bs64").scaled(n_seqs=3, lengths=("list", (333, 517, 1000)))
        return w, [333, 517, 1000]
    if name == "c4s":
        return get("c4_long_bs1").scaled(lengths=("list", (1400,))), [1400]
    if name == "c5s":
        w = get("c5_qwen3_32b_step").scaled(n_seqs=2, lengths=("list", (700, 1000)))
        return w, [700, 1000]
    if name == "demote1":   # OSCAR's one-token demotion, no sink
        w = get("c1_tiny").scaled(s_sink=0, s_keep=5, s_flush=1, group=64)
        return w, [300]
    if name == "oddflush":  # flush not page aligned, odd sink
        w = get("c3_bs64").scaled(n_seqs=2, hkv=2, hq=8, s_sink=5, s_keep=40, s_flush=24,
                                   group=32, lengths=("list", (250, 401)))
        return w, [250, 401]
    if name == "bigv":      # value rows of magnitude ~1e3: fp16 value scales above 128
        w = get("c3_bs64").scaled(n_seqs=2, v_scale=1000.0, lengths=("list", (700, 1100)))
        return w, [700, 1100]
    raise KeyError(name)


CASES = ["c1", "c2s", "c3s", "c4s", "c5s", "demote1", "oddflush", "bigv"]


def _check_head(cache, w, i, h, L, hc):
    """Bit-exact comparison of one (sequence, KV head) of the cache."""
    ng = 128 // w.group
    bt = cache.host_block_table
    a, b = hc.int2
    for m in range(placement.n_int2_pages(L, w.s_sink, w.s_keep, w.s_flush)):
        blk = cache.page_head(int(bt[i, m]), h)
        kc, vc, ks, kz, vs, vz = layout.unpack_page_head(blk, w.group)
        _, nv = hc.page_block(m)
        r = slice(16 * m, 16 * m + nv)
        assert np.array_equal(kc[:nv], hc.kc[r]), (i, h, m)
        assert np.array_equal(vc[:nv], hc.vc[r]), (i, h, m)
        assert np.array_equal(ks[:nv], hc.ks[r]) and np.array_equal(kz[:nv], hc.kz[r]), (i, h, m)
        assert np.array_equal(vs[:nv], hc.vs[r]) and np.array_equal(vz[:nv], hc.vz[r]), (i, h, m)
        assert ks.shape[1] == ng
    wb = cache.window_blocks(i, h)
    for (blk, t), p in hc.window_rows().items():
        k_rows, v_rows = layout.unpack_window_block(wb[blk])
        assert np.array_equal(k_rows[t], hc.k_rot[p]), (i, h, p)
        assert np.array_equal(v_rows[t], hc.v_rot[p]), (i, h, p)
    kd, vd = cache.dequant(i, L, 0, L)
    kd = kd[:, h].cpu().numpy()
    vd = vd[:, h].cpu().numpy()
    ek, ev = hc.dequant_f32()
    assert np.array_equal(kd.view(np.uint32), ek.view(np.uint32)), (i, h)
    assert np.array_equal(vd.view(np.uint32), ev.view(np.uint32)), (i, h)


@pytest.mark.parametrize("identity", [True, False])
@pytest.mark.parametrize("name", CASES)
def test_append_bit_exact_and_decode(name, identity):
    w, lens = small(name)
    print(f"[case] {name} identity={identity} lens={lens}", flush=True)
    cache = make_cache(w, lens, identity=identity)
    q_rot = fill(cache, w, lens, chunk=300)
    r_k, r_v = cache.host_r
    out = cache.decode(__import__("ultra_bit_kv_amd").SeqBatch(range(len(lens)), lens), q_rot)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    qr = q_rot.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    worst = (0.0, 0.0)
    for i, L in enumerate(lens):
        assert np.array_equal(qr[i], oracle_q_rot(w, i, L, r_k)), i
        for h in range(w.hkv):
            hc = oracle_head(w, i, h, L, r_k, r_v)
            _check_head(cache, w, i, h, L, hc)
            want = oracle_decode(w, i, h, L, r_k, r_v, hc)
            # the error budget is relative to the values' magnitude (fp32
            # accumulation, P' as fp16 hi + lo): the absolute bar scales with it
            err, rel, ok = compare_attention(out[i, h * w.g:(h + 1) * w.g], want,
                                             tol_abs=2e-3 * w.v_scale)
            worst = (max(worst[0], err), max(worst[1], rel))
            assert ok, (name, i, h, err, rel)
    print(f"[case] {name} max_abs={worst[0]:.3e} rel_l2={worst[1]:.3e}", flush=True)


def test_path_independence():
    """Chunked prefill and token-by-token appends give the same cache bytes."""
    from ultra_bit_kv_amd import SeqBatch
    w = get("c3_bs64").scaled(n_seqs=2, hkv=2, hq=8, lengths=("list", (420, 610)))
    lens = [420, 610]
    c1 = make_cache(w, lens)
    q1 = fill(c1, w, lens, chunk=4096)
    c2 = make_cache(w, lens)
    # first 300 tokens in odd chunks, the rest one token at a time
    done = [0, 0]
    sizes = [37, 1, 150, 112]
    for n in sizes:
        k = np.concatenate([w.keys(i, done[i], done[i] + n) for i in range(2)])
        v = np.concatenate([w.values(i, done[i], done[i] + n) for i in range(2)])
        c2.append_tokens([0, 1], done, [n, n], k, v)
        done = [d + n for d in done]
    while any(d < L - 1 for d, L in zip(done, lens)):
        idx = [i for i in range(2) if done[i] < lens[i] - 1]
        k = np.concatenate([w.keys(i, done[i], done[i] + 1) for i in idx])
        v = np.concatenate([w.values(i, done[i], done[i] + 1) for i in idx])
        c2.append_tokens(idx, [done[i] for i in idx], [1] * len(idx), k, v)
        for i in idx:
            done[i] += 1
    k = np.concatenate([w.keys(i, lens[i] - 1, lens[i]) for i in range(2)])
    v = np.concatenate([w.values(i, lens[i] - 1, lens[i]) for i in range(2)])
    q = np.concatenate([w.queries(i, lens[i] - 1, lens[i]) for i in range(2)])
    q2, _, _ = c2.append_tokens([0, 1], [L - 1 for L in lens], [1, 1], k, v, q)
    for i, L in enumerate(lens):
        kd1, vd1 = c1.dequant(i, L, 0, L)
        kd2, vd2 = c2.dequant(i, L, 0, L)
        assert torch.equal(kd1, kd2) and torch.equal(vd1, vd2)
    b = SeqBatch([0, 1], lens)
    assert torch.equal(c1.decode(b, q1), c2.decode(b, q2))


def test_decode_deterministic_and_edge_lengths():
    """Repeated calls are bitwise equal; short contexts (sink only, ring only,
    first flush) match the oracle."""
    from ultra_bit_kv_amd import SeqBatch
    w = get("c3_bs64").scaled(n_seqs=9, hkv=2, hq=8)
    lens = [1, 2, 63, 64, 65, 319, 320, 336, 337]
    w = w.scaled(lengths=("list", tuple(lens)))
    cache = make_cache(w, lens)
    q_rot = fill(cache, w, lens, chunk=64)
    b = SeqBatch(range(len(lens)), lens)
    o1 = cache.decode(b, q_rot)
    o2 = cache.decode(b, q_rot)
    assert torch.equal(o1, o2)
    # the two-call form (split launch, then merge launch) computes the same bits
    cache.decode_partials(b, q_rot)
    assert torch.equal(cache.decode_merge(b), o1)
    out = o1.cpu().numpy()
    r_k, r_v = cache.host_r
    for i, L in enumerate(lens):
        for h in range(w.hkv):
            want = oracle_decode(w, i, h, L, r_k, r_v)
            err, rel, ok = compare_attention(out[i, h * w.g:(h + 1) * w.g], want)
            assert ok, (L, h, err, rel)


def test_decode_many_splits_long_context():
    """Thousands of INT2 pages, many splits, G = 32 (4 groups per row)."""
    from ultra_bit_kv_amd import SeqBatch
    w = get("c4_long_bs1").scaled(hkv=2, hq=8, lengths=("list", (20000,)))
    lens = [20000]
    cache = make_cache(w, lens)
    q_rot = fill(cache, w, lens, chunk=8192)
    out = cache.decode(SeqBatch([0], lens), q_rot).cpu().numpy()
    r_k, r_v = cache.host_r
    for h in range(w.hkv):
        want = oracle_decode(w, 0, h, 20000, r_k, r_v)
        err, rel, ok = compare_attention(out[0, h * w.g:(h + 1) * w.g], want)
        assert ok, (h, err, rel)


@pytest.mark.parametrize("hq, hkv, group, length", [
    (48, 4, 128, 12000),   # g = 12 in a 16-head pass: the merge's work-groups for heads 12..15 stay idle
    (24, 6, 64, 9000),     # g = 4, two groups, three two-head waves
])
def test_decode_many_splits_head_layouts(hq, hkv, group, length):
    """Rows with more than 32 splits (the one-launch wide merge) for head
    layouts whose last query-head pass is partly empty, against the oracle."""
    from ultra_bit_kv_amd import SeqBatch
    w = get("c3_bs64").scaled(n_seqs=1, hq=hq, hkv=hkv, group=group, lengths=("list", (length,)))
    lens = [length]
    cache = make_cache(w, lens)
    q_rot = fill(cache, w, lens, chunk=4096)
    out = cache.decode(SeqBatch([0], lens), q_rot).cpu().numpy()
    r_k, r_v = cache.host_r
    worst = 0.0
    for h in range(w.hkv):
        want = oracle_decode(w, 0, h, length, r_k, r_v)
        err, rel, ok = compare_attention(out[0, h * w.g:(h + 1) * w.g], want)
        worst = max(worst, err)
        assert ok, (hq, hkv, group, h, err, rel)
    print(f"[case] many splits hq{hq} hkv{hkv} G{group} L{length} max_abs={worst:.3e}", flush=True)


@pytest.mark.parametrize("hq, hkv, group, lens", [
    (2, 2, 128, (300, 517)),     # one query head per KV head: two KV heads per wave, 1 head per pass
    (4, 2, 128, (400, 90)),      # g = 2, one group
    (4, 2, 32, (333, 700)),      # g = 2, four groups: two KV heads per wave, 2 heads per pass
    (8, 2, 64, (260, 500)),      # g = 4, two groups: two KV heads per wave
    (24, 6, 64, (350, 450)),     # six KV heads: three two-head waves, one work-group per row
    (12, 3, 64, (300, 401)),     # odd KV head count: one KV head per wave
    (48, 4, 128, (300, 340)),    # g = 12: one group, 16 heads per pass, one KV head per wave
])
def test_decode_head_layouts(hq, hkv, group, lens):
    """Every (groups, heads per pass, KV heads per wave) layout of the split
    kernel's MFMA columns against the oracle."""
    from ultra_bit_kv_amd import SeqBatch
    lens = list(lens)
    w = get("c3_bs64").scaled(n_seqs=len(lens), hq=hq, hkv=hkv, group=group,
                              lengths=("list", tuple(lens)))
    cache = make_cache(w, lens)
    q_rot = fill(cache, w, lens, chunk=256)
    out = cache.decode(SeqBatch(range(len(lens)), lens), q_rot).cpu().numpy()
    r_k, r_v = cache.host_r
    worst = 0.0
    for i, L in enumerate(lens):
        for h in range(w.hkv):
            want = oracle_decode(w, i, h, L, r_k, r_v)
            err, rel, ok = compare_attention(out[i, h * w.g:(h + 1) * w.g], want)
            worst = max(worst, err)
            assert ok, (hq, hkv, group, L, h, err, rel)
    print(f"[case] layout hq{hq} hkv{hkv} G{group} max_abs={worst:.3e}", flush=True)


@pytest.mark.parametrize("out_rotated", [False, True])
def test_query_transform_and_absorbed_output(out_rotated):
    """A non-orthogonal key transform T with the query transform T^-T (scores
    unchanged), and the absorbed-R_V output (rotated basis): q' bit-exact,
    cache rows bit-exact, attention against the oracle."""
    from ultra_bit_kv_amd import OscarKVCache, SeqBatch
    from oracle import rotate as orot, attention as oatt
    from tests.oscar_testlib import page_needs
    w = get("c3_bs64").scaled(n_seqs=2, hkv=2, hq=8, lengths=("list", (300, 517)))
    lens = [300, 517]
    rng = np.random.default_rng(31)
    rk0, r_v = w.rotations()
    scale = rng.uniform(0.7, 1.4, (w.hkv, 1, 128)).astype(np.float32)
    t = (rk0 * scale).astype(np.float32)                          # k' = k . T
    r_q = np.stack([np.linalg.inv(t[h].astype(np.float64)).T for h in range(w.hkv)]).astype(np.float32)
    kk, kv = w.kappas()
    bt, total = w.page_pool(page_needs(w, lens))
    cache = OscarKVCache(num_q_heads=w.hq, num_kv_heads=w.hkv, group_size=w.group,
                         s_sink=w.s_sink, s_keep=w.s_keep, s_flush=w.s_flush, max_seqs=2,
                         max_pages_per_seq=bt.shape[1], num_pages=total, clip_k=kk, clip_v=kv,
                         r_k=t, r_v=r_v, block_table=bt, r_q=r_q, out_rotated=out_rotated)
    cache.host_block_table = bt
    cache.host_r = (t, r_v)
    q_rot = fill(cache, w, lens, chunk=128)
    out = cache.decode(SeqBatch([0, 1], lens), q_rot).cpu().numpy()
    qr = q_rot.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    worst = 0.0
    for i, L in enumerate(lens):
        want_q = orot.rotate_heads_to_bf16(w.queries(i, L - 1, L), r_q, g=w.g)[0]
        assert np.array_equal(qr[i], want_q), i
        for h in range(w.hkv):
            hc = oracle_head(w, i, h, L, t, r_v)
            _check_head(cache, w, i, h, L, hc)
            q64 = bf16_bits_to_f64(want_q[h * w.g:(h + 1) * w.g])
            if out_rotated:
                want = oatt.attend(q64, hc.k_dec, hc.v_dec)
            else:
                want = oatt.decode_head(q64, hc.k_dec, hc.v_dec, r_v[h])
            err, rel, ok = compare_attention(out[i, h * w.g:(h + 1) * w.g], want)
            worst = max(worst, err)
            assert ok, (out_rotated, i, h, err, rel)
    print(f"[case] query transform out_rotated={out_rotated} max_abs={worst:.3e}", flush=True)


def test_large_grid_device_item_lookup():
    """A launch with more work-groups than the host item table holds (one
    KV head: one-wave work-groups, 200 sequences): the work-groups find their
    items from the device lengths.  Sampled sequences against the oracle."""
    from ultra_bit_kv_amd import SeqBatch
    rng = np.random.default_rng(77)
    lens = [int(x) for x in rng.integers(560, 640, 200)]
    w = get("c1_tiny").scaled(n_seqs=200, lengths=("list", tuple(lens)))
    print(f"[case] large grid: {len(lens)} sequences, 1 KV head", flush=True)
    cache = make_cache(w, lens)
    q_rot = fill(cache, w, lens, chunk=700)
    out = cache.decode(SeqBatch(range(len(lens)), lens), q_rot).cpu().numpy()
    r_k, r_v = cache.host_r
    for i in (0, 137):
        want = oracle_decode(w, i, 0, lens[i], r_k, r_v)
        err, rel, ok = compare_attention(out[i, :w.g], want)
        assert ok, (i, err, rel)
    print("[case] large grid ok", flush=True)


def test_append_many_sequences_device_lookup():
    """600 sequences per append call: beyond the host's per-sequence table in
    the kernel arguments (512), so the quantizer finds each position's
    sequence with its own prefix sum over the device arrays (chunked appends
    with flushes, then a one-token step); sampled rows bit-exact, decode
    within the attention bar."""
    from ultra_bit_kv_amd import SeqBatch
    n = 600
    lens = [30 + (7 * i) % 43 for i in range(n)]
    w = get("c1_tiny").scaled(n_seqs=n, hq=2, hkv=1, s_sink=4, s_keep=8, s_flush=8, group=32,
                              lengths=("list", tuple(lens)))
    print(f"[case] {n} sequences, lens {min(lens)}..{max(lens)}", flush=True)
    cache = make_cache(w, lens)
    q_rot = fill(cache, w, lens, chunk=16)
    r_k, r_v = cache.host_r
    out = cache.decode(SeqBatch(range(n), lens), q_rot).cpu().numpy()
    for i in list(range(0, n, 37)) + [n - 1]:
        hc = oracle_head(w, i, 0, lens[i], r_k, r_v)
        _check_head(cache, w, i, 0, lens[i], hc)
        err, rel, ok = compare_attention(out[i, :w.g], oracle_decode(w, i, 0, lens[i], r_k, r_v, hc))
        assert ok, (i, err, rel)
