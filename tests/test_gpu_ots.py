"""GPU parity of the OScaR key mode (OScaR notes, step two "Omni-Token
Scaling", the background "KIVI and the per-channel paradigm" and the cache
layout figure), through the C ABI, against ``oracle.ots.OtsHeadCache``.

Bars: every OScaR page-head block (K codes, V codes and parameters, token
scales, per-channel Delta / z) and every window row bit-exact, the rotated
query bit-exact, dequantized rows bit-exact, attention within max-abs 2e-3 /
rel-L2 1e-3.

Cases: the workload's own windows (no sink, no kept rows, 128-token flushes)
at reduced batch, a sink and kept rows with 32-token flushes, appends in
300-token chunks and token by token (each one-token step that completes a
flush moves a whole key block), the dense per-head rotation and both
structured rotations, a context whose recent ring is empty, and a sequence
with no INT2 block yet.
"""

import numpy as np
import pytest

from oracle import layout, placement
from synth import get
from tests.oscar_testlib import (make_cache, fill, oracle_ots_head, oracle_q_rot,
                                 compare_attention)
from oracle.rounding import bf16_bits_to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

D = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ultra_bit_kv_amd import lib
    lib()


def _case_workload(name):
    base = get("ots_bs48")
    if name == "flush128":   # the workload's windows; 4096 empties the ring
        return base.scaled(n_seqs=4, hq=8, hkv=2, lengths=("list", (4096, 1000, 333, 100))), \
            [4096, 1000, 333, 100]
    if name == "sink_keep":  # a sink, kept rows, 32-token flushes
        w = base.scaled(n_seqs=3, hq=16, hkv=4, s_sink=16, s_keep=40, s_flush=32,
                        kappa=(1.0, 0.93), lengths=("list", (700, 129, 1250)))
        return w, [700, 129, 1250]
    raise KeyError(name)


def _check_ots_head(cache, w, i, h, L, hc):
    bt = cache.host_block_table
    n_pages = placement.n_int2_pages(L, w.s_sink, w.s_keep, w.s_flush)
    assert n_pages % 2 == 0
    for m in range(n_pages):
        got = cache.page_head(int(bt[i, m]), h)
        want, nv = hc.page_block(m)
        assert nv == 16
        if not np.array_equal(got, want):
            g = layout.unpack_ots_page_head(got)
            e = layout.unpack_ots_page_head(want)
            names = ["kc", "vc", "ks16", "kd16", "kz16", "vs", "vz"]
            bad = [n for n, a, b in zip(names, g, e) if not np.array_equal(a, b)]
            raise AssertionError(f"seq {i} head {h} page {m}: fields differ: {bad}")
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


def _decode_head(w, i, h, L, r_k, r_v, hc):
    from oracle import attention
    qr = bf16_bits_to_f64(oracle_q_rot(w, i, L, r_k)[h * w.g:(h + 1) * w.g])
    return attention.decode_head(qr, hc.k_dec, hc.v_dec, r_v[h])


@pytest.mark.parametrize("rotation", [0, 1, 2])
@pytest.mark.parametrize("name", ["flush128", "sink_keep"])
def test_ots_append_bit_exact_and_decode(name, rotation):
    from ultra_bit_kv_amd import SeqBatch
    w, lens = _case_workload(name)
    print(f"[case] ots {name} rotation={rotation} lens={lens}", flush=True)
    cache = make_cache(w, lens, rotation=rotation, key_mode=1)
    q_rot = fill(cache, w, lens, chunk=300)
    r_k, r_v = cache.host_r
    out = cache.decode(SeqBatch(range(len(lens)), lens), q_rot)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    qr = q_rot.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    worst = (0.0, 0.0)
    for i, L in enumerate(lens):
        assert np.array_equal(qr[i], oracle_q_rot(w, i, L, r_k)), i
        for h in range(w.hkv):
            hc = oracle_ots_head(w, i, h, L, r_k, r_v)
            _check_ots_head(cache, w, i, h, L, hc)
            want = _decode_head(w, i, h, L, r_k, r_v, hc)
            err, rel, ok = compare_attention(out[i, h * w.g:(h + 1) * w.g], want)
            worst = (max(worst[0], err), max(worst[1], rel))
            assert ok, (name, rotation, i, h, err, rel)
    print(f"[case] ots {name} rotation={rotation} max_abs={worst[0]:.3e} rel={worst[1]:.3e}",
          flush=True)


def test_ots_token_by_token_equals_chunked():
    """Every step appends one token; the steps that complete a flush move a
    whole key block (the general append path).  The cache must equal the
    one built from chunks, and the oracle's."""
    from ultra_bit_kv_amd import SeqBatch
    w = get("ots_bs48").scaled(n_seqs=2, hq=8, hkv=2, s_sink=4, s_keep=3, s_flush=32,
                               lengths=("list", (200, 150)))
    lens = [200, 150]
    print(f"[case] ots token-by-token lens={lens}", flush=True)
    a = make_cache(w, lens, rotation=1, key_mode=1)
    b = make_cache(w, lens, rotation=1, key_mode=1)
    fill(a, w, lens, chunk=1)
    q_rot = fill(b, w, lens, chunk=64)
    # (ring slots that no longer hold a live row keep whatever the history
    # left there, so only the live window rows are compared)
    assert torch.equal(a.pages, b.pages)
    r_k, r_v = b.host_r
    out = b.decode(SeqBatch(range(len(lens)), lens), q_rot).cpu().numpy()
    for i, L in enumerate(lens):
        for h in range(w.hkv):
            hc = oracle_ots_head(w, i, h, L, r_k, r_v)
            _check_ots_head(a, w, i, h, L, hc)
            _check_ots_head(b, w, i, h, L, hc)
            err, rel, ok = compare_attention(out[i, h * w.g:(h + 1) * w.g],
                                             _decode_head(w, i, h, L, r_k, r_v, hc))
            assert ok, (i, h, err, rel)


def test_ots_workload_sampled():
    """The benchmark's workload and launch plan (48 sequences x 4096 tokens,
    8 KV heads, Hadamard rotation): cache bytes of sampled sequences
    bit-exact, their decode outputs within the bar."""
    from ultra_bit_kv_amd import SeqBatch
    w = get("ots_bs48")
    lens = [int(x) for x in w.lengths_after()]
    print(f"[case] ots workload {len(lens)} x {lens[0]}", flush=True)
    cache = make_cache(w, lens, rotation=1, key_mode=1)
    q_rot = fill(cache, w, lens, chunk=4096)
    r_k, r_v = cache.host_r
    out = cache.decode(SeqBatch(range(len(lens)), lens), q_rot).cpu().numpy()
    for i in (0, 17, 47):
        for h in (0, 5):
            hc = oracle_ots_head(w, i, h, lens[i], r_k, r_v)
            _check_ots_head(cache, w, i, h, lens[i], hc)
            err, rel, ok = compare_attention(out[i, h * w.g:(h + 1) * w.g],
                                             _decode_head(w, i, h, lens[i], r_k, r_v, hc))
            assert ok, (i, h, err, rel)
    print("[case] ots workload sampled heads ok", flush=True)


def test_ots_prefill_rejected():
    from ultra_bit_kv_amd import OscarError, SeqBatch
    w, lens = _case_workload("flush128")
    cache = make_cache(w, lens[:1], rotation=1, key_mode=1)
    k = w.keys(0, 0, 64)
    v = w.values(0, 0, 64)
    q = w.queries(0, 0, 64)
    q_rot, k_rot, v_rot = cache.append_tokens([0], [0], [64], k, v, q, want_rot=True)
    with pytest.raises(OscarError):
        cache.prefill_attn(SeqBatch([0], [0], [64]), q_rot, k_rot, v_rot)
