"""Pins of the oracle's chunked-prefill attention (O6), on the CPU.

* Without quantization and with identity rotations the chunk output is plain
  causal attention with a position offset: checked against torch's
  scaled_dot_product_attention (fp64, explicit boolean mask).
* A one-token chunk is a decode step: its output equals the decode oracle on
  the same cache, also when its append flushes older ring rows to INT2 (so
  the prefix is read as stored after the append).  When the append quantizes
  the chunk's own rows the two differ: the chunk attends to them in bf16.
* Causality: later chunk rows do not change earlier outputs.
"""

import numpy as np
import pytest

from oracle import attention, cache, placement, prefill, rotate
from oracle.rounding import bf16_bits_to_f64
from synth import get

torch = pytest.importorskip("torch")


def _head(w, h, L, r_k, r_v, k=None, v=None):
    kk, kv = w.kappas()
    k = w.keys(0, 0, L)[:, h] if k is None else k
    v = w.values(0, 0, L)[:, h] if v is None else v
    return cache.HeadCache(k, v, r_k[h], r_v[h], kk[h], kv[h], w.group, w.s_sink, w.s_keep,
                           w.s_flush)


def _q_rot(w, lb, L, r_k, h):
    q = w.queries(0, lb, L)                                  # [n, Hq, D] bf16 bits
    qr = rotate.rotate_heads_to_bf16(q, r_k, g=w.g)          # [n, Hq, D]
    return bf16_bits_to_f64(qr[:, h * w.g:(h + 1) * w.g])    # [n, g, D]


def test_prefill_is_causal_attention_without_quantization():
    # identity rotations, windows wider than the row: every row stays bf16
    w = get("c1_tiny").scaled(s_sink=4, s_keep=4096)
    lb, n = 150, 70
    L = lb + n
    eye = np.broadcast_to(np.eye(128, dtype=np.float32), (w.hkv, 128, 128)).copy()
    hc = _head(w, 0, L, eye, eye)
    assert placement.segments(L, w.s_sink, w.s_keep, w.s_flush)[1] == (4, 4)
    q = _q_rot(w, lb, L, eye, 0)
    got = prefill.prefill_head(q, hc, lb)                    # [n, g, D]

    kf = torch.from_numpy(bf16_bits_to_f64(w.keys(0, 0, L)[:, 0]))
    vf = torch.from_numpy(bf16_bits_to_f64(w.values(0, 0, L)[:, 0]))
    qf = torch.from_numpy(q).permute(1, 0, 2).contiguous()  # [g, n, D]
    mask = torch.arange(L)[None, :] <= (lb + torch.arange(n))[:, None]   # [n, L]
    want = torch.nn.functional.scaled_dot_product_attention(
        qf, kf.expand(w.g, L, 128).contiguous(), vf.expand(w.g, L, 128).contiguous(),
        attn_mask=mask)
    want = want.permute(1, 0, 2).numpy()
    assert np.abs(got - want).max() < 1e-12


@pytest.mark.parametrize("lb", [37, 60, 61, 200])
def test_one_token_chunk_equals_decode(lb):
    # s_sink 4, s_keep 40, s_flush 16: appending token lb flushes [S_quant, +16)
    # when (lb + 1 - 44) is a multiple of 16 (lb = 59 + 16 k); 60 and 61 sit
    # just after such flushes, 37 is before any INT2 row exists
    w = get("c1_tiny").scaled(s_sink=4, s_keep=40, s_flush=16, group=64)
    r_k, r_v = w.rotations()
    L = lb + 1
    hc = _head(w, 0, L, r_k, r_v)
    q = _q_rot(w, lb, L, r_k, 0)
    got = prefill.prefill_head(q, hc, lb, r_v=r_v[0])[0]
    want = attention.decode_head(q[0], hc.k_dec, hc.v_dec, r_v[0])
    assert np.array_equal(got, want)


def test_one_token_chunk_after_flush_reads_int2_prefix():
    # lb = 59: the append of token 59 flushes positions [4, 20) of the ring to
    # INT2; the prefix of the chunk is read as INT2 there, exactly as decode
    w = get("c1_tiny").scaled(s_sink=4, s_keep=40, s_flush=16, group=64)
    r_k, r_v = w.rotations()
    lb = 59
    assert placement.s_quant(lb, 4, 40, 16) == 4 and placement.s_quant(lb + 1, 4, 40, 16) == 20
    hc = _head(w, 0, lb + 1, r_k, r_v)
    k, _ = prefill.context_rows(hc, lb, lb)
    assert not np.array_equal(k[4:20], bf16_bits_to_f64(hc.k_rot[4:20]))   # INT2 rows
    assert np.array_equal(k[:4], bf16_bits_to_f64(hc.k_rot[:4]))            # sink rows
    assert np.array_equal(k[20:], bf16_bits_to_f64(hc.k_rot[20:lb + 1]))    # ring + itself
    q = _q_rot(w, lb, lb + 1, r_k, 0)
    got = prefill.prefill_head(q, hc, lb, r_v=r_v[0])[0]
    want = attention.decode_head(q[0], hc.k_dec, hc.v_dec, r_v[0])
    assert np.array_equal(got, want)


def test_chunk_rows_are_read_in_bf16_even_when_quantized():
    # a long chunk: its append quantizes most of the chunk's own rows, which
    # the decode of its last token reads as INT2 but the chunk reads in bf16
    w = get("c1_tiny").scaled(s_sink=4, s_keep=40, s_flush=16, group=64)
    r_k, r_v = w.rotations()
    lb, n = 100, 200
    L = lb + n
    hc = _head(w, 0, L, r_k, r_v)
    sq = placement.s_quant(L, 4, 40, 16)
    assert sq > lb + 100
    q = _q_rot(w, lb, L, r_k, 0)
    last = prefill.prefill_head(q, hc, lb, r_v=r_v[0], rows=[n - 1])[n - 1]
    dec = attention.decode_head(q[-1], hc.k_dec, hc.v_dec, r_v[0])
    bf = attention.decode_head(q[-1], np.concatenate([hc.k_dec[:lb],
                                                      bf16_bits_to_f64(hc.k_rot[lb:])]),
                               np.concatenate([hc.v_dec[:lb], bf16_bits_to_f64(hc.v_rot[lb:])]),
                               r_v[0])
    assert np.abs(last - dec).max() > 1e-4       # the chunk rows differ from their INT2 form
    assert np.abs(last - bf).max() < 1e-12


def test_prefill_is_causal():
    w = get("c1_tiny").scaled(s_sink=4, s_keep=40, s_flush=16, group=64)
    r_k, r_v = w.rotations()
    lb, n = 80, 48
    L = lb + n
    k = w.keys(0, 0, L)[:, 0].copy()
    v = w.values(0, 0, L)[:, 0].copy()
    hc = _head(w, 0, L, r_k, r_v, k, v)
    q = _q_rot(w, lb, L, r_k, 0)
    base = prefill.prefill_head(q, hc, lb, r_v=r_v[0])
    # change the rows of chunk positions 30 .. 47: the cache after the append
    # changes there (and in INT2 groups those rows join), outputs 0 .. 29 do not
    k2, v2 = k.copy(), v.copy()
    k2[lb + 30:] ^= 0x0040
    v2[lb + 30:] ^= 0x0040
    hc2 = _head(w, 0, L, r_k, r_v, k2, v2)
    pert = prefill.prefill_head(q, hc2, lb, r_v=r_v[0])
    sq = placement.s_quant(L, 4, 40, 16)
    # quantization is per token, so the prefix (below lb) holds the same INT2
    # and window rows in both caches; earlier outputs are identical
    assert sq >= lb
    assert np.array_equal(base[:30], pert[:30])
    assert not np.array_equal(base[30:], pert[30:])
