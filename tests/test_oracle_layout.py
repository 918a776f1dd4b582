"""Pins of the documented byte layout (``oracle/layout.py``) against the
layout text of include/oscar_kv.h, element by element, and of the batched
page packer against the per-page one."""

import numpy as np
import pytest

from oracle import layout


def test_param_word_order_group_major():
    # "K params, uint32 word (16 gr + t): fp16 scale (bits 0..15), fp16 zero
    # (bits 16..31) of group gr, slot t" -- one (group, slot) set, all else 0
    for ng, gr, t in ((4, 1, 3), (2, 1, 15), (1, 0, 7), (4, 3, 0)):
        s = np.zeros((16, ng), np.uint16)
        z = np.zeros((16, ng), np.uint16)
        s[t, gr] = 0x1234
        z[t, gr] = 0xABCD
        w = layout.pack_params(s, z)
        assert w.shape == (16 * ng,)
        assert w[16 * gr + t] == 0xABCD1234 and np.count_nonzero(w) == 1


def test_param_words_in_the_page_block():
    # K params start at byte 1024, V params at 1024 + 64 ng
    for g in (32, 64, 128):
        ng = 128 // g
        zc = np.zeros((16, 128), np.uint8)
        zp = np.zeros((16, ng), np.uint16)
        ks = zp.copy()
        ks[2, ng - 1] = 0x3C00          # fp16 1.0, last group, slot 2
        vz = zp.copy()
        vz[9, 0] = 0xC000               # fp16 -2.0 as a V zero point, group 0, slot 9
        blk = layout.pack_page_head(zc, zc, ks, zp, zp, vz, g).view(np.uint32)
        assert blk[256 + 16 * (ng - 1) + 2] == 0x3C00
        assert blk[256 + 16 * ng + 9] == 0xC000 << 16
        assert np.count_nonzero(blk) == 2


def test_window_v_element_index():
    # "part 1 (V) holds (t, c) at element 32 (16 (t/4) + c/8) + 4 (c%8) + t%4"
    for t, c in ((5, 10), (0, 0), (15, 127), (3, 8), (12, 71)):
        k = np.zeros((16, 128), np.uint16)
        v = np.zeros((16, 128), np.uint16)
        v[t, c] = 0xBEEF
        k[t, c] = 0x1111
        blk = layout.pack_window_block(k, v)
        want_v = 2048 + 32 * (16 * (t // 4) + c // 8) + 4 * (c % 8) + t % 4
        assert blk[want_v] == 0xBEEF and blk[128 * t + c] == 0x1111
        assert np.count_nonzero(blk) == 2
    assert layout.v_window_index(5, 10) == 32 * 17 + 8 + 1


def test_window_v_index_is_a_permutation():
    t = np.arange(16)[:, None]
    c = np.arange(128)[None, :]
    idx = layout.v_window_index(t, c).reshape(-1)
    assert sorted(idx.tolist()) == list(range(2048))


@pytest.mark.parametrize("g", [32, 64, 128])
def test_batched_packer_equals_per_page_packer(g):
    rng = np.random.default_rng(300 + g)
    ng = 128 // g
    n = 7
    kc = rng.integers(0, 4, (n, 16, 128)).astype(np.uint8)
    vc = rng.integers(0, 4, (n, 16, 128)).astype(np.uint8)
    ks, kz, vs, vz = (rng.integers(0, 1 << 16, (n, 16, ng)).astype(np.uint16) for _ in range(4))
    got = layout.pack_page_heads(kc, vc, ks, kz, vs, vz, g)
    assert got.shape == (n, layout.page_head_bytes(g))
    for i in range(n):
        assert np.array_equal(got[i], layout.pack_page_head(kc[i], vc[i], ks[i], kz[i], vs[i],
                                                            vz[i], g)), i
