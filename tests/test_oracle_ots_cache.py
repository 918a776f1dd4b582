"""Pins of the OScaR cache as a whole (``oracle.ots.OtsHeadCache``) and of its
page layout (``oracle.layout.pack_ots_page_head``): the INT2 keys are exactly
the pinned per-block O7 path, the windows and values are the OSCAR cache's,
and every field of the page block sits where the layout text puts it."""

import numpy as np
import pytest

from oracle import layout, ots, placement, rotate
from oracle.cache import HeadCache
from oracle.rounding import bf16_bits_to_f64
from synth.workloads import bf16_from_f32


def _rows(seed, n, scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 128)).astype(np.float32) * np.float32(scale)
    x[:, [3, 70]] *= np.float32(20.0)              # outlier channels
    x[:4] *= np.float32(0.05)                      # low-norm tokens
    return bf16_from_f32(x)


@pytest.mark.parametrize("s_sink,s_keep,s_flush,n", [(0, 0, 128, 700), (64, 0, 128, 1000),
                                                     (16, 32, 64, 333), (0, 0, 32, 32)])
def test_int2_keys_are_the_block_path(s_sink, s_keep, s_flush, n):
    k, v = _rows(1, n), _rows(2, n)
    had = rotate.Hadamard(128)
    hc = ots.OtsHeadCache(k, v, had, had, np.float32(1.0), 32, s_sink, s_keep, s_flush)
    a, b = hc.int2
    assert (a, b) == placement.segments(n, s_sink, s_keep, s_flush)[1]
    assert (b - a) % 32 == 0
    if b > a:
        # ots_keys runs rotation, scaling and per-block quantization from the raw rows
        assert np.array_equal(hc.k_dec[a:b], ots.ots_keys(k[a:b], 32))
    # windows keep the rotated rows
    win = [p for p in range(n) if not a <= p < b]
    assert np.array_equal(hc.k_dec[win], bf16_bits_to_f64(rotate.hadamard_rotate_to_bf16(k, False))[win])


def test_values_are_the_per_token_quantizer():
    n = 640
    k, v = _rows(3, n), _rows(4, n, 3.0)
    had = rotate.Hadamard(128, bitrev=True)
    o = ots.OtsHeadCache(k, v, had, had, np.float32(0.93), 32, 0, 0, 128)
    h = HeadCache(k, v, had, had, np.float32(0.9), np.float32(0.93), 32, 0, 0, 128)
    assert np.array_equal(o.v_dec, h.v_dec)
    assert np.array_equal(o.vc, h.vc) and np.array_equal(o.vs, h.vs) and np.array_equal(o.vz, h.vz)


def test_ots_page_fields_where_the_layout_puts_them():
    z = np.zeros((16, 128), np.uint8)
    zp = np.zeros((16, 4), np.uint16)
    ks = np.zeros(16, np.uint16)
    ks[5] = 0x3F80                                   # bf16 1.0 as the scale of slot 5
    kd = np.zeros(64, np.uint16)
    kz = np.zeros(64, np.uint16)
    kd[9], kz[9] = 0x3E00, 0x4040                    # Delta, z of the page's channel 9
    blk = layout.pack_ots_page_head(z, z, ks, kd, kz, zp, zp)
    assert blk.shape == (1568,)
    assert blk[1280:1312].view(np.uint16)[5] == 0x3F80
    assert blk[1312 + 4 * 9:1312 + 4 * 10].view(np.uint32)[0] == 0x3E00 | (0x4040 << 16)
    assert np.count_nonzero(blk.view(np.uint16)) == 3   # the scale and the two halves of the pair
    vs = zp.copy()
    vs[7, 2] = 0x1234                                # V params keep the (group, slot) order
    blk = layout.pack_ots_page_head(z, z, np.zeros(16, np.uint16), kd * 0, kz * 0, vs, zp)
    assert blk[1024 + 4 * (16 * 2 + 7):1024 + 4 * (16 * 2 + 8)].view(np.uint32)[0] == 0x1234


def test_page_blocks_split_the_channels_of_a_key_block():
    n = 64 + 4 * 32 + 5
    k, v = _rows(5, n), _rows(6, n)
    had = rotate.Hadamard(128)
    hc = ots.OtsHeadCache(k, v, had, had, np.float32(1.0), 32, 64, 0, 32)
    a, b = hc.int2
    assert b - a == 128                              # four blocks, eight pages
    for m in range(8):
        blk, nv = hc.page_block(m)
        kc, vc, ts, kd, kz, vs, vz = layout.unpack_ots_page_head(blk)
        assert nv == 16
        r = slice(16 * m, 16 * m + 16)
        assert np.array_equal(kc, hc.kc[r]) and np.array_equal(ts, hc.ks16[r])
        ch = slice(64 * (m % 2), 64 * (m % 2) + 64)
        assert np.array_equal(kd, hc.kd16[m // 2, ch]) and np.array_equal(kz, hc.kz16[m // 2, ch])


def test_memory_per_token_head():
    # codes 32 + 32 B, token scale 2 B, value params 4 x 4 B, key channel
    # params 2 x 2 x 128 B per 32 tokens: 98 B against 512 B in BF16
    per_token = layout.OTS_PAGE_HEAD_BYTES / 16
    assert per_token == 98.0
    assert abs(512 / per_token - 5.22) < 0.01        # the OScaR notes report 5.3x
