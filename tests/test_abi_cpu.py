"""The C ABI on the host: symbols, sizes and every argument check (no GPU).

All checks in liboscar_kv run on the host before anything is enqueued, so the
error paths are exercised here without a device.  Pointers in these calls are
dummies that are never dereferenced.
"""

import ctypes
import os
import re

import numpy as np
import pytest

from ultra_bit_kv_amd import _lib
from ultra_bit_kv_amd._lib import KvCache, KvConfig

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oscar_kv.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("liboscar_kv.so not built")
    return _lib.lib()


def declared_functions(headers=(HEADER,)):
    names = set()
    for hdr in headers:
        text = open(hdr).read()
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(oscar_\w+)\s*\(", text, re.M))
    return sorted(names)


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("oscar_rotate_quant_append", "oscar_int2_decode_attn", "oscar_dequant",
              "oscar_workspace_size", "oscar_status_string", "oscar_check_config"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    names = declared_functions(HEADERS)
    assert "oscar_read_probe" in names
    for n in names:
        assert hasattr(L, n), n


def test_read_probe_argument_checks(L):
    f = L.oscar_read_probe
    buf, sink = DUMMY, DUMMY
    assert f(None, 1024, None, 0, 0, sink, 1, 4, None) == -1
    assert f(buf, 1024, None, 0, 0, None, 1, 4, None) == -1
    assert f(ctypes.c_void_p(DUMMY.value + 4), 1024, None, 0, 0, sink, 1, 4, None) == -10
    assert f(buf, 1000, None, 0, 0, sink, 1, 4, None) == -10          # not a multiple of 1 KB
    assert f(buf, 1024, None, 0, 0, sink, 2, 4, None) == -10          # sink too small for the grid
    assert f(buf, 1024, None, 0, 0, sink, 0, 4, None) == -10
    assert f(buf, 4096, DUMMY, 4, 1000, sink, 1, 4, None) == -10      # chunk size
    assert f(buf, 4096, DUMMY, -1, 1024, sink, 1, 4, None) == -10
    assert f(buf, 4096, None, 0, 0, sink, 1, 4, None) in (-9, -8, 0)  # reaches the device check


def cfg(**kw):
    c = KvConfig()
    c.head_dim, c.num_q_heads, c.num_kv_heads, c.group_size, c.page_size = 128, 32, 8, 64, 16
    c.s_sink, c.s_keep, c.s_flush = 64, 256, 16
    c.max_seqs, c.max_pages_per_seq, c.num_pages = 4, 100, 400
    for h in range(64):
        c.clip_k[h] = 0.96
        c.clip_v[h] = 0.92
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("kw, status", [
    ({}, 0),
    ({"head_dim": 64}, -2), ({"page_size": 32}, -2), ({"num_kv_heads": 0}, -2),
    ({"num_kv_heads": 65}, -2), ({"num_q_heads": 30}, -2),
    ({"group_size": 48}, -3), ({"group_size": 256}, -3),
    ({"s_flush": 0}, -5), ({"s_sink": -1}, -5), ({"s_keep": -3}, -5),
    ({"max_seqs": 0}, -6),
])
def test_check_config(L, kw, status):
    c = cfg(**kw)
    assert L.oscar_check_config(ctypes.byref(c)) == status
    assert L.oscar_status_string(status)


def test_clip_range_checked(L):
    for bad in (0.49, 1.01, float("nan")):
        c = cfg()
        c.clip_v[3] = bad
        assert L.oscar_check_config(ctypes.byref(c)) == -4
    c = cfg()
    c.clip_k[7], c.clip_v[0] = 0.5, 1.0
    assert L.oscar_check_config(ctypes.byref(c)) == 0
    c.clip_k[8] = 7.0      # beyond num_kv_heads: ignored
    assert L.oscar_check_config(ctypes.byref(c)) == 0


def test_sizes(L):
    for g, pb in ((128, 1152), (64, 1280), (32, 1536)):
        assert L.oscar_page_head_bytes(g) == pb
    assert L.oscar_page_head_bytes(48) == 0
    c = cfg()
    assert L.oscar_pages_bytes(ctypes.byref(c)) == 400 * 8 * 1280
    assert L.oscar_ring_capacity(ctypes.byref(c)) == 272
    nb = 64 // 16 + 272 // 16
    assert L.oscar_win_bytes(ctypes.byref(c)) == 4 * 8 * nb * 2 * 16 * 128 * 2
    # longest row: S_quant(len) - S_sink <= 16 * 100
    mx = L.oscar_max_seq_len(ctypes.byref(c))
    assert mx == 64 + 256 + (100 + 1) * 16 - 1
    assert L.oscar_workspace_size(ctypes.byref(c), 4, 1000) > 2 * 1000 * 8 * 128 * 2
    c5 = cfg(s_flush=24)
    mx5 = L.oscar_max_seq_len(ctypes.byref(c5))
    # len = mx5 fits, len = mx5 + 1 needs one more page than the row has
    sq = lambda n: 64 + 24 * max(0, (n - 64 - 256) // 24)
    assert -(-(sq(mx5) - 64) // 16) <= 100 < -(-(sq(mx5 + 1) - 64) // 16)


DUMMY = ctypes.c_void_p(0x1000)


def _cache(c, r_q=None, out_rotated=0, r_v=0x1000, r_k=0x1000, rotation=0):
    return KvCache(c, 0x1000, 0x1000, 0x1000, r_k, r_v, r_q, out_rotated, rotation)


def _i32(a):
    a = np.ascontiguousarray(np.asarray(a, np.int32))
    return a, a.ctypes.data_as(ctypes.c_void_p)


def append(L, c, slots, lb, n_new, ws_bytes=1 << 40, k=DUMMY, q=None, q_rot=None, cache=None):
    cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)
    keep = [_i32(slots), _i32(lb), _i32(cu)]
    return L.oscar_rotate_quant_append(
        ctypes.byref(cache or _cache(c)), len(slots), keep[0][1], keep[1][1], keep[2][1],
        DUMMY, DUMMY, DUMMY, k, DUMMY, q, q_rot, None, None, DUMMY, ws_bytes, None)


def decode(L, c, slots, lens, ws_bytes=1 << 40, out=DUMMY):
    keep = [_i32(slots), _i32(lens)]
    return L.oscar_int2_decode_attn(ctypes.byref(_cache(c)), len(slots), keep[0][1], keep[1][1],
                                    DUMMY, DUMMY, DUMMY, out, DUMMY, ws_bytes, None)


def test_append_argument_checks(L):
    c = cfg()
    assert append(L, c, [0], [0], [5], k=None) == -1                 # null keys
    assert append(L, c, [0], [0], [5], q=None, q_rot=DUMMY) == -1    # q_rot without q
    assert append(L, c, [4], [0], [5]) == -6                          # slot >= max_seqs
    assert append(L, c, [1, 1], [0, 0], [5, 5]) == -10                # duplicate slot
    assert append(L, c, [0], [-1], [5]) == -10                        # negative length
    mx = L.oscar_max_seq_len(ctypes.byref(c))
    assert append(L, c, [0], [mx], [1]) == -6                         # beyond the row
    assert append(L, c, [0], [0], [5], ws_bytes=10) == -7             # workspace
    bad = cfg(group_size=7)
    assert append(L, bad, [0], [0], [5]) == -3
    # a valid call reaches the device check: without a GPU that is a HIP error
    st = append(L, c, [0, 2], [0, 10], [5, 7])
    assert st in (-9, -8, 0)


def test_decode_argument_checks(L):
    c = cfg()
    assert decode(L, c, [0], [0]) == -10                              # empty context
    assert decode(L, c, [9], [10]) == -6
    assert decode(L, c, [0], [10], out=None) == -1
    assert decode(L, c, [0], [10], ws_bytes=100) == -7
    assert decode(L, c, [0, 1, 2, 3, 0], [5] * 5) == -10              # n_seqs > max_seqs
    mx = L.oscar_max_seq_len(ctypes.byref(c))
    assert decode(L, c, [0], [mx + 1]) == -6
    assert decode(L, c, [0], [mx]) in (-9, -8, 0)


def test_misaligned_pointers_are_rejected(L):
    c = cfg()
    bad = ctypes.c_void_p(DUMMY.value + 4)
    assert decode(L, c, [0], [10], out=bad) == -10
    assert append(L, c, [0], [0], [5], k=bad) == -10


def test_decode_phase_argument_checks(L):
    c = cfg()
    keep = [_i32([0]), _i32([10])]
    part = lambda q, ws=1 << 40: L.oscar_int2_decode_partials(
        ctypes.byref(_cache(c)), 1, keep[0][1], keep[1][1], DUMMY, DUMMY, q, DUMMY, ws, None)
    merge = lambda out, ws=1 << 40: L.oscar_int2_decode_merge(
        ctypes.byref(_cache(c)), 1, keep[0][1], keep[1][1], DUMMY, DUMMY, out, DUMMY, ws, None)
    assert part(None) == -1                                           # the split needs q_rot
    assert merge(None) == -1                                          # the merge needs out
    assert part(DUMMY, ws=100) == -7 and merge(DUMMY, ws=100) == -7
    assert part(DUMMY) in (-9, -8, 0) and merge(DUMMY) in (-9, -8, 0)
    # the separate calls share one launch's workspace: at most 2048 sequences
    big = cfg(max_seqs=3000)
    sl, ln = _i32(np.arange(2049)), _i32(np.full(2049, 10))
    assert L.oscar_int2_decode_partials(ctypes.byref(_cache(big)), 2049, sl[1], ln[1], DUMMY, DUMMY,
                                        DUMMY, DUMMY, 1 << 40, None) == -10
    assert L.oscar_int2_decode_merge(ctypes.byref(_cache(big)), 2049, sl[1], ln[1], DUMMY, DUMMY,
                                     DUMMY, DUMMY, 1 << 40, None) == -10


def test_dequant_argument_checks(L):
    c = cfg()
    cache = _cache(c)
    f = L.oscar_dequant
    assert f(ctypes.byref(cache), 0, 100, 50, 40, DUMMY, DUMMY, None) == -10
    assert f(ctypes.byref(cache), 0, 100, 0, 101, DUMMY, DUMMY, None) == -10
    assert f(ctypes.byref(cache), 5, 100, 0, 10, DUMMY, DUMMY, None) == -6
    assert f(ctypes.byref(cache), 0, 100, 0, 10, None, DUMMY, None) == -1


# ---- plain BF16 paged cache (the uncompressed comparison point) ----------

def bcache(**kw):
    b = _lib.Bf16Cache(128, 32, 8, 16, 4, 100, 400, 0x1000, 0x1000)
    for k, v in kw.items():
        setattr(b, k, v)
    return b


def bdecode(L, b, slots, lens, ws_bytes=1 << 40, q=DUMMY, out=DUMMY, n=None):
    keep = [_i32(slots), _i32(lens)]
    return L.oscar_bf16_paged_decode_attn(ctypes.byref(b), len(slots) if n is None else n,
                                          keep[0][1], keep[1][1], DUMMY, DUMMY, q, out, DUMMY,
                                          ws_bytes, None)


@pytest.mark.parametrize("kw, status", [
    ({"head_dim": 64}, -2), ({"page_size": 8}, -2), ({"num_kv_heads": 0}, -2),
    ({"num_kv_heads": 65}, -2), ({"num_q_heads": 30}, -2),
    ({"num_q_heads": 512, "num_kv_heads": 1}, -2),
    ({"max_seqs": 0}, -6), ({"max_pages_per_seq": 65537}, -6), ({"num_pages": -1}, -6),
])
def test_bf16_description_checks(L, kw, status):
    b = bcache(**kw)
    assert bdecode(L, b, [0], [10]) == status
    assert L.oscar_bf16_workspace_size(ctypes.byref(b), 4) == 0


def test_bf16_workspace_size(L):
    # g = 4 -> 4 heads per pass, one pass; a record is 8 + 4 * 128 floats.
    # 16K records per launch: n = 4 -> 32 rows -> 256 splits
    b = bcache()
    rec = 8 + 4 * 128
    for n, cap in ((4, 256), (64, 32), (2048, 1)):
        rows = n * 8
        want = -(-(rows * cap * rec * 4) // 256) * 256
        assert L.oscar_bf16_workspace_size(ctypes.byref(b), n) == want, n
    # the largest row always fits: 65536 pages = 32768 pairs needs 129 splits
    big = bcache(max_pages_per_seq=65536, max_seqs=4096)
    assert L.oscar_bf16_workspace_size(ctypes.byref(big), 2048) >= 2048 * 8 * 129 * rec * 4


def test_bf16_decode_argument_checks(L):
    b = bcache()
    assert bdecode(L, b, [0], [0]) == -10                              # empty row
    assert bdecode(L, b, [9], [10]) == -6                              # slot
    assert bdecode(L, b, [0], [100 * 16 + 1]) == -6                    # more pages than the row
    assert bdecode(L, b, [0], [10], q=None) == -1
    assert bdecode(L, b, [0], [10], out=None) == -1
    assert bdecode(L, b, [0], [10], ws_bytes=100) == -7
    assert bdecode(L, b, [0, 1, 2, 3, 0], [5] * 5) == -10              # n_seqs > max_seqs
    assert bdecode(L, b, [0], [10], n=0) == -10
    bad = ctypes.c_void_p(DUMMY.value + 4)
    assert bdecode(L, b, [0], [10], q=bad) == -10
    assert bdecode(L, bcache(num_pages=0), [0], [10]) == -6            # no pages to read
    assert bdecode(L, b, [0, 3], [100 * 16, 1]) in (-9, -8, 0)         # valid: device check


def test_query_transform_and_absorbed_output_checks(L):
    c = cfg()
    keep = [_i32([0]), _i32([10])]
    dec = lambda cache: L.oscar_int2_decode_attn(ctypes.byref(cache), 1, keep[0][1], keep[1][1],
                                                 DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, 1 << 40, None)
    assert dec(_cache(c, r_v=None)) == -1                          # un-rotation needs R_V
    assert dec(_cache(c, r_v=None, out_rotated=1)) in (-9, -8, 0)   # absorbed: R_V not read
    assert dec(_cache(c, r_q=DUMMY.value + 4)) == -10               # misaligned query transform
    assert append(L, c, [0], [0], [5], cache=_cache(c, r_q=DUMMY.value + 4)) == -10
    assert append(L, c, [0], [0], [5], cache=_cache(c, r_q=DUMMY.value)) in (-9, -8, 0)


def prefill(L, c, slots, lb, n_new, q_rot=DUMMY, k_rot=DUMMY, v_rot=DUMMY, out=DUMMY,
            cache=None, cu=None):
    cu = np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32) if cu is None else np.asarray(cu, np.int32)
    keep = [_i32(slots), _i32(lb), _i32(cu)]
    return L.oscar_int2_prefill_attn(
        ctypes.byref(cache or _cache(c)), len(slots), keep[0][1], keep[1][1], keep[2][1],
        DUMMY, DUMMY, DUMMY, q_rot, k_rot, v_rot, out, None)


def test_prefill_argument_checks(L):
    c = cfg()
    assert prefill(L, c, [0], [0], [5], q_rot=None) == -1
    assert prefill(L, c, [0], [0], [5], k_rot=None) == -1
    assert prefill(L, c, [0], [0], [5], out=None) == -1
    assert prefill(L, c, [0], [0], [5], cache=_cache(c, r_v=0)) == -1      # un-rotation needs R_V
    assert prefill(L, c, [0], [0], [5], out=ctypes.c_void_p(0x1004)) == -10  # misaligned
    assert prefill(L, c, [4], [0], [5]) == -6                               # slot >= max_seqs
    assert prefill(L, c, [1, 1], [0, 0], [5, 5]) == -10                     # duplicate slot
    assert prefill(L, c, [0], [-1], [5]) == -10                             # negative length
    assert prefill(L, c, [0], [0], [5], cu=[1, 6]) == -10                   # cu_new[0] != 0
    assert prefill(L, c, [0, 1], [0, 0], [5, 5], cu=[0, 5, 3]) == -10       # negative count
    mx = L.oscar_max_seq_len(ctypes.byref(c))
    assert prefill(L, c, [0], [mx - 2], [3]) == -6                          # beyond the row
    assert prefill(L, c, [0, 1, 2, 3, 0], [0] * 5, [1] * 5) == -10          # n_seqs > max_seqs
    # without R_V the rotated-basis output is still valid; a valid call reaches
    # the device check (a HIP error without a GPU)
    assert prefill(L, c, [0], [0], [5], cache=_cache(c, r_v=0, out_rotated=1)) in (-9, -8, 0)
    assert prefill(L, c, [0, 2], [100, 0], [7, 300]) in (-9, -8, 0)


def test_structured_rotation_argument_checks(L):
    c = cfg()
    bare = dict(r_k=None, r_v=None)
    for kind in (1, 2):
        ok = _cache(c, rotation=kind, **bare)
        # the structured kinds take no matrices; a valid call reaches the device check
        assert append(L, c, [0], [0], [5], cache=ok) in (-9, -8, 0)
        assert prefill(L, c, [0], [0], [5], cache=ok) in (-9, -8, 0)
        keep = [_i32([0]), _i32([10])]
        assert L.oscar_int2_decode_attn(ctypes.byref(ok), 1, keep[0][1], keep[1][1], DUMMY, DUMMY,
                                        DUMMY, DUMMY, DUMMY, 1 << 40, None) in (-9, -8, 0)
        # a matrix alongside a structured kind is rejected
        for extra in (dict(r_k=0x1000, r_v=None), dict(r_k=None, r_v=0x1000),
                      dict(r_k=None, r_v=None, r_q=0x1000)):
            bad = _cache(c, rotation=kind, **extra)
            assert append(L, c, [0], [0], [5], cache=bad) == -10
            assert prefill(L, c, [0], [0], [5], cache=bad) == -10
    for kind in (-1, 3):
        assert append(L, c, [0], [0], [5], cache=_cache(c, rotation=kind, **bare)) in (-1, -10)
        assert append(L, c, [0], [0], [5], cache=_cache(c, rotation=kind)) == -10
        assert prefill(L, c, [0], [0], [5], cache=_cache(c, rotation=kind)) == -10


def test_noalloc_decode_argument_checks(L):
    """oscar_int2_decode_attn_noalloc: the host checks of the workspace form,
    and a launch whose split records cannot fit the fixed scratch is refused
    before anything reaches the device."""
    f = L.oscar_int2_decode_attn_noalloc

    def call(c, slots, lens, q=DUMMY, out=DUMMY):
        cache = KvCache(c, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, None, 0, 0)
        s = np.asarray(slots, np.int32)
        ln = np.asarray(lens, np.int32)
        return f(ctypes.byref(cache), len(s), s.ctypes.data_as(ctypes.c_void_p),
                 ln.ctypes.data_as(ctypes.c_void_p), DUMMY, DUMMY, q, out, None)

    c = cfg()
    assert call(c, [0], [0]) == -10
    assert call(c, [9], [10]) == -6
    assert call(c, [0], [10], out=None) == -1
    assert call(c, [0], [10], q=ctypes.c_void_p(DUMMY.value + 4)) == -10
    assert call(c, [0], [10]) in (-9, -8, 0)
    # 2048 sequences x 64 KV heads x one query head each: one split record
    # per row is already 2048 * 64 * 528 B > 64 MiB
    big = cfg(num_q_heads=64, num_kv_heads=64, max_seqs=2048, max_pages_per_seq=4)
    assert call(big, list(range(2048)), [10] * 2048) == -7
