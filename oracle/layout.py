"""The documented on-HBM byte layout of the INT2 pages and BF16 window blocks.

Test infrastructure (see ``oracle/__init__.py``).  Written from the layout
definition in ``include/oscar_kv.h`` (four 2-bit codes per byte, as in the
OSCAR summary page, section 4 "KV Cache Update"), independently of the kernels,
so the tests can compare the GPU cache bytes with the oracle's bit for bit.

Page-head block (one physical page, one KV head, 16 token slots), PB bytes,
PB = 1024 + 128 * ng with ng = 128 / G:
  [0, 512)            K codes, token-major: uint32 word (8 t + w) holds
                      channels 16 w + i (i = 0..15) of slot t at bits 2i..2i+1.
  [512, 1024)         V codes: uint32 word u = 2 (16 a + m) + e holds
                      code(slot 4a + 2e,     channel 8m + j) at bits 2j..2j+1 and
                      code(slot 4a + 2e + 1, channel 8m + j) at bits 16+2j..17+2j,
                      for a = 0..3, m = 0..15, e = 0..1, j = 0..7.
  [1024, 1024+64ng)   K params: uint32 word (16 gr + t) = fp16 scale | fp16 zero << 16
                      for group gr, slot t.
  [1024+64ng, PB)     V params, same order.

OScaR page-head block (keys per channel over blocks of 32 tokens, G = 32),
1568 bytes:
  [0, 512)            K codes, as above.
  [512, 1024)         V codes, as above.
  [1024, 1280)        V params, as above (4 groups).
  [1280, 1312)        K token scales: bf16 s_t of slot t at uint16 index t.
  [1312, 1568)        K channel params of channels 64 h .. 64 h + 63, h = (logical
                      INT2 page) mod 2 (the page's half of its 32-token block):
                      uint32 word j = bf16 Delta | bf16 z << 16 of channel 64 h + j.

Window block (16 token slots, bf16), 2 * 16 * 128 elements:
  [0, 2048)           K, row-major: element 128 t + c.
  [2048, 4096)        V: element 2048 + 32 (16 (t // 4) + c // 8) + 4 (c % 8) + t % 4.
"""

import numpy as np

D = 128
PAGE = 16


def page_head_bytes(group):
    return 1024 + 128 * (D // group)


def pack_k_codes(codes):
    """codes uint8 [16, 128] -> uint32 [128] (token-major K code words)."""
    c = np.asarray(codes, dtype=np.uint32).reshape(PAGE, 8, 16)
    words = np.zeros((PAGE, 8), dtype=np.uint32)
    for i in range(16):
        words |= c[:, :, i] << np.uint32(2 * i)
    return words.reshape(-1)


def pack_v_codes(codes):
    """codes uint8 [16, 128] -> uint32 [128] (V code words, see module doc)."""
    c = np.asarray(codes, dtype=np.uint32)
    words = np.zeros(128, dtype=np.uint32)
    for a in range(4):
        for m in range(16):
            for e in range(2):
                u = 2 * (16 * a + m) + e
                t0 = 4 * a + 2 * e
                w = np.uint32(0)
                for j in range(8):
                    w |= c[t0, 8 * m + j] << np.uint32(2 * j)
                    w |= c[t0 + 1, 8 * m + j] << np.uint32(16 + 2 * j)
                words[u] = w
    return words


def pack_params(s16, z16):
    """s16, z16 uint16 [16, ng] -> uint32 [ng * 16] ordered (group, slot)."""
    s = np.asarray(s16, dtype=np.uint32)
    z = np.asarray(z16, dtype=np.uint32)
    return (s | (z << np.uint32(16))).T.reshape(-1)


def pack_page_head(kc, vc, ks, kz, vs, vz, group):
    """One page-head block as uint8 [PB] from per-slot codes and params."""
    ng = D // group
    out = np.zeros(page_head_bytes(group) // 4, dtype=np.uint32)
    out[0:128] = pack_k_codes(kc)
    out[128:256] = pack_v_codes(vc)
    out[256:256 + 16 * ng] = pack_params(ks, kz)
    out[256 + 16 * ng:256 + 32 * ng] = pack_params(vs, vz)
    return out.view(np.uint8)


OTS_PAGE_HEAD_BYTES = 1568


def pack_ots_page_head(kc, vc, ks16, kd16, kz16, vs, vz, group=32):
    """One OScaR page-head block as uint8 [1568]: codes [16, 128], token scales
    [16], the page's 64 channel (Delta, z) pairs, value params [16, 4]."""
    assert group == 32
    out = np.zeros(OTS_PAGE_HEAD_BYTES // 4, dtype=np.uint32)
    out[0:128] = pack_k_codes(kc)
    out[128:256] = pack_v_codes(vc)
    out[256:320] = pack_params(vs, vz)
    ts = np.asarray(ks16, dtype=np.uint32).reshape(PAGE)
    out[320:328] = ts[0::2] | (ts[1::2] << np.uint32(16))
    out[328:392] = (np.asarray(kd16, dtype=np.uint32) |
                    (np.asarray(kz16, dtype=np.uint32) << np.uint32(16)))
    return out.view(np.uint8)


def unpack_ots_page_head(block):
    """Inverse of ``pack_ots_page_head``: (kc, vc, ks16, kd16, kz16, vs, vz)."""
    w = np.ascontiguousarray(block).view(np.uint32)
    kc, vc, _, _, vs, vz = unpack_page_head(np.concatenate([block[:1024], np.zeros(256, np.uint8),
                                                            block[1024:1280]]), 32)
    ts = np.empty(PAGE, np.uint16)
    ts[0::2] = w[320:328] & 0xFFFF
    ts[1::2] = w[320:328] >> 16
    cp = w[328:392]
    return kc, vc, ts, (cp & 0xFFFF).astype(np.uint16), (cp >> 16).astype(np.uint16), vs, vz


def pack_page_heads(kc, vc, ks, kz, vs, vz, group):
    """Many page-head blocks at once: uint8 [N, PB] from codes [N, 16, 128] and
    params [N, 16, ng].  The same word layout as ``pack_page_head``, written
    with array operations so whole caches can be packed quickly; the tests
    check it against ``pack_page_head`` block by block."""
    kc = np.asarray(kc, dtype=np.uint32)
    vc = np.asarray(vc, dtype=np.uint32)
    n = kc.shape[0]
    ng = D // group
    out = np.zeros((n, page_head_bytes(group) // 4), dtype=np.uint32)
    # K: word (8 t + w), channel 16 w + i at bits 2i
    kk = kc.reshape(n, PAGE, 8, 16)
    sh = (2 * np.arange(16, dtype=np.uint32))
    out[:, 0:128] = np.bitwise_or.reduce(kk << sh, axis=3).reshape(n, 128)
    # V: word 2 (16 a + m) + e, slot 4a + 2e + s, channel 8m + j at bits 16 s + 2j
    vv = vc.reshape(n, 4, 2, 2, 16, 8)                      # [n, a, e, s, m, j]
    shv = (16 * np.arange(2, dtype=np.uint32))[:, None, None] + (2 * np.arange(8, dtype=np.uint32))
    words = np.bitwise_or.reduce(vv << shv, axis=(3, 5))   # [n, a, e, m]
    out[:, 128:256] = words.transpose(0, 1, 3, 2).reshape(n, 128)
    # params: word (16 gr + t) = scale | zero << 16
    def params(s16, z16):
        s = np.asarray(s16, dtype=np.uint32)
        z = np.asarray(z16, dtype=np.uint32)
        return (s | (z << np.uint32(16))).transpose(0, 2, 1).reshape(n, 16 * ng)
    out[:, 256:256 + 16 * ng] = params(ks, kz)
    out[:, 256 + 16 * ng:256 + 32 * ng] = params(vs, vz)
    return out.view(np.uint8)


def unpack_page_head(block, group):
    """Inverse of ``pack_page_head``: (kc, vc, ks, kz, vs, vz)."""
    ng = D // group
    w = np.ascontiguousarray(block).view(np.uint32)
    kc = np.zeros((PAGE, D), dtype=np.uint8)
    kw = w[0:128].reshape(PAGE, 8)
    for t in range(PAGE):
        for c in range(D):
            kc[t, c] = (int(kw[t, c // 16]) >> (2 * (c % 16))) & 3
    vc = np.zeros((PAGE, D), dtype=np.uint8)
    vw = w[128:256]
    for a in range(4):
        for m in range(16):
            for e in range(2):
                word = int(vw[2 * (16 * a + m) + e])
                for j in range(8):
                    vc[4 * a + 2 * e, 8 * m + j] = (word >> (2 * j)) & 3
                    vc[4 * a + 2 * e + 1, 8 * m + j] = (word >> (16 + 2 * j)) & 3
    kp = w[256:256 + 16 * ng].reshape(ng, PAGE).T
    vp = w[256 + 16 * ng:256 + 32 * ng].reshape(ng, PAGE).T
    return (kc, vc, (kp & 0xFFFF).astype(np.uint16), (kp >> 16).astype(np.uint16),
            (vp & 0xFFFF).astype(np.uint16), (vp >> 16).astype(np.uint16))


def v_window_index(t, c):
    """Element index of V (slot t, channel c) inside a window block's V half."""
    return 32 * (16 * (t // 4) + c // 8) + 4 * (c % 8) + t % 4


def pack_window_block(k_rows, v_rows):
    """k_rows, v_rows bf16 bits [16, 128] -> uint16 [4096] window block."""
    out = np.zeros(2 * PAGE * D, dtype=np.uint16)
    out[:PAGE * D] = np.asarray(k_rows, dtype=np.uint16).reshape(-1)
    t = np.arange(PAGE)[:, None]
    c = np.arange(D)[None, :]
    out[PAGE * D + v_window_index(t, c)] = np.asarray(v_rows, dtype=np.uint16)
    return out


def unpack_window_block(block):
    """Inverse of ``pack_window_block``: (k_rows, v_rows) bf16 bits [16, 128]."""
    block = np.asarray(block, dtype=np.uint16)
    k = block[:PAGE * D].reshape(PAGE, D).copy()
    t = np.arange(PAGE)[:, None]
    c = np.arange(D)[None, :]
    v = block[PAGE * D + v_window_index(t, c)]
    return k, v
