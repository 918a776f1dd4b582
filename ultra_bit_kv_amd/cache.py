"""Thin Python wrapper over the liboscar_kv C ABI.

torch provides device memory and the current HIP stream; every step of the
hot path runs in the library's kernels.  The functions here only marshal
arguments (pointers, sizes, host/device copies of the per-sequence arrays).
"""

import ctypes

import numpy as np
import torch

from ._lib import Bf16Cache, KvCache, KvConfig, check, lib, MAX_KV_HEADS

D = 128
PAGE = 16


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _host_i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _hp(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def current_stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def as_bf16(x, device="cuda"):
    """bf16 bits (numpy uint16) or a bf16 tensor -> contiguous bf16 device tensor."""
    if isinstance(x, torch.Tensor):
        assert x.dtype == torch.bfloat16
        return x.to(device).contiguous()
    a = np.ascontiguousarray(np.asarray(x, dtype=np.uint16))
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)


def bf16_bits(t):
    """bf16 tensor -> numpy uint16 bit patterns (host)."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class SeqBatch:
    """Host and device copies of the per-sequence arrays of one call."""

    def __init__(self, slots, lens, n_new=None, device="cuda"):
        self.slots = _host_i32(slots)
        self.lens = _host_i32(lens)
        self.n = len(self.slots)
        self.d_slots = torch.from_numpy(self.slots).to(device)
        self.d_lens = torch.from_numpy(self.lens).to(device)
        if n_new is not None:
            self.cu_new = _host_i32(np.concatenate([[0], np.cumsum(np.asarray(n_new, np.int64))]))
            self.d_cu_new = torch.from_numpy(self.cu_new).to(device)
        else:
            self.cu_new = None
            self.d_cu_new = None


class OscarKVCache:
    """Device buffers of one INT2 KV cache (one layer) and the calls on it."""

    def __init__(self, *, num_q_heads, num_kv_heads, group_size, s_sink, s_keep, s_flush,
                 max_seqs, max_pages_per_seq, num_pages, clip_k, clip_v, r_k, r_v, block_table,
                 r_q=None, out_rotated=False, rotation=0, key_mode=0, device="cuda"):
        """rotation: 0 uses the dense per-head r_k / r_v (/ r_q); 1 and 2 are the
        structured R = H / sqrt(128) and H P_br / sqrt(128), which take
        r_k = r_v = r_q = None.  key_mode: 0 the per-token clipped key groups,
        1 the OScaR token scale with per-channel key blocks (group_size 32)."""
        cfg = KvConfig()
        cfg.head_dim = D
        cfg.num_q_heads = num_q_heads
        cfg.num_kv_heads = num_kv_heads
        cfg.group_size = group_size
        cfg.page_size = PAGE
        cfg.s_sink, cfg.s_keep, cfg.s_flush = s_sink, s_keep, s_flush
        cfg.max_seqs = max_seqs
        cfg.max_pages_per_seq = max_pages_per_seq
        cfg.num_pages = num_pages
        cfg.key_mode = int(key_mode)
        ck = np.asarray(clip_k, np.float32)
        cv = np.asarray(clip_v, np.float32)
        assert ck.shape == (num_kv_heads,) and cv.shape == (num_kv_heads,) and num_kv_heads <= MAX_KV_HEADS
        for h in range(num_kv_heads):
            cfg.clip_k[h] = float(ck[h])
            cfg.clip_v[h] = float(cv[h])
        L = lib()
        check(L.oscar_check_config(ctypes.byref(cfg)), "oscar_check_config")
        self.cfg = cfg
        self.device = device
        self.pages = torch.zeros(max(1, L.oscar_pages_bytes(ctypes.byref(cfg))), dtype=torch.uint8,
                                 device=device)
        self.win = torch.zeros(L.oscar_win_bytes(ctypes.byref(cfg)) // 2, dtype=torch.int16,
                               device=device)
        bt = np.zeros((max_seqs, max(1, max_pages_per_seq)), np.int32)
        src = np.asarray(block_table, np.int32)
        bt[:src.shape[0], :src.shape[1]] = src
        self.block_table = torch.from_numpy(bt).to(device)
        def dev(r):
            return (torch.as_tensor(np.asarray(r, np.float32)).to(device).contiguous()
                    if r is not None else None)

        self.rotation = int(rotation)
        self.r_k, self.r_v = dev(r_k), dev(r_v)
        # optional query transform (a non-orthogonal key transform T pairs with T^-T)
        self.r_q = dev(r_q)
        if self.rotation == 0:
            assert self.r_k.shape == (num_kv_heads, D, D) and self.r_v.shape == (num_kv_heads, D, D)
            assert self.r_q is None or self.r_q.shape == (num_kv_heads, D, D)

        def ptr(t):
            return t.data_ptr() if t is not None else None

        self.st = KvCache(cfg, self.pages.data_ptr(), self.block_table.data_ptr(),
                          self.win.data_ptr(), ptr(self.r_k), ptr(self.r_v), ptr(self.r_q),
                          1 if out_rotated else 0, self.rotation)
        self.workspace = None
        self.ring_capacity = L.oscar_ring_capacity(ctypes.byref(cfg))
        self.max_seq_len = L.oscar_max_seq_len(ctypes.byref(cfg))
        self.page_head_bytes = L.oscar_config_page_head_bytes(ctypes.byref(cfg))
        self.key_mode = int(key_mode)

    @property
    def hq(self):
        return self.cfg.num_q_heads

    @property
    def hkv(self):
        return self.cfg.num_kv_heads

    def workspace_for(self, n_seqs, max_new_tokens):
        need = lib().oscar_workspace_size(ctypes.byref(self.cfg), int(n_seqs), int(max_new_tokens))
        if self.workspace is None or self.workspace.numel() < need:
            self.workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self.workspace

    # ------------------------------------------------------------------ calls
    def append(self, batch, k, v, q=None, q_rot=None, k_rot=None, v_rot=None):
        """oscar_rotate_quant_append for a SeqBatch built with n_new."""
        n_tok = int(batch.cu_new[-1])
        k = as_bf16(k, self.device)
        v = as_bf16(v, self.device)
        assert k.shape == (n_tok, self.hkv, D) and v.shape == (n_tok, self.hkv, D)
        if q is not None:
            q = as_bf16(q, self.device)
            assert q.shape == (n_tok, self.hq, D)
        ws = self.workspace_for(batch.n, n_tok)
        st = lib().oscar_rotate_quant_append(
            ctypes.byref(self.st), batch.n, _hp(batch.slots), _hp(batch.lens), _hp(batch.cu_new),
            _p(batch.d_slots), _p(batch.d_lens), _p(batch.d_cu_new), _p(k), _p(v), _p(q),
            _p(q_rot), _p(k_rot), _p(v_rot), _p(ws), ws.numel(), current_stream())
        check(st, "oscar_rotate_quant_append")
        return q_rot

    def append_tokens(self, slots, len_before, n_new, k, v, q=None, want_rot=False):
        """Convenience form: builds the SeqBatch and output buffers."""
        batch = SeqBatch(slots, len_before, n_new, self.device)
        n_tok = int(batch.cu_new[-1])
        q_rot = (torch.empty((n_tok, self.hq, D), dtype=torch.bfloat16, device=self.device)
                 if q is not None else None)
        k_rot = v_rot = None
        if want_rot:
            k_rot = torch.empty((n_tok, self.hkv, D), dtype=torch.bfloat16, device=self.device)
            v_rot = torch.empty_like(k_rot)
        self.append(batch, k, v, q, q_rot, k_rot, v_rot)
        return q_rot, k_rot, v_rot

    def decode(self, batch, q_rot, out=None):
        """oscar_int2_decode_attn: fp32 [n, Hq, 128] in the original basis (the
        rotated basis when the cache was built with out_rotated)."""
        assert q_rot.dtype == torch.bfloat16 and q_rot.shape == (batch.n, self.hq, D)
        if out is None:
            out = torch.empty((batch.n, self.hq, D), dtype=torch.float32, device=self.device)
        ws = self.workspace_for(batch.n, 0)
        st = lib().oscar_int2_decode_attn(
            ctypes.byref(self.st), batch.n, _hp(batch.slots), _hp(batch.lens), _p(batch.d_slots),
            _p(batch.d_lens), _p(q_rot), _p(out), _p(ws), ws.numel(), current_stream())
        check(st, "oscar_int2_decode_attn")
        return out

    def decode_noalloc(self, batch, q_rot, out):
        """oscar_int2_decode_attn_noalloc: the same decode with the split
        records in the library's fixed device scratch (no workspace)."""
        assert q_rot.dtype == torch.bfloat16 and q_rot.shape == (batch.n, self.hq, D)
        assert out.dtype == torch.float32 and out.shape == (batch.n, self.hq, D)
        st = lib().oscar_int2_decode_attn_noalloc(
            ctypes.byref(self.st), batch.n, _hp(batch.slots), _hp(batch.lens), _p(batch.d_slots),
            _p(batch.d_lens), _p(q_rot), _p(out), current_stream())
        check(st, "oscar_int2_decode_attn_noalloc")
        return out

    def decode_partials(self, batch, q_rot):
        """oscar_int2_decode_partials: the split launch of a decode step."""
        assert q_rot.dtype == torch.bfloat16 and q_rot.shape == (batch.n, self.hq, D)
        ws = self.workspace_for(batch.n, 0)
        st = lib().oscar_int2_decode_partials(
            ctypes.byref(self.st), batch.n, _hp(batch.slots), _hp(batch.lens), _p(batch.d_slots),
            _p(batch.d_lens), _p(q_rot), _p(ws), ws.numel(), current_stream())
        check(st, "oscar_int2_decode_partials")

    def decode_merge(self, batch, out=None):
        """oscar_int2_decode_merge: the merge launch of the same decode step."""
        if out is None:
            out = torch.empty((batch.n, self.hq, D), dtype=torch.float32, device=self.device)
        ws = self.workspace_for(batch.n, 0)
        st = lib().oscar_int2_decode_merge(
            ctypes.byref(self.st), batch.n, _hp(batch.slots), _hp(batch.lens), _p(batch.d_slots),
            _p(batch.d_lens), _p(out), _p(ws), ws.numel(), current_stream())
        check(st, "oscar_int2_decode_merge")
        return out

    def prefill_attn(self, batch, q_rot, k_rot, v_rot, out=None):
        """oscar_int2_prefill_attn for the chunk of an append made with ``batch``
        (a SeqBatch built with n_new): fp32 [n_tok, Hq, 128]."""
        n_tok = int(batch.cu_new[-1])
        assert q_rot.dtype == torch.bfloat16 and q_rot.shape == (n_tok, self.hq, D)
        assert k_rot.dtype == torch.bfloat16 and k_rot.shape == (n_tok, self.hkv, D)
        assert v_rot.dtype == torch.bfloat16 and v_rot.shape == (n_tok, self.hkv, D)
        if out is None:
            out = torch.empty((n_tok, self.hq, D), dtype=torch.float32, device=self.device)
        st = lib().oscar_int2_prefill_attn(
            ctypes.byref(self.st), batch.n, _hp(batch.slots), _hp(batch.lens), _hp(batch.cu_new),
            _p(batch.d_slots), _p(batch.d_lens), _p(batch.d_cu_new), _p(q_rot), _p(k_rot),
            _p(v_rot), _p(out), current_stream())
        check(st, "oscar_int2_prefill_attn")
        return out

    def dequant(self, slot, seq_len, t0, t1):
        """oscar_dequant: decoded (k, v) fp32 [t1 - t0, Hkv, 128], rotated basis."""
        k = torch.empty((max(0, t1 - t0), self.hkv, D), dtype=torch.float32, device=self.device)
        v = torch.empty_like(k)
        st = lib().oscar_dequant(ctypes.byref(self.st), slot, seq_len, t0, t1, _p(k), _p(v),
                                 current_stream())
        check(st, "oscar_dequant")
        return k, v

    # ------------------------------------------------------------- accessors
    def page_head(self, phys, h):
        """Raw bytes of one page-head block (host numpy)."""
        pb = self.page_head_bytes
        off = (phys * self.hkv + h) * pb
        return self.pages[off:off + pb].cpu().numpy()

    def window_blocks(self, slot, h):
        """Raw window blocks of one cache row and KV head: uint16 [NB, 4096]."""
        sb = -(-self.cfg.s_sink // PAGE)
        nb = sb + self.ring_capacity // PAGE
        per = 2 * PAGE * D
        off = (slot * self.hkv + h) * nb * per
        return self.win[off:off + nb * per].cpu().numpy().view(np.uint16).reshape(nb, per)


class BF16PagedCache:
    """Device buffers of a plain BF16 paged KV cache (one layer) and
    oscar_bf16_paged_decode_attn on it: the uncompressed comparison point.

    ``pages`` is bf16 [num_pages, Hkv, 2, 16, 128] (part 0 = K rows of the
    page's 16 slots, part 1 = V rows); the caller writes it.  Token p of a
    row lives in logical page p // 16, slot p % 16."""

    def __init__(self, *, num_q_heads, num_kv_heads, max_seqs, max_pages_per_seq, num_pages,
                 block_table, device="cuda"):
        self.device = device
        self.pages = torch.zeros((max(1, num_pages), num_kv_heads, 2, PAGE, D), dtype=torch.bfloat16,
                                 device=device)
        bt = np.zeros((max_seqs, max(1, max_pages_per_seq)), np.int32)
        src = np.asarray(block_table, np.int32)
        bt[:src.shape[0], :src.shape[1]] = src
        self.block_table = torch.from_numpy(bt).to(device)
        self.st = Bf16Cache(D, num_q_heads, num_kv_heads, PAGE, max_seqs, max_pages_per_seq,
                            num_pages, self.pages.data_ptr(), self.block_table.data_ptr())
        self.hq, self.hkv = num_q_heads, num_kv_heads
        self.workspace = None

    def workspace_for(self, n_seqs):
        need = lib().oscar_bf16_workspace_size(ctypes.byref(self.st), int(n_seqs))
        if need == 0:
            check(-2, "oscar_bf16_workspace_size")
        if self.workspace is None or self.workspace.numel() < need:
            self.workspace = torch.zeros(need, dtype=torch.uint8, device=self.device)
        return self.workspace

    def decode(self, batch, q, out=None):
        """oscar_bf16_paged_decode_attn: fp32 [n, Hq, 128]."""
        assert q.dtype == torch.bfloat16 and q.shape == (batch.n, self.hq, D)
        if out is None:
            out = torch.empty((batch.n, self.hq, D), dtype=torch.float32, device=self.device)
        ws = self.workspace_for(batch.n)
        st = lib().oscar_bf16_paged_decode_attn(
            ctypes.byref(self.st), batch.n, _hp(batch.slots), _hp(batch.lens), _p(batch.d_slots),
            _p(batch.d_lens), _p(q), _p(out), _p(ws), ws.numel(), current_stream())
        check(st, "oscar_bf16_paged_decode_attn")
        return out
