"""ctypes view of liboscar_kv (the C ABI in include/oscar_kv.h).

The library is loaded after torch so that both bind to the one HIP runtime
torch already has in the process.  There is no fallback: if the shared
library is missing, loading fails loudly.
"""

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime first)

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liboscar_kv.so")
MAX_KV_HEADS = 64

c_i32 = ctypes.c_int32
c_i64 = ctypes.c_int64
c_size = ctypes.c_size_t
c_p = ctypes.c_void_p


class KvConfig(ctypes.Structure):
    _fields_ = [
        ("head_dim", c_i32), ("num_q_heads", c_i32), ("num_kv_heads", c_i32),
        ("group_size", c_i32), ("page_size", c_i32), ("s_sink", c_i32), ("s_keep", c_i32),
        ("s_flush", c_i32), ("max_seqs", c_i32), ("max_pages_per_seq", c_i32),
        ("num_pages", c_i32), ("clip_k", ctypes.c_float * MAX_KV_HEADS),
        ("clip_v", ctypes.c_float * MAX_KV_HEADS), ("key_mode", c_i32),
    ]


# key modes of KvConfig.key_mode (oscar_key_mode in oscar_kv.h)
KEYS_CLIP, KEYS_OTS = 0, 1


class KvCache(ctypes.Structure):
    _fields_ = [("cfg", KvConfig), ("pages", c_p), ("block_table", c_p), ("win", c_p),
                ("r_k", c_p), ("r_v", c_p), ("r_q", c_p), ("out_rotated", c_i32),
                ("rotation", c_i32)]


# rotation kinds of KvCache.rotation (oscar_rotation in oscar_kv.h)
ROT_DENSE, ROT_HADAMARD, ROT_HADAMARD_BITREV = 0, 1, 2


class Bf16Cache(ctypes.Structure):
    _fields_ = [("head_dim", c_i32), ("num_q_heads", c_i32), ("num_kv_heads", c_i32),
                ("page_size", c_i32), ("max_seqs", c_i32), ("max_pages_per_seq", c_i32),
                ("num_pages", c_i32), ("pages", c_p), ("block_table", c_p)]


STATUS = {0: "OSCAR_OK", -1: "OSCAR_ERR_NULL", -2: "OSCAR_ERR_SHAPE", -3: "OSCAR_ERR_GROUP",
          -4: "OSCAR_ERR_CLIP", -5: "OSCAR_ERR_WINDOW", -6: "OSCAR_ERR_CAPACITY",
          -7: "OSCAR_ERR_WORKSPACE", -8: "OSCAR_ERR_DEVICE", -9: "OSCAR_ERR_HIP",
          -10: "OSCAR_ERR_ARG"}

_PROTOS = {
    "oscar_check_config": (c_i32, [ctypes.POINTER(KvConfig)]),
    "oscar_page_head_bytes": (c_size, [c_i32]),
    "oscar_config_page_head_bytes": (c_size, [ctypes.POINTER(KvConfig)]),
    "oscar_pages_bytes": (c_size, [ctypes.POINTER(KvConfig)]),
    "oscar_win_bytes": (c_size, [ctypes.POINTER(KvConfig)]),
    "oscar_ring_capacity": (c_i32, [ctypes.POINTER(KvConfig)]),
    "oscar_max_seq_len": (c_i64, [ctypes.POINTER(KvConfig)]),
    "oscar_workspace_size": (c_size, [ctypes.POINTER(KvConfig), c_i32, c_i64]),
    "oscar_rotate_quant_append": (c_i32, [ctypes.POINTER(KvCache), c_i32, c_p, c_p, c_p, c_p, c_p,
                                          c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_size, c_p]),
    "oscar_int2_decode_attn": (c_i32, [ctypes.POINTER(KvCache), c_i32, c_p, c_p, c_p, c_p, c_p, c_p,
                                       c_p, c_size, c_p]),
    "oscar_int2_decode_attn_noalloc": (c_i32, [ctypes.POINTER(KvCache), c_i32, c_p, c_p, c_p, c_p,
                                               c_p, c_p, c_p]),
    "oscar_int2_decode_partials": (c_i32, [ctypes.POINTER(KvCache), c_i32, c_p, c_p, c_p, c_p, c_p,
                                           c_p, c_size, c_p]),
    "oscar_int2_decode_merge": (c_i32, [ctypes.POINTER(KvCache), c_i32, c_p, c_p, c_p, c_p, c_p,
                                        c_p, c_size, c_p]),
    "oscar_int2_prefill_attn": (c_i32, [ctypes.POINTER(KvCache), c_i32, c_p, c_p, c_p, c_p, c_p,
                                        c_p, c_p, c_p, c_p, c_p, c_p]),
    "oscar_dequant": (c_i32, [ctypes.POINTER(KvCache), c_i32, c_i32, c_i32, c_i32, c_p, c_p, c_p]),
    "oscar_bf16_workspace_size": (c_size, [ctypes.POINTER(Bf16Cache), c_i32]),
    "oscar_bf16_paged_decode_attn": (c_i32, [ctypes.POINTER(Bf16Cache), c_i32, c_p, c_p, c_p, c_p,
                                             c_p, c_p, c_p, c_size, c_p]),
    "oscar_status_string": (ctypes.c_char_p, [c_i32]),
    "oscar_round_f64_host": (c_i32, [c_i32, c_p, c_p, c_i64]),
    "oscar_read_probe": (c_i32, [c_p, c_size, c_p, c_i32, c_i32, c_p, c_i32, c_i32, c_p]),
}

_LIB = None


class OscarError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        msg = _LIB.oscar_status_string(status).decode() if _LIB is not None else ""
        super().__init__(f"{what}: {STATUS.get(status, status)} ({msg})")


def lib():
    """The loaded liboscar_kv (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m ultra_bit_kv_amd.build` (there is no fallback path)")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _PROTOS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _LIB = h
    return _LIB


def check(status, what):
    if status != 0:
        raise OscarError(status, what)
