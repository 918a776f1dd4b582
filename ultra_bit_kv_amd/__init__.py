"""liboscar_kv on MI355X: INT2 KV cache with fixed per-head rotation and
clipped asymmetric 2-bit quantization, BF16 sink/recent windows, and split-K
paged GQA decode attention.  The compute runs in the HIP library
(``liboscar_kv.so``, C ABI in ``include/oscar_kv.h``); this package is the
Python binding.
"""

from .cache import BF16PagedCache, OscarKVCache, SeqBatch, as_bf16, bf16_bits  # noqa: F401
from ._lib import lib, OscarError, LIB_PATH  # noqa: F401
