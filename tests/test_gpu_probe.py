"""The read probe (measurement aid, include/oscar_probe.h) reads every word it
is given exactly once: the XOR of its per-wave sink words equals the XOR of
all 32-bit words of the buffer (sequential sweep) or of the chosen chunks
(gather).  A word read twice would cancel out of the XOR, a skipped one would
be missing."""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _probe(L, buf, nbytes, ids, chunk_bytes, grid):
    sink = torch.zeros(4 * grid, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if ids is None:
        st = L.oscar_read_probe(ctypes.c_void_p(buf.data_ptr()), nbytes, None, 0, 0,
                                ctypes.c_void_p(sink.data_ptr()), grid, 4 * grid, stream)
    else:
        st = L.oscar_read_probe(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                ctypes.c_void_p(ids.data_ptr()), int(ids.numel()), chunk_bytes,
                                ctypes.c_void_p(sink.data_ptr()), grid, 4 * grid, stream)
    assert st == 0
    torch.cuda.synchronize()
    return int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)))


@pytest.mark.parametrize("nbytes, grid", [(1 << 20, 7), (3 * 1024 * 1024 + 5 * 1024, 64),
                                          (1 << 24, 2048), (64 * 1024, 2048)])
def test_sequential_sweep_reads_every_word_once(nbytes, grid):
    from ultra_bit_kv_amd import lib
    L = lib()
    words = np.random.default_rng(nbytes + grid).integers(0, 2**32, nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to("cuda")
    print(f"[case] sequential {nbytes} B grid {grid}", flush=True)
    assert _probe(L, buf, nbytes, None, 0, grid) == int(np.bitwise_xor.reduce(words))


@pytest.mark.parametrize("chunk_kb, grid", [(10, 2048), (1, 3), (17, 64)])
def test_chunk_gather_reads_the_chosen_chunks_once(chunk_kb, grid):
    from ultra_bit_kv_amd import lib
    L = lib()
    cb = chunk_kb * 1024
    n_ch = 300
    nbytes = n_ch * cb
    rng = np.random.default_rng(chunk_kb)
    words = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to("cuda")
    pick = rng.permutation(n_ch)[:200].astype(np.int32)
    pick_dev = np.concatenate([pick, np.array([-1, n_ch, 10**6], dtype=np.int32)])   # skipped ids
    ids = torch.from_numpy(pick_dev).to("cuda")
    want = 0
    per = cb // 4
    for c in pick:
        want ^= int(np.bitwise_xor.reduce(words[c * per:(c + 1) * per]))
    print(f"[case] gather {chunk_kb} KB chunks grid {grid}", flush=True)
    assert _probe(L, buf, nbytes, ids, cb, grid) == want
