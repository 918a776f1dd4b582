"""Parity at the workloads' full sizes, through the C ABI, in the launch
configuration the benchmark times: whole caches are built on the GPU and
decoded; sampled (sequence, KV head) outputs are checked one by one against
the fp64 oracle, and sampled cache rows bit for bit."""
import numpy as np
import pytest
import torch

from synth import get
from tests.oscar_testlib import (compare_attention, fill, make_cache, oracle_decode,
                                 oracle_head)

pytestmark = pytest.mark.gpu


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _check_decode(w, cache, q_rot, lens, samples):
    from ultra_bit_kv_amd import SeqBatch
    out = cache.decode(SeqBatch(range(len(lens)), lens), q_rot).cpu().numpy()
    r_k, r_v = cache.host_r
    for i, h in samples:
        want = oracle_decode(w, i, h, int(lens[i]), r_k, r_v)
        err, rel, ok = compare_attention(out[i, h * w.g:(h + 1) * w.g], want)
        print(f"[case] {w.name} seq {i} head {h} len {int(lens[i])} max_abs={err:.3e} rel_l2={rel:.3e}",
              flush=True)
        assert ok, (i, h, err, rel)


@pytest.mark.parametrize("name,samples,rotation", [
    ("c2_qwen3_8b_bs1", [(0, 0), (0, 5)], 0),
    ("c2_qwen3_8b_bs1", [(0, 3)], 1),        # structured H / sqrt(128): two-level merge un-rotation
    ("c4_long_bs1", [(0, 2)], 0),
])
def test_fullsize_long_context(name, samples, rotation):
    w = get(name)
    lens = [int(x) for x in w.lengths_after()]
    _case(f"{name} full size, lens {lens}, rotation {rotation}")
    cache = make_cache(w, lens, rotation=rotation)
    q_rot = fill(cache, w, lens, chunk=8192)
    _check_decode(w, cache, q_rot, lens, samples)


@pytest.mark.parametrize("rotation", [0, 2])
def test_fullsize_bs64(rotation):
    """The benchmark's workload and launch plan: 64 sequences, U[4096, 8192];
    with the dense per-head rotation and the structured H P_br / sqrt(128)."""
    w = get("c3_bs64")
    lens = [int(x) for x in w.lengths_after()]
    _case(f"c3_bs64 full size, {len(lens)} sequences, rotation {rotation}")
    cache = make_cache(w, lens, max_seqs=len(lens), rotation=rotation)
    q_rot = fill(cache, w, lens, chunk=8192)
    rng = np.random.default_rng(11)
    seqs = [int(np.argmax(lens)), int(np.argmin(lens))] + list(rng.choice(len(lens), 2, replace=False))
    _check_decode(w, cache, q_rot, lens, [(int(i), int(rng.integers(w.hkv))) for i in seqs])


def test_fullsize_serving_step():
    """The Qwen3-32B-shaped serving step: one append call carrying 256 decode
    tokens (8 of them trigger a 256-token flush) and 16 fresh 2048-token
    prefill chunks, then the decode of the 256 sequences."""
    from ultra_bit_kv_amd import SeqBatch
    w = get("c5_qwen3_32b_step")
    lens = [int(x) for x in w.lengths_after()]                # after the step
    n_dec, n_pre, plen = len(lens), w.prefill_chunks, w.prefill_len
    _case(f"c5 full size: {n_dec} decode sequences + {n_pre} x {plen} prefill")
    cache = make_cache(w, lens + [plen] * n_pre, max_seqs=n_dec + n_pre)
    fill(cache, w, lens, chunk=4096, last_step=False)          # positions [0, L - 1)
    # the step: decode tokens of sequences 0..255, prefill of sequences 256..271
    slots = list(range(n_dec + n_pre))
    before = [L - 1 for L in lens] + [0] * n_pre
    n_new = [1] * n_dec + [plen] * n_pre
    k = np.concatenate([w.keys(i, b, b + n) for i, b, n in zip(slots, before, n_new)])
    v = np.concatenate([w.values(i, b, b + n) for i, b, n in zip(slots, before, n_new)])
    q = np.concatenate([w.queries(i, b, b + n) for i, b, n in zip(slots, before, n_new)])
    q_rot, _, _ = cache.append_tokens(slots, before, n_new, k, v, q)
    torch.cuda.synchronize()
    flushing = [i for i, L in enumerate(lens) if L == w.lengths[3]]
    assert len(flushing) == 8
    _check_decode(w, cache, q_rot[:n_dec], lens, [(flushing[0], 1), (flushing[5], 6), (3, 4)])
    # a prefilled sequence's cache rows, bit for bit
    r_k, r_v = cache.host_r
    seq, h = n_dec + 7, 2
    kd, vd = cache.dequant(seq, plen, 0, plen)
    hc = oracle_head(w, seq, h, plen, r_k, r_v)
    kw, vw = hc.dequant_f32()
    assert np.array_equal(kd[:, h].cpu().numpy().view(np.uint32), kw.view(np.uint32))
    assert np.array_equal(vd[:, h].cpu().numpy().view(np.uint32), vw.view(np.uint32))
