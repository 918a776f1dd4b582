"""GPU parity of the structured rotations R = H / sqrt(128) and
R = H P_br / sqrt(128) (OScaR notes, step one "Canalized Rotation"; OSCAR
summary page, section 5 "Rotation Analysis"), through the C ABI.

The library runs them as an in-register fast Walsh-Hadamard transform and
generates the un-rotation entries; the oracle multiplies by the matrix and
rounds the exact product (``oracle/rotate.py``).  Bars: rotated rows, cache
pages, window rows and dequantized rows bit-exact; attention within the decode
bar (max-abs 2e-3, rel-L2 1e-3).

Cases: the multi-token rotation launch (one and eight 16-token blocks per
work-group, ragged tails), the one-token append launch (decode steps, with
and without flushes), decode over sink + INT2 + ring for the workload shapes,
chunked prefill with un-rotated and rotated-basis outputs.
"""

import numpy as np
import pytest

from oracle import rotate
from synth import get
from tests.oscar_testlib import (make_cache, fill, oracle_head, oracle_q_rot, oracle_decode,
                                 compare_attention)
from tests.test_gpu_parity import small, _check_head
from tests.test_gpu_prefill import run_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ultra_bit_kv_amd import lib
    lib()


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("kind", [1, 2])
@pytest.mark.parametrize("name", ["c1", "c3s", "c5s", "demote1", "oddflush"])
def test_structured_append_bit_exact_and_decode(name, kind):
    from ultra_bit_kv_amd import SeqBatch
    w, lens = small(name)
    print(f"[case] {name} rotation={kind} lens={lens}", flush=True)
    cache = make_cache(w, lens, rotation=kind)
    q_rot = fill(cache, w, lens, chunk=300)
    r_k, r_v = cache.host_r
    out = cache.decode(SeqBatch(range(len(lens)), lens), q_rot)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    qr = _bits(q_rot)
    worst = 0.0
    for i, L in enumerate(lens):
        assert np.array_equal(qr[i], oracle_q_rot(w, i, L, r_k)), i
        for h in range(w.hkv):
            hc = oracle_head(w, i, h, L, r_k, r_v)
            _check_head(cache, w, i, h, L, hc)
            want = oracle_decode(w, i, h, L, r_k, r_v, hc)
            err, rel, ok = compare_attention(out[i, h * w.g:(h + 1) * w.g], want)
            worst = max(worst, err)
            assert ok, (name, kind, i, h, err, rel)
    print(f"[case] {name} rotation={kind} max_abs={worst:.3e}", flush=True)


@pytest.mark.parametrize("kind", [1, 2])
def test_structured_rotated_rows(kind):
    # call 1: chunks of 1100 / 39 / 600 tokens from position 0 (more than 64
    # blocks of 16 rows: eight blocks per work-group, ragged tails); call 2: one
    # token per sequence (the one-token append launch)
    w = get("c3_bs64").scaled(n_seqs=3, hq=8, hkv=2, lengths=("list", (1200, 40, 700)))
    lens = [1200, 40, 700]
    ns = [1100, 39, 600]
    print(f"[case] rotated rows rotation={kind} chunks={ns}", flush=True)
    cache = make_cache(w, lens, rotation=kind)
    had = rotate.Hadamard(128, bitrev=kind == 2)
    for lb, nn in ((0, ns), (ns, [1, 1, 1])):
        lb = [0] * 3 if lb == 0 else lb
        idx = [0, 1, 2]
        k = np.concatenate([w.keys(i, lb[i], lb[i] + nn[i]) for i in idx])
        v = np.concatenate([w.values(i, lb[i], lb[i] + nn[i]) for i in idx])
        q = np.concatenate([w.queries(i, lb[i], lb[i] + nn[i]) for i in idx])
        q_rot, k_rot, v_rot = cache.append_tokens(idx, lb, nn, k, v, q, want_rot=True)
        torch.cuda.synchronize()
        for x, got, heads in ((k, k_rot, w.hkv), (v, v_rot, w.hkv), (q, q_rot, w.hq)):
            want = rotate.rotate_heads_to_bf16(x, [had] * heads)
            assert np.array_equal(_bits(got), want), (kind, nn, heads)


@pytest.mark.parametrize("kind", [1, 2])
def test_structured_prefill(kind):
    run_case(get("c1_tiny"), [700], [100], rotation=kind)
    w = get("c5_qwen3_32b_step").scaled(n_seqs=2, hq=16, hkv=2, lengths=("list", (800, 900)))
    run_case(w, [530, 0], [130, 300], rotation=kind)


def test_structured_rotated_basis_output():
    from oracle import attention
    from oracle.rounding import bf16_bits_to_f64
    from ultra_bit_kv_amd import SeqBatch
    w = get("c3_bs64").scaled(n_seqs=2, hkv=2, hq=8, lengths=("list", (300, 517)))
    lens = [300, 517]
    cache = make_cache(w, lens, rotation=2, out_rotated=True)
    q_rot = fill(cache, w, lens, chunk=128)
    out = cache.decode(SeqBatch([0, 1], lens), q_rot).cpu().numpy()
    r_k, r_v = cache.host_r
    for i, L in enumerate(lens):
        qr = bf16_bits_to_f64(oracle_q_rot(w, i, L, r_k))
        for h in range(w.hkv):
            hc = oracle_head(w, i, h, L, r_k, r_v)
            want = attention.attend(qr[h * w.g:(h + 1) * w.g], hc.k_dec, hc.v_dec)
            err, rel, ok = compare_attention(out[i, h * w.g:(h + 1) * w.g], want)
            assert ok, (i, h, err, rel)
    run_case(get("c1_tiny"), [500], [64], out_rotated=True, rotation=1)
