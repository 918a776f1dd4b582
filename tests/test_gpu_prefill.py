"""GPU parity of the chunked-prefill attention (oscar_int2_prefill_attn)
against the oracle's O6 (``oracle/prefill.py``), through the C ABI.

Each case builds the prefix of every sequence with the library's own append
path, appends one chunk per sequence with its queries (the call whose
q_rot / k_rot / v_rot outputs feed the prefill), then compares every chunk
row's output with the oracle, which builds its cache from the same seeded
inputs.  Bar: max-abs <= 2e-3 and rel-L2 <= 1e-3 per (sequence, KV head),
the attention bar of the decode path (keys and values are staged in fp16,
sums in fp32).

Cases: prefixes that span sink, INT2 and ring rows; a chunk whose append
flushes prefix ring rows to INT2; fresh prefills (no prefix) whose rows the
append quantizes; chunks longer than the ring; ragged chunks in one call
(tile tails, an empty chunk); G = 32 / 64 / 128; GQA 1, 4, 8, 16; the
rotated-basis output; S_sink = 0.
"""

import numpy as np
import pytest

from oracle import prefill, rotate
from oracle.rounding import bf16_bits_to_f64
from synth import get
from tests.oscar_testlib import make_cache, fill, oracle_head, compare_attention

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ultra_bit_kv_amd import lib
    lib()


def run_case(w, lbs, ns, out_rotated=False, identity=False, sample=None, rotation=0):
    from ultra_bit_kv_amd import SeqBatch
    print(f"[case] {w.name} G={w.group} Hq/Hkv={w.hq}/{w.hkv} windows=({w.s_sink},{w.s_keep},"
          f"{w.s_flush}) len_before={lbs} n_new={ns} out_rotated={out_rotated} "
          f"rotation={rotation}", flush=True)
    lens = [lb + n for lb, n in zip(lbs, ns)]
    cache = make_cache(w, [max(1, L) for L in lens], identity=identity, out_rotated=out_rotated,
                       rotation=rotation)
    fill(cache, w, [lb + 1 for lb in lbs], chunk=512, last_step=False)    # positions [0, lb)
    idx = list(range(len(lbs)))
    k = np.concatenate([w.keys(i, lbs[i], lens[i]) for i in idx])
    v = np.concatenate([w.values(i, lbs[i], lens[i]) for i in idx])
    q = np.concatenate([w.queries(i, lbs[i], lens[i]) for i in idx])
    q_rot, k_rot, v_rot = cache.append_tokens(idx, lbs, ns, k, v, q, want_rot=True)
    out = cache.prefill_attn(SeqBatch(idx, lbs, ns), q_rot, k_rot, v_rot).cpu().numpy()
    torch.cuda.synchronize()
    r_k, r_v = cache.host_r
    cu = np.concatenate([[0], np.cumsum(ns)])
    worst = 0.0
    for i in idx:
        if ns[i] == 0:
            continue
        qr = bf16_bits_to_f64(rotate.rotate_heads_to_bf16(w.queries(i, lbs[i], lens[i]), r_k, g=w.g))
        rows = None if sample is None else sorted(set(range(0, ns[i], sample)) | {ns[i] - 1})
        for h in range(w.hkv):
            hc = oracle_head(w, i, h, lens[i], r_k, r_v)
            want = prefill.prefill_head(qr[:, h * w.g:(h + 1) * w.g], hc, lbs[i],
                                        r_v=None if out_rotated else r_v[h], rows=rows)
            got = out[cu[i]:cu[i + 1], h * w.g:(h + 1) * w.g]
            sel = slice(None) if rows is None else rows
            err, rel, ok = compare_attention(got[sel], want[sel])
            worst = max(worst, err)
            assert ok, (i, h, err, rel)
    print(f"[case] ok max_abs={worst:.3e}", flush=True)


def test_prefix_with_flush_c1():
    # 700-token prefix (sink 4, INT2, ring), a 100-token chunk whose append
    # flushes earlier ring rows to INT2
    run_case(get("c1_tiny"), [700], [100])


def test_fresh_prefill_quantized_chunk_rows():
    # no prefix: the append moves most chunk rows to INT2, the prefill reads
    # them in bf16; 300 rows x 4 heads = 19 tiles (ragged)
    run_case(get("c1_tiny"), [0], [301])


def test_prefix_in_windows_bf16_rows_only():
    # prefixes still held by the sink and the ring (no INT2 row below any
    # chunk): every key and value of the call is a bf16 row; ragged chunks,
    # stage boundaries inside the sink, ring and chunk rows
    w = get("c1_tiny").scaled(n_seqs=3, lengths=("list", (120, 77, 120)))
    run_case(w, [100, 3, 60], [20, 74, 60])


def test_chunk_longer_than_ring_identity():
    run_case(get("c1_tiny").scaled(s_keep=40, s_flush=16), [500], [600], identity=True)


@pytest.mark.parametrize("group", [32, 64])
def test_ragged_batch_groups(group):
    # three sequences in one call: GQA 4, 2 KV heads, an empty chunk, tile tails
    w = get("c3_bs64").scaled(n_seqs=4, hq=8, hkv=2, group=group, s_sink=64, s_keep=256,
                              s_flush=16, lengths=("list", (900, 1200, 400, 700)))
    run_case(w, [333, 0, 400, 690], [150, 270, 0, 9])


@pytest.mark.parametrize("hq,hkv", [(16, 2), (2, 2), (32, 2), (24, 2), (12, 4)])
def test_gqa_shapes(hq, hkv):
    # GQA 8 (the Qwen3-32B shape's ratio, G = 128, flush 256), 1, 16, 12 and 3 (row / g by a
    # magic multiplier in the kernel: also g not a power of two)
    w = get("c5_qwen3_32b_step").scaled(n_seqs=2, hq=hq, hkv=hkv, lengths=("list", (800, 900)))
    run_case(w, [530, 640], [130, 77])


@pytest.mark.parametrize("out_rotated", [True])
def test_rotated_output_no_sink(out_rotated):
    w = get("c3_bs64").scaled(n_seqs=1, hq=8, hkv=2, s_sink=0, s_keep=64, s_flush=16,
                              lengths=("list", (500,)))
    run_case(w, [300], [140], out_rotated=out_rotated)


def test_c5_prefill_chunk_sampled():
    # a fresh 2048-token chunk at the Qwen3-32B shape (64 / 8 heads, G = 128,
    # windows 64 / 256 / 256), outputs sampled every 97 rows on 8 KV heads
    w = get("c5_qwen3_32b_step").scaled(n_seqs=1, lengths=("list", (2048,)))
    run_case(w, [0], [2048], sample=97)
