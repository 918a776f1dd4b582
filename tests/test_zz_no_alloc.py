"""oscar_int2_decode_attn_noalloc (fixed device scratch, no workspace) against
oscar_int2_decode_attn on the same cache and queries: two calls in a row, the
second smaller, so a stale scratch from the first call would show."""
import numpy as np
import pytest

from synth import get
from tests.oscar_testlib import compare_attention, fill, make_cache

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def test_noalloc_matches_workspace_decode():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ultra_bit_kv_amd import SeqBatch
    w = get("c3_bs64").scaled(n_seqs=3, lengths=("list", (333, 517, 1000)))
    lens = [333, 517, 1000]
    print(f"[case] noalloc c3 reduced lens={lens}", flush=True)
    cache = make_cache(w, lens)
    q_rot = fill(cache, w, lens, chunk=300)
    for idx in ([0, 1, 2], [1]):          # the second call is smaller
        b = SeqBatch(idx, [lens[i] for i in idx])
        q = q_rot[idx].contiguous()
        want = cache.decode(b, q).cpu().numpy()
        out = torch.full((len(idx), w.hq, 128), float("nan"), dtype=torch.float32, device="cuda")
        got = cache.decode_noalloc(b, q, out).cpu().numpy()
        err, rel, ok = compare_attention(got.reshape(-1), want.reshape(-1))
        print(f"[case] noalloc seqs {idx}: max_abs={err:.3e} rel_l2={rel:.3e}", flush=True)
        assert ok, (idx, err, rel)
        # same plan, same kernels: the outputs are identical
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), idx
