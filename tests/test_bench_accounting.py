"""bench.py's byte accounting (closed-form S_quant) agrees with the oracle's
placement rule on every workload shape."""
import numpy as np
import pytest

import bench
from oracle import placement
from synth import CONFIGS


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_algorithmic_bytes_matches_oracle_placement(name):
    w = CONFIGS[name]
    lens = [int(x) for x in w.lengths_after()] + [1, 2, w.s_sink, w.s_sink + w.s_keep,
                                                  w.s_sink + w.s_keep + w.s_flush + 3]
    per = 64 + 1024 // w.group
    want = 0
    for L in lens:
        sink, int2, rec = placement.segments(L, w.s_sink, w.s_keep, w.s_flush)
        n2 = int2[1] - int2[0]
        nb = (sink[1] - sink[0]) + (rec[1] - rec[0])
        want += w.hkv * (n2 * per + nb * 512) + 4 * (-(-n2 // 16))
    want += len(lens) * w.hq * 128 * 2
    assert bench.algorithmic_bytes(w, np.array(lens)) == want
