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


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_int2_pages_matches_oracle_placement(name):
    w = CONFIGS[name]
    for L in [int(x) for x in w.lengths_after()] + [0, 1, w.s_sink, w.s_sink + w.s_keep + 1,
                                                    w.s_sink + w.s_keep + w.s_flush,
                                                    w.s_sink + w.s_keep + 5 * w.s_flush + 7]:
        assert bench.int2_pages(w, L) == placement.n_int2_pages(L, w.s_sink, w.s_keep, w.s_flush)


def test_timed_path_does_not_load_the_oracle():
    """Only the CPU-baseline leg may touch the oracle: importing bench and
    running its set-up arithmetic must leave oracle modules unloaded."""
    import subprocess
    import sys
    code = ("import sys, bench, synth; w = synth.get('c3_bs64'); "
            "bench.int2_pages(w, 5000); bench.algorithmic_bytes(w, w.lengths_after()); "
            "bad = [m for m in sys.modules if m == 'oracle' or m.startswith('oracle.') "
            "or m.startswith('tests')]; print(bad); sys.exit(1 if bad else 0)")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       cwd=str(__import__("pathlib").Path(bench.__file__).parent))
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_append_bytes_matches_oracle_placement(name):
    w = CONFIGS[name]
    ns = [1, 2, w.s_sink, w.s_sink + w.s_keep, w.s_sink + w.s_keep + w.s_flush + 3, 2048]
    per = 64 + 1024 // w.group
    want = 0
    for n in ns:
        sink, int2, rec = placement.segments(n, w.s_sink, w.s_keep, w.s_flush)
        n2 = int2[1] - int2[0]
        nb = (sink[1] - sink[0]) + (rec[1] - rec[0])
        want += n * (2 * w.hkv + 2 * w.hq) * 256 + w.hkv * (n2 * per + nb * 512)
    assert bench.append_bytes(w, ns) == want
