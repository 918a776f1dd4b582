"""The seeded input generators: the bf16 rounding of the drawn fp32 values is
torch's cast (round to nearest even) bit for bit, and slices regenerate."""

import numpy as np
import torch

from synth import get
from synth.workloads import bf16_from_f32


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(20.0),
        rng.standard_normal(1000).astype(np.float32) * np.float32(1e-39),     # subnormals
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8,
                  1.0 + 2 ** -8 + 2 ** -20, 65504.0, 1e-45], np.float32),
    ])
    # ties: halfway between two bf16 values with even and odd lower neighbours
    ties = (np.arange(1, 4000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_from_f32(x), want)


def test_slices_regenerate():
    w = get("c3_bs64")
    full = w.keys(3, 0, 700)
    assert np.array_equal(full[250:600], w.keys(3, 250, 600))
    assert np.array_equal(w.values(3, 0, 700)[511:513], w.values(3, 511, 513))
