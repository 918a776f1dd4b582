"""Pins of the oracle's rotation (O1), attention (O5) and cache builder (CPU)."""

import math

import numpy as np
import pytest

from oracle import rotate, attention, cache, placement, quant
from oracle.rounding import bf16_bits_to_f64, f64_to_bf16_bits
from synth import bf16_from_f32, get


def _haar(rng, d=128):
    q, r = np.linalg.qr(rng.standard_normal((d, d)))
    return q * np.sign(np.diag(r))[None, :]


def test_generated_rotations_are_orthogonal():
    rk, rv = get("c2_qwen3_8b_bs1").rotations()
    for r in np.concatenate([rk, rv]):
        r = r.astype(np.float64)
        assert np.abs(r.T @ r - np.eye(128)).max() < 2e-6   # fp32-rounded Q factor
    q = _haar(np.random.default_rng(0))
    assert np.abs(q.T @ q - np.eye(128)).max() < 1e-13


def test_rotation_preserves_inner_products():
    # orthogonal x' = x R keeps q.k (attention scores) unchanged before rounding
    rng = np.random.default_rng(1)
    r = _haar(rng)
    q = rng.standard_normal((50, 128))
    k = rng.standard_normal((70, 128))
    lhs = rotate.rotate_f64(q, r) @ rotate.rotate_f64(k, r).T
    rhs = q @ k.T
    scale = np.linalg.norm(q, axis=1)[:, None] * np.linalg.norm(k, axis=1)[None, :]
    assert (np.abs(lhs - rhs) <= 1e-12 * scale).all()
    assert np.allclose(np.linalg.norm(rotate.rotate_f64(q, r), axis=1), np.linalg.norm(q, axis=1), rtol=1e-13)


def test_rotation_orientation_signed_permutation():
    # x' = x . R with R[i, pi(i)] = s_i  ->  x'[pi(i)] = s_i x[i] (catches R vs R^T)
    rng = np.random.default_rng(2)
    pi = rng.permutation(128)
    s = rng.choice([-1.0, 1.0], 128)
    r = np.zeros((128, 128), np.float32)
    r[np.arange(128), pi] = s
    xb = bf16_from_f32(rng.standard_normal((9, 128)).astype(np.float32))
    out = rotate.rotate_to_bf16(xb, r)
    x = bf16_bits_to_f64(xb)
    exp = np.zeros_like(x)
    exp[:, pi] = x * s
    assert np.array_equal(bf16_bits_to_f64(out), exp)
    assert np.array_equal(rotate.rotate_to_bf16(xb, np.eye(128, dtype=np.float32)), xb)


def test_rotation_correctly_rounded_small_exact():
    rng = np.random.default_rng(3)
    r = _haar(rng).astype(np.float32)
    xb = bf16_from_f32(rng.standard_normal((3, 128)).astype(np.float32))
    out = rotate.rotate_to_bf16(xb, r)
    x = bf16_bits_to_f64(xb)
    rd = r.astype(np.float64)
    for i in range(3):
        for j in range(0, 128, 9):
            assert out[i, j] == rotate.exact_row_dot_bf16(x[i], rd[:, j])


def test_rotation_guard_catches_fp64_double_rounding():
    # exact x.R = 1 + 2^-8 + 2^-60 lies just above a bf16 tie; the fp64 sum
    # drops 2^-60 and lands on the tie (-> 1.0); the guard recomputes exactly.
    x = np.zeros((1, 128), np.float32)
    x[0, :3] = 1.0
    r = np.zeros((128, 128), np.float32)
    r[0, 0], r[1, 0], r[2, 0] = 1.0, 2.0 ** -8, 2.0 ** -60
    r[0, 1], r[1, 1] = 1.0, 2.0 ** -8            # exact tie -> even -> 1.0
    out = rotate.rotate_to_bf16(bf16_from_f32(x), r)
    assert bf16_bits_to_f64(out[0, 0]) == 1.0 + 2.0 ** -7
    assert bf16_bits_to_f64(out[0, 1]) == 1.0
    naive = f64_to_bf16_bits(bf16_bits_to_f64(bf16_from_f32(x)) @ r.astype(np.float64))
    assert bf16_bits_to_f64(naive[0, 0]) == 1.0          # what the unguarded path gives


def _brute_attention(q, k, v):
    """softmax(q k^T / sqrt(d)) v with plain Python loops and math.exp."""
    d = len(q)
    logits = [sum(q[i] * kr[i] for i in range(d)) / math.sqrt(d) for kr in k]
    m = max(logits)
    w = [math.exp(l - m) for l in logits]
    tot = sum(w)
    return [sum(w[t] * v[t][j] for t in range(len(v))) / tot for j in range(d)]


@pytest.mark.parametrize("t", [1, 2, 5, 8])
def test_attention_brute_force(t):
    rng = np.random.default_rng(10 + t)
    q = rng.standard_normal((3, 128)) * 2
    k = rng.standard_normal((t, 128))
    v = rng.standard_normal((t, 128))
    got = attention.attend(q, k, v)
    for i in range(3):
        assert np.allclose(got[i], _brute_attention(q[i].tolist(), k.tolist(), v.tolist()),
                           rtol=0, atol=1e-13)


def test_attention_special_cases():
    rng = np.random.default_rng(20)
    k = rng.standard_normal((7, 128))
    v = rng.standard_normal((7, 128))
    q = rng.standard_normal((4, 128))
    one = attention.attend(q, k[:1], v[:1])
    assert np.array_equal(one, np.repeat(v[:1], 4, axis=0))           # single token
    assert np.allclose(attention.attend(np.zeros((2, 128)), k, v), v.mean(0), atol=1e-15)


def test_split_merge_equals_unsplit():
    rng = np.random.default_rng(21)
    k = rng.standard_normal((300, 128)) * 2
    v = rng.standard_normal((300, 128))
    q = rng.standard_normal((4, 128)) * 3
    full = attention.attend(q, k, v)
    for cuts in ([150], [1, 2, 299], [17, 100, 101, 250], list(range(10, 300, 10))):
        assert np.abs(attention.attend_split(q, k, v, cuts) - full).max() <= 1e-14


def test_unrotate_orientation_and_basis_invariance():
    rng = np.random.default_rng(22)
    rk, rv = _haar(rng), _haar(rng)
    q = rng.standard_normal((4, 128))
    k = rng.standard_normal((40, 128))
    v = rng.standard_normal((40, 128))
    # attention in the rotated basis, un-rotated with R_V^T, equals attention
    # in the original basis (no quantization, no rounding)
    o = attention.decode_head(rotate.rotate_f64(q, rk), rotate.rotate_f64(k, rk),
                              rotate.rotate_f64(v, rv), rv)
    assert np.abs(o - attention.attend(q, k, v)).max() < 1e-12


def test_head_cache_identity_rotation_segments():
    w = get("c1_tiny")
    n = 700
    k = w.keys(0, 0, n)[:, 0]
    v = w.values(0, 0, n)[:, 0]
    eye = np.eye(128, dtype=np.float32)
    hc = cache.HeadCache(k, v, eye, eye, np.float32(0.9), np.float32(0.9), 128, 4, 128, 16)
    assert np.array_equal(hc.k_rot, k) and np.array_equal(hc.v_rot, v)
    a, b = hc.int2
    assert (a, b) == (4, placement.s_quant(n, 4, 128, 16))
    c, s16, z16 = quant.quantize_rows(bf16_bits_to_f64(k[a:b]), np.float32(0.9), 128)
    assert np.array_equal(c, hc.kc) and np.array_equal(s16, hc.ks)
    kd, vd = hc.dequant_f32()
    assert np.array_equal(kd[:4], bf16_bits_to_f64(k[:4]).astype(np.float32))
    assert np.array_equal(kd[b:], bf16_bits_to_f64(k[b:]).astype(np.float32))
    assert np.array_equal(kd[a:b], quant.dequant_rows(c, s16, z16, 128).astype(np.float32))
    rows = hc.window_rows()
    assert sorted(rows.values()) == list(range(4)) + list(range(b, n))


def test_general_invertible_key_transform_keeps_scores():
    # WUSH-KV notes, "core method": a mutually inverse pair between the two
    # factors of K^T Q leaves the scores unchanged, so a non-orthogonal key
    # transform T pairs with the query transform T^-T (row vectors)
    rng = np.random.default_rng(23)
    t = _haar(rng) * rng.uniform(0.5, 2.0, 128)[None, :]   # anisotropic scaling
    tq = np.linalg.inv(t).T
    q = rng.standard_normal((30, 128))
    k = rng.standard_normal((60, 128))
    lhs = rotate.rotate_f64(q, tq) @ rotate.rotate_f64(k, t).T
    rhs = q @ k.T
    scale = np.linalg.norm(q, axis=1)[:, None] * np.linalg.norm(k, axis=1)[None, :]
    assert (np.abs(lhs - rhs) <= 1e-11 * scale).all()
    # an orthogonal T is its own inverse transpose: the query transform is R_K
    r = _haar(rng)
    assert np.abs(np.linalg.inv(r).T - r).max() < 1e-12
    # the same transform keeps attention itself unchanged when values are untouched
    v = rng.standard_normal((60, 128))
    o = attention.attend(rotate.rotate_f64(q[:4], tq), rotate.rotate_f64(k, t), v)
    assert np.abs(o - attention.attend(q[:4], k, v)).max() < 1e-11


def test_absorbed_value_transform_output_basis():
    # OSCAR summary s4 / WUSH-KV notes: with R_V folded into the output
    # projection the decode output stays in the rotated basis: o' = o . R_V
    rng = np.random.default_rng(24)
    rv = _haar(rng)
    q = rng.standard_normal((4, 128))
    k = rng.standard_normal((40, 128))
    v = rng.standard_normal((40, 128))
    o_rot = attention.attend(q, k, rotate.rotate_f64(v, rv))
    assert np.abs(o_rot - rotate.rotate_f64(attention.attend(q, k, v), rv)).max() < 1e-12
    assert np.abs(attention.unrotate(o_rot, rv) - attention.attend(q, k, v)).max() < 1e-12


# ---- structured rotation R = H (P_br) / sqrt(d) (OScaR notes, "Canalized
# Rotation"; OSCAR summary page, section 5 "Rotation Analysis")

def _bits(vals):
    return f64_to_bf16_bits(np.asarray(vals, np.float64))


def test_hadamard_signs_match_library_sylvester():
    from scipy.linalg import hadamard
    for d in (2, 4, 32, 128):
        assert np.array_equal(rotate.hadamard_signs(d), hadamard(d))
    assert np.array_equal(rotate.hadamard_signs(2), np.array([[1, 1], [1, -1]]))


def test_hadamard_bit_reversal_permutation():
    from scipy.linalg import hadamard
    br = [rotate.bit_reverse(k, 7) for k in range(128)]
    assert (br[0], br[1], br[3], br[64], br[127]) == (0, 64, 96, 1, 127)
    assert sorted(br) == list(range(128)) and all(br[br[k]] == k for k in range(128))
    s, h = rotate.hadamard_signs(128, True), hadamard(128)
    assert np.array_equal(s, h[:, br])            # H P_br: columns of H in bit-reversed order
    assert np.array_equal(s, h[br, :])            # which equals P_br H
    assert np.all(s[1, :64] == 1) and np.all(s[1, 64:] == -1)
    assert np.array_equal(rotate.hadamard_signs(128)[1], np.tile([1, -1], 64))


@pytest.mark.parametrize("bitrev", [False, True])
def test_hadamard_rotation_orthogonal_and_preserves_scores(bitrev):
    r = rotate.Hadamard(128, bitrev).matrix()
    assert np.abs(r @ r.T - np.eye(128)).max() < 1e-14
    assert np.all(np.abs(np.abs(r) - 1 / math.sqrt(128)) < 1e-17)
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal((4, 128)), rng.standard_normal((6, 128))
    assert np.abs((q @ r) @ (k @ r).T - q @ k.T).max() < 1e-12


@pytest.mark.parametrize("bitrev", [False, True])
def test_hadamard_all_ones_row(bitrev):
    # x . H = (128, 0, ..., 0), and bit reversal keeps index 0: x' = (sqrt(128), 0, ...),
    # sqrt(128) = 11.3137... rounds to bf16 11.3125
    out = rotate.hadamard_rotate_to_bf16(_bits(np.ones((1, 128))), bitrev)
    assert bf16_bits_to_f64(out)[0, 0] == 11.3125 and out[0, 0] == 0x4135
    assert np.all(bf16_bits_to_f64(out)[0, 1:] == 0)


def test_hadamard_one_hot_spreads_energy_evenly():
    # a one-hot row becomes a row of H / sqrt(d): every channel +-|k| / sqrt(d)
    from scipy.linalg import hadamard
    h = hadamard(128)
    for i in (0, 1, 5, 127):
        x = np.zeros((1, 128))
        x[0, i] = 1.0
        out = bf16_bits_to_f64(rotate.hadamard_rotate_to_bf16(_bits(x)))[0]
        assert np.array_equal(out, 0.08837890625 * h[i])      # bf16(1 / sqrt(128))


def test_round_scaled_ties_and_values():
    from fractions import Fraction
    # d = 64: s / 8 is rational, so exact ties occur and go to the even significand
    assert rotate.round_scaled_to_bf16(Fraction(8) * (1 + Fraction(1, 256)), 64) == 0x3F80
    assert rotate.round_scaled_to_bf16(Fraction(8) * (1 + Fraction(3, 256)), 64) == 0x3F82
    assert rotate.round_scaled_to_bf16(-Fraction(8) * (1 + Fraction(1, 256)), 64) == 0xBF80
    assert rotate.round_scaled_to_bf16(Fraction(8) * (1 + Fraction(5, 512)), 64) == 0x3F81
    assert rotate.round_scaled_to_bf16(Fraction(1), 128) == 0x3DB5          # 1 / sqrt(128)
    assert rotate.round_scaled_to_bf16(Fraction(0), 128) == 0


@pytest.mark.parametrize("bitrev", [False, True])
def test_hadamard_rotate_matches_dense_and_exact(bitrev):
    from fractions import Fraction
    rng = np.random.default_rng(11)
    x = rng.standard_normal((48, 128)) * np.exp(rng.uniform(-3, 3, (48, 1)))
    x[::7, 3] *= 300.0                               # channel outliers
    xb = _bits(x)
    got = rotate.hadamard_rotate_to_bf16(xb, bitrev)
    dense = f64_to_bf16_bits(bf16_bits_to_f64(xb) @ rotate.Hadamard(128, bitrev).matrix())
    assert np.array_equal(got, dense)
    sg = rotate.hadamard_signs(128, bitrev)
    xf = bf16_bits_to_f64(xb)
    for i, j in [(0, 0), (5, 17), (7, 64), (47, 127), (21, 3)]:
        s = sum((Fraction(a) * int(b) for a, b in zip(xf[i].tolist(), sg[:, j].tolist())), Fraction(0))
        assert got[i, j] == rotate.round_scaled_to_bf16(s, 128)


def test_hadamard_head_cache_and_unrotation():
    rng = np.random.default_rng(5)
    k = _bits(rng.standard_normal((40, 128)))
    v = _bits(rng.standard_normal((40, 128)))
    had = rotate.Hadamard(128, True)
    hc = cache.HeadCache(k, v, had, had, 1.0, 1.0, 64, 4, 8, 8)
    assert np.array_equal(hc.k_rot, rotate.hadamard_rotate_to_bf16(k, True))
    o = rng.standard_normal((3, 128))
    assert np.abs(attention.unrotate(o @ had.matrix(), had) - o).max() < 1e-12
