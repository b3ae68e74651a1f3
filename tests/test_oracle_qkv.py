"""Pins of the oracle's QKV epilogue (query/key RMS normalization + rotary embedding), CPU only.

Each pin checks the oracle against something other than its own formula: closed-form rows, a
library RMS norm, complex multiplication, exact rotations by special angles, the relative-position
property that makes the rotation useful, and index-tagged inputs for the layout.
"""
import math

import numpy as np
import pytest
import torch

from oracle.qkv import HEAD_DIM, qkv_split_norm_rope, rms_norm, rope_pairs

D = HEAD_DIM


@pytest.mark.parametrize("c", [1.0, -3.5, 1e-3, 250.0])
def test_rms_norm_of_a_constant_row(c):
    """All entries c: the root mean square is |c|, so each entry becomes c / sqrt(c^2 + eps) w."""
    rng = np.random.default_rng(1)
    w = rng.standard_normal(D)
    out = rms_norm(np.full((2, D), c), w, eps=1e-6)
    want = c / math.sqrt(c * c + 1e-6) * w
    assert np.allclose(out, want[None, :], rtol=1e-14, atol=0)


def test_rms_norm_of_a_row_with_two_magnitudes():
    """Half the entries a and half b: the mean square is (a^2 + b^2) / 2."""
    a, b = 3.0, -4.0
    v = np.array([a, b] * (D // 2))
    out = rms_norm(v[None, :], np.ones(D), eps=0.0)[0]
    r = math.sqrt((a * a + b * b) / 2)
    assert np.allclose(out, v / r, rtol=1e-15, atol=0)


def test_rms_norm_matches_the_library():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((7, 3, D)) * 5
    w = rng.standard_normal(D)
    lib = torch.nn.functional.rms_norm(torch.from_numpy(v), (D,), torch.from_numpy(w), eps=1e-6)
    assert np.allclose(rms_norm(v, w, 1e-6), lib.numpy(), rtol=1e-13, atol=1e-15)


def test_rms_norm_ignores_the_scale_of_its_input():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((4, D))
    w = rng.standard_normal(D)
    assert np.allclose(rms_norm(v, w, 0.0), rms_norm(1e3 * v, w, 0.0), rtol=1e-13, atol=0)


def _angles(M, seed=4):
    rng = np.random.default_rng(seed)
    return rng.uniform(-math.pi, math.pi, (M, D // 2))


def test_rope_special_angles_are_exact():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((3, 2, D))
    one, zero = np.ones((3, D // 2)), np.zeros((3, D // 2))
    assert np.array_equal(rope_pairs(v, one, zero), v)                 # angle 0
    quarter = rope_pairs(v, zero, one)                                # angle pi/2: (a, b) -> (-b, a)
    assert np.array_equal(quarter[..., 0::2], -v[..., 1::2])
    assert np.array_equal(quarter[..., 1::2], v[..., 0::2])
    half = rope_pairs(v, -one, zero)                                  # angle pi: negation
    assert np.array_equal(half, -v)


def test_rope_is_complex_multiplication_of_adjacent_pairs():
    """Channels (2i, 2i + 1) as the complex number a + ib, turned by exp(i theta)."""
    M = 5
    rng = np.random.default_rng(6)
    v = rng.standard_normal((M, 3, D))
    th = _angles(M)
    z = v[..., 0::2] + 1j * v[..., 1::2]
    rz = z * np.exp(1j * th)[:, None, :]
    out = rope_pairs(v, np.cos(th), np.sin(th))
    assert np.allclose(out[..., 0::2], rz.real, rtol=1e-13, atol=1e-14)
    assert np.allclose(out[..., 1::2], rz.imag, rtol=1e-13, atol=1e-14)


def test_rope_keeps_pair_lengths():
    M = 4
    rng = np.random.default_rng(7)
    v = rng.standard_normal((M, 2, D))
    th = _angles(M, 8)
    out = rope_pairs(v, np.cos(th), np.sin(th))
    assert np.allclose(np.hypot(out[..., 0::2], out[..., 1::2]),
                       np.hypot(v[..., 0::2], v[..., 1::2]), rtol=1e-13, atol=0)


def test_rope_scores_depend_only_on_relative_position():
    """With angles m * omega_i, the dot product of a query at position m1 and a key at m2 after
    the rotation depends only on m1 - m2."""
    rng = np.random.default_rng(9)
    qv, kv = rng.standard_normal(D), rng.standard_normal(D)
    omega = 10000.0 ** (-np.arange(D // 2) / (D // 2))

    def rot(x, m):
        th = (m * omega)[None, :]
        return rope_pairs(x[None, :], np.cos(th), np.sin(th))[0]

    for m1, m2, shift in [(3, 7, 11), (0, 5, 100), (40, 2, -2)]:
        s0 = rot(qv, m1) @ rot(kv, m2)
        s1 = rot(qv, m1 + shift) @ rot(kv, m2 + shift)
        assert math.isclose(s0, s1, rel_tol=1e-11, abs_tol=1e-11)
    # and it does change with the distance
    assert not math.isclose(rot(qv, 0) @ rot(kv, 1), rot(qv, 0) @ rot(kv, 5), rel_tol=1e-6)


def test_split_and_head_major_layout():
    """Index-tagged input: v[m, n] = 1000 m + n. With angle 0, unit norm scales and the values
    region, every output position must come from the right (token, column)."""
    H, M = 3, 5
    N = 3 * H * D
    v = 1000.0 * np.arange(M)[:, None] + np.arange(N)[None, :]
    one, zero = np.ones((M, D // 2)), np.zeros((M, D // 2))
    q, k, vv = qkv_split_norm_rope(v, H, np.ones(D), np.ones(D), one, zero, eps=0.0)
    assert q.shape == k.shape == vv.shape == (H, M, D)
    for h in range(H):
        for m in range(M):
            assert np.array_equal(vv[h, m], v[m, 2 * H * D + h * D:2 * H * D + (h + 1) * D])
            for out, base in ((q, 0), (k, H * D)):
                row = v[m, base + h * D:base + (h + 1) * D]
                want = row / math.sqrt(float(np.mean(row * row)))
                assert np.allclose(out[h, m], want, rtol=1e-14, atol=0)


def test_norm_scales_are_per_region():
    """The query scale acts on queries only, the key scale on keys only, values are untouched."""
    H, M = 2, 3
    rng = np.random.default_rng(10)
    v = rng.standard_normal((M, 3 * H * D))
    wq, wk = rng.standard_normal(D), rng.standard_normal(D)
    one, zero = np.ones((M, D // 2)), np.zeros((M, D // 2))
    q1, k1, v1 = qkv_split_norm_rope(v, H, wq, wk, one, zero)
    q2, k2, v2 = qkv_split_norm_rope(v, H, np.ones(D), np.ones(D), one, zero)
    assert np.allclose(q1, q2 * wq, rtol=1e-14, atol=0)
    assert np.allclose(k1, k2 * wk, rtol=1e-14, atol=0)
    assert np.array_equal(v1, v2)


def test_rotation_comes_after_the_norm():
    """Normalizing then rotating keeps each head's mean square at 1 (unit scales, eps 0); the
    other order would too, so also check one value against a hand computation."""
    M = 2
    v = np.zeros((M, 3 * D))
    v[:, 0], v[:, 1] = 3.0, 4.0            # query head 0: pair 0 = (3, 4), rest zero
    v[:, D] = 1.0                            # keys not all zero (eps is 0 here)
    th = np.zeros((M, D // 2))
    th[:, 0] = math.pi / 3
    q, _, _ = qkv_split_norm_rope(v, 1, np.ones(D), np.ones(D), np.cos(th), np.sin(th), eps=0.0)
    r = math.sqrt(25.0 / D)                  # rms of (3, 4, 0, ..., 0)
    a, b = 3.0 / r, 4.0 / r
    c, s = math.cos(math.pi / 3), math.sin(math.pi / 3)
    assert math.isclose(q[0, 0, 0], c * a - s * b, rel_tol=1e-14)
    assert math.isclose(q[0, 0, 1], s * a + c * b, rel_tol=1e-14)
    assert np.allclose(np.mean(q * q, axis=-1), 1.0, rtol=1e-14)
