"""Pins of the oracle's per-row quantizer (CPU only).

Expected values come from hand-worked rows (tests/golden), closed-form rows whose scale is an
exact power of two, exact rational evaluation, and invariants that any correct per-row
round-to-nearest quantizer must satisfy.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import decode_table, quantize_rows
from exact_ref import bruteforce_quantize_row, fraction_to_f32
from workloads import bf16_bits_to_f32, f32_to_bf16_bits, make_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_rows():
    rows = []
    with open(os.path.join(GOLDEN, "quantize_rows.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, sbits, xs, cs = [p.strip() for p in line.split("|")]
            x = np.array([float.fromhex(t) for t in xs.split()], dtype=np.float64)
            codes = np.array([int(t, 16) for t in cs.split()], dtype=np.uint8)
            rows.append((name, np.uint32(int(sbits, 16)), x, codes))
    return rows


@pytest.mark.parametrize("row", _load_rows(), ids=lambda r: r[0])
def test_golden_rows(row):
    name, sbits, x, codes = row
    x32 = x.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), x)
    assert np.array_equal(bf16_bits_to_f32(f32_to_bf16_bits(x32)), x32)   # bf16 values
    q, s = quantize_rows(x32[None, :])
    assert s.dtype == np.float32
    assert s.view(np.uint32)[0] == sbits
    assert [hex(c) for c in q[0]] == [hex(c) for c in codes]


def test_closed_form_rows_power_of_two_scale():
    """x = dec(c) * 2^j with a +-448 code in the row: scale = 2^j exactly and q == c."""
    t = decode_table()
    rng = np.random.default_rng(11)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    R, K = 64, 200
    codes = rng.choice(finite, size=(R, K))
    codes[np.arange(R), rng.integers(0, K, R)] = rng.choice([0x7E, 0xFE], R)
    j = rng.integers(-100, 100, size=R)
    x = (t[codes] * np.ldexp(1.0, j)[:, None]).astype(np.float32)
    assert np.array_equal(bf16_bits_to_f32(f32_to_bf16_bits(x)), x)
    q, s = quantize_rows(x)
    assert np.array_equal(s.astype(np.float64), np.ldexp(1.0, j))
    assert np.array_equal(q, codes)


def _rows(seed, M=48, K=1000):
    return bf16_bits_to_f32(make_rows(M, K, seed, n_outliers=10, factor=30.0))


def test_scale_is_correctly_rounded_amax_over_448():
    x = _rows(1)
    _, s = quantize_rows(x)
    amax = np.abs(x).max(axis=1)
    for a, sv in zip(amax, s):
        assert sv == np.float32(fraction_to_f32(Fraction(float(a)) / 448))


def test_amax_position_holds_448():
    x = _rows(2)
    q, s = quantize_rows(x)
    idx = np.abs(x).argmax(axis=1)
    for r, k in enumerate(idx):
        assert q[r, k] == (0xFE if x[r, k] < 0 else 0x7E)


def test_negation_flips_only_the_sign_bit():
    x = _rows(3)
    x[0, :5] = 0.0
    q, s = quantize_rows(x)
    qn, sn = quantize_rows(-x)
    assert np.array_equal(s, sn)
    assert np.array_equal(qn, q ^ 0x80)


@pytest.mark.parametrize("j", [-30, -7, 1, 9, 40])
def test_power_of_two_rescaling(j):
    x = _rows(4)
    q, s = quantize_rows(x)
    xs = (x.astype(np.float64) * 2.0 ** j).astype(np.float32)
    q2, s2 = quantize_rows(xs)
    assert np.array_equal(q2, q)
    assert np.array_equal(s2.astype(np.float64), s.astype(np.float64) * 2.0 ** j)


def test_rounding_error_within_half_step():
    """|dec(q) - x/scale| <= half the E4M3 grid step at |x/scale| (step 2^(max(e,-6)-3))."""
    x = _rows(5)
    q, s = quantize_rows(x)
    t = decode_table()
    quot = (x / s[:, None]).astype(np.float32).astype(np.float64)
    a = np.abs(quot)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    step = np.ldexp(1.0, (np.maximum(e, -6) - 3).astype(np.int64))
    err = np.abs(t[q] - quot)
    assert np.all(err <= step / 2)
    # exact ties (common when the scale is a power of two) must land on even codes
    tie = (err == step / 2) & (a < 448)
    assert tie.any()
    assert np.all(q[tie] % 2 == 0)


@pytest.mark.parametrize("seed", range(6))
def test_small_rows_match_exact_rational_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    K = 24
    rows = []
    # ordinary, huge, tiny (subnormal scale), and mixed-magnitude rows
    for scale_exp in (0, 100, -120, -130, -60):
        r = rng.standard_normal(K).astype(np.float32) * np.float32(2.0 ** scale_exp)
        rows.append(r)
    r = rng.standard_normal(K).astype(np.float32)
    r[rng.integers(0, K)] = np.float32(2.0 ** 60)
    rows.append(r)
    x = bf16_bits_to_f32(f32_to_bf16_bits(np.array(rows, dtype=np.float32)))
    q, s = quantize_rows(x)
    for i, row in enumerate(x):
        codes, scale = bruteforce_quantize_row(row)
        assert np.float32(scale).view(np.uint32) == s[i].view(np.uint32), i
        assert list(q[i]) == codes, i


def test_edge_rows():
    bf16_min_sub = np.float32(2.0 ** -133)
    x = np.array([
        [0.0] * 8,
        [-0.0, 0.0, -0.0, -0.0, 0.0, 0.0, -0.0, 0.0],
        [bf16_min_sub, -bf16_min_sub, 0, 0, -0.0, bf16_min_sub, 0, 0],          # subnormal amax
        [2.0 ** -126, 3 * 2.0 ** -133, -(2.0 ** -127), 0, 0, 0, 0, 1.5 * 2.0 ** -126],
        [5.0, 5.0, 5.0, 5.0, -5.0, -5.0, 5.0, 5.0],                               # all equal |x|
        [0, 0, 0, -7.0, 0, 0, 0, 0],                                              # one nonzero
        [3.0e38, -3.0e38, 1.0, -1.0, 2.0 ** -100, 0, 0, 1e30],                     # huge amax
    ], dtype=np.float32)
    x = bf16_bits_to_f32(f32_to_bf16_bits(x))
    q, s = quantize_rows(x)
    assert s[0] == 0 and s[1] == 0
    assert list(q[0]) == [0] * 8
    assert list(q[1]) == [0x80, 0, 0x80, 0x80, 0, 0, 0x80, 0]
    for i, row in enumerate(x):
        codes, scale = bruteforce_quantize_row(row)
        assert np.float32(scale).view(np.uint32) == s[i].view(np.uint32), i
        assert list(q[i]) == codes, i
    # a subnormal scale: the quotient can exceed 448 and must saturate, never produce NaN
    assert 0x7F not in q and 0xFF not in q


def test_numpy_float32_division_keeps_subnormals():
    """The oracle relies on IEEE float32 division with subnormals (no flush to zero)."""
    tiny = np.float32(2.0 ** -149)
    assert np.float32(2.0 ** -140) / np.float32(2.0 ** 8) == np.float32(2.0 ** -148)
    assert tiny / np.float32(1.0) == tiny
    assert np.float32(3 * 2.0 ** -149) / np.float32(2.0) == np.float32(2.0 ** -148)  # tie to even
