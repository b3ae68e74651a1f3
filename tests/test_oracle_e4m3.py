"""Pins of the oracle's E4M3 decode table and encoder (CPU only).

Every expected value comes from somewhere other than the oracle's own arithmetic: hand-worked
landmarks (tests/golden), exact rationals built from the bit fields, exhaustive nearest-value
search, and torch's float8_e4m3fn cast and decoder (library routines).
"""
import os

import numpy as np
import pytest

from oracle import decode_table, encode_e4m3
from exact_ref import (e4m3_values_exact, e4m3_values_torch, nearest_code_bruteforce,
                       torch_encode)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_landmarks():
    vals, codes = [], []
    with open(os.path.join(GOLDEN, "e4m3_landmarks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            vals.append(float.fromhex(parts[0]))
            codes.append(int(parts[1], 16))
    return np.array(vals, dtype=np.float64), np.array(codes, dtype=np.uint8)


def test_landmarks_are_float32_values():
    vals, _ = _load_landmarks()
    assert np.array_equal(vals.astype(np.float32).astype(np.float64), vals)


def test_encode_landmarks():
    vals, codes = _load_landmarks()
    got = encode_e4m3(vals.astype(np.float32))
    assert [hex(c) for c in got] == [hex(c) for c in codes]


def test_decode_spot_values():
    t = decode_table()
    assert t[0x7E] == 448.0
    assert t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6
    assert t[0x01] == 2.0 ** -9
    assert t[0x38] == 1.0
    assert t[0x00] == 0.0 and not np.signbit(t[0x00])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isfinite(np.delete(t, [0x7F, 0xFF])).all()


def test_decode_matches_exact_rationals():
    t = decode_table()
    ex = e4m3_values_exact()
    for c in range(127):
        assert t[c] == float(ex[c])
        assert t[c | 0x80] == -float(ex[c])


def test_decode_matches_torch_decoder():
    t = decode_table()
    tt = e4m3_values_torch()
    nan = np.isnan(t)
    assert np.array_equal(nan, np.isnan(tt))
    assert np.array_equal(t[~nan], tt[~nan])
    assert np.array_equal(np.signbit(t[~nan]), np.signbit(tt[~nan]))


def test_decode_strictly_increasing():
    t = decode_table()
    assert np.all(np.diff(t[:0x7F]) > 0)
    assert len(set(t[:0x7F].tolist())) == 127


def test_encode_roundtrips_every_finite_code():
    t = decode_table()
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    got = encode_e4m3(t[codes].astype(np.float32))
    assert np.array_equal(got, codes)


def _all_finite_bf16_as_f32():
    u = np.arange(1 << 16, dtype=np.uint32)
    f = (u << 16).view(np.float32)
    return f[np.isfinite(f)]


def test_encode_exhaustive_bf16_vs_bruteforce():
    v = _all_finite_bf16_as_f32()
    assert v.size == 65536 - 2 - 2 * 127  # +-inf and the 254 NaN patterns excluded
    assert np.array_equal(encode_e4m3(v), nearest_code_bruteforce(v))


def test_encode_exhaustive_bf16_vs_torch():
    v = _all_finite_bf16_as_f32()
    assert np.array_equal(encode_e4m3(v), torch_encode(v))


def _midpoints():
    ex = [float(x) for x in e4m3_values_exact()]          # 0 .. 448
    mids = [(a + b) / 2 for a, b in zip(ex[:-1], ex[1:])]  # exact in float64, fit in float32
    return np.array(mids, dtype=np.float64)


def test_encode_midpoints_and_neighbours():
    mids = _midpoints().astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), _midpoints())
    bits = mids.view(np.int32)
    pts = [mids]
    for k in (1, 2, 3):
        pts.append((bits + k).view(np.float32))
        pts.append((bits - k).view(np.float32))
    pts.append(np.array([448.0, 464.0, 465.0, 447.99997, 448.00003, 480.0, 3.0e38], np.float32))
    v = np.concatenate(pts)
    v = np.concatenate([v, -v])
    got = encode_e4m3(v)
    assert np.array_equal(got, nearest_code_bruteforce(v))
    assert np.array_equal(got, torch_encode(v))


def test_encode_random_float32_vs_torch():
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    assert np.array_equal(encode_e4m3(v), torch_encode(v))


def test_encode_random_float32_vs_bruteforce():
    rng = np.random.default_rng(7)
    # exponents concentrated where the codes live (2^-12 .. 2^9), every mantissa pattern possible
    e = rng.integers(127 - 12, 127 + 10, size=300_000).astype(np.uint32)
    m = rng.integers(0, 1 << 23, size=300_000).astype(np.uint32)
    s = rng.integers(0, 2, size=300_000).astype(np.uint32)
    v = ((s << 31) | (e << 23) | m).view(np.float32)
    assert np.array_equal(encode_e4m3(v), nearest_code_bruteforce(v))


def test_encode_float32_subnormals_and_sign():
    v = np.array([1e-45, -1e-45, 1e-40, -1e-40, 1.1754942e-38, -1.1754942e-38], dtype=np.float32)
    got = encode_e4m3(v)
    assert list(got) == [0x00, 0x80, 0x00, 0x80, 0x00, 0x80]


def test_encode_rejects_nonfinite():
    with pytest.raises(ValueError):
        encode_e4m3(np.array([np.inf], np.float32))
    with pytest.raises(ValueError):
        encode_e4m3(np.array([np.nan], np.float32))
