"""Pins of the oracle's contraction and epilogues (CPU only).

Expected values come from integer matrix products, permutation weights (closed form), exact
rational evaluation of the whole chain on tiny shapes, the GELU's odd-part identity and torch's
GELU (library routine), and the gated epilogue's special cases.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import (EPI_BIAS, EPI_GATED_RESIDUAL, EPI_GELU_TANH, decode_table, gelu_tanh,
                    linear_ref, quantize_rows, round_to_bf16)
from oracle.linear import contract
from exact_ref import bruteforce_linear, e4m3_values_exact
from workloads import bf16_bits_to_f32, f32_to_bf16_bits, make_linear_inputs, workload

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def _int_values():
    """code -> integer dec(code) * 2^9, built from exact rationals (not the oracle's table)."""
    ex = e4m3_values_exact()
    iv = np.zeros(256, dtype=np.int64)
    for c in range(127):
        n = ex[c] * 512
        assert n.denominator == 1
        iv[c] = n.numerator
        iv[c | 0x80] = -n.numerator
    return iv


@pytest.mark.parametrize("M,N,K", [(16, 24, 15360), (37, 29, 256), (5, 3, 1), (64, 64, 3072)])
def test_contraction_is_exact_integer_product(M, N, K):
    rng = np.random.default_rng(M * 1000 + K)
    q = rng.choice(FINITE, size=(M, K))
    qw = rng.choice(FINITE, size=(N, K))
    iv = _int_values()
    exact = iv[q] @ iv[qw].T                    # int64, no rounding anywhere
    acc = contract(q, qw)
    assert np.array_equal(acc * 2.0 ** 18, exact.astype(np.float64))
    assert np.all(np.abs(exact) < 2 ** 53)


def test_contraction_extreme_magnitudes_exact():
    """All-448 rows (largest partial sums) and all-2^-9 rows (smallest terms) at K = 15360."""
    K = 15360
    q = np.array([[0x7E] * K, [0x01] * K, [0xFE, 0x7E] * (K // 2)], dtype=np.uint8)
    qw = np.array([[0x7E] * K, [0x01] * K], dtype=np.uint8)
    acc = contract(q, qw)
    assert acc[0, 0] == 448.0 * 448.0 * K
    assert acc[1, 1] == 2.0 ** -18 * K
    assert acc[0, 1] == 448.0 * 2.0 ** -9 * K
    assert acc[2, 0] == 0.0


def test_permutation_weights():
    """W = 448 P (P a permutation): sw = 1, qw holds 0x7E at pi(n), and
    y[:, n] = 448 * dec(q[:, pi(n)]) * sa + bias[n]."""
    rng = np.random.default_rng(5)
    M, K = 33, 96
    N = K
    perm = rng.permutation(K)
    W = np.zeros((N, K), dtype=np.float32)
    W[np.arange(N), perm] = 448.0
    qw, sw = quantize_rows(W)
    assert np.all(sw == 1.0)
    assert np.all(qw[np.arange(N), perm] == 0x7E)
    assert np.count_nonzero(qw) == N
    x = bf16_bits_to_f32(f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32)))
    q, sa = quantize_rows(x)
    bias = bf16_bits_to_f32(f32_to_bf16_bits(rng.standard_normal(N).astype(np.float32)))
    y = linear_ref(q, sa, qw, sw, bias, EPI_BIAS)
    t = decode_table()
    want = 448.0 * t[q[:, perm]] * sa.astype(np.float64)[:, None] + bias.astype(np.float64)[None, :]
    assert np.allclose(y, want, rtol=1e-15, atol=0)


def test_identity_weights_transposed_shapes():
    """M != N != K with W = 448 * [I | 0]: catches transposed operands and swapped scales."""
    rng = np.random.default_rng(6)
    M, K, N = 7, 40, 24
    W = np.zeros((N, K), dtype=np.float32)
    W[np.arange(N), np.arange(N)] = 448.0
    qw, sw = quantize_rows(W)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x = bf16_bits_to_f32(f32_to_bf16_bits(x))
    q, sa = quantize_rows(x)
    y = linear_ref(q, sa, qw, sw, None, EPI_BIAS)
    t = decode_table()
    assert np.allclose(y, 448.0 * t[q[:, :N]] * sa.astype(np.float64)[:, None], rtol=1e-15, atol=0)


def test_row_and_column_scales_apply_to_the_right_axis():
    """Power-of-two scales that differ per row and per column, exact integer reference."""
    rng = np.random.default_rng(8)
    M, N, K = 6, 10, 64
    q = rng.choice(FINITE, size=(M, K))
    qw = rng.choice(FINITE, size=(N, K))
    ea = rng.integers(-20, 20, M)
    eb = rng.integers(-20, 20, N)
    sa = np.ldexp(1.0, ea).astype(np.float32)
    sw = np.ldexp(1.0, eb).astype(np.float32)
    iv = _int_values()
    exact = (iv[q] @ iv[qw].T).astype(np.float64)
    want = exact * 2.0 ** -18 * np.ldexp(1.0, ea)[:, None] * np.ldexp(1.0, eb)[None, :]
    y = linear_ref(q, sa, qw, sw, None, EPI_BIAS)
    assert np.array_equal(y, want)


def test_bias_none_is_zero_bias():
    rng = np.random.default_rng(9)
    q = rng.choice(FINITE, size=(4, 32))
    qw = rng.choice(FINITE, size=(6, 32))
    sa = rng.random(4).astype(np.float32)
    sw = rng.random(6).astype(np.float32)
    for epi in (EPI_BIAS, EPI_GELU_TANH):
        assert np.array_equal(linear_ref(q, sa, qw, sw, None, epi),
                              linear_ref(q, sa, qw, sw, np.zeros(6, np.float32), epi))


def test_gelu_pins():
    v = np.linspace(-12, 12, 20001)
    g = gelu_tanh(v)
    assert gelu_tanh(0.0) == 0.0
    # odd part: gelu(v) - gelu(-v) = v for the tanh form
    assert np.allclose(g - gelu_tanh(-v), v, rtol=0, atol=1e-14)
    # library routine
    ref = torch.nn.functional.gelu(torch.from_numpy(v), approximate="tanh").numpy()
    assert np.allclose(g, ref, rtol=1e-13, atol=1e-15)
    # tails
    assert np.allclose(gelu_tanh(np.array([30.0, 100.0])), [30.0, 100.0], rtol=0, atol=0)
    assert np.all(np.abs(gelu_tanh(np.array([-30.0, -100.0]))) < 1e-300)
    # a value worked by hand: v = 1: u = sqrt(2/pi)(1 + 0.044715) = 0.833506..., 0.5(1+tanh u)
    u = math.sqrt(2 / math.pi) * 1.044715
    assert gelu_tanh(1.0) == pytest.approx(0.5 * (1 + math.tanh(u)), rel=1e-15)
    assert gelu_tanh(1.0) == pytest.approx(0.8411919906082768, rel=1e-12)


def test_gated_residual_special_cases():
    rng = np.random.default_rng(10)
    M, N, K = 9, 12, 64
    q = rng.choice(FINITE, size=(M, K))
    qw = rng.choice(FINITE, size=(N, K))
    sa = rng.random(M).astype(np.float32)
    sw = rng.random(N).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    res = rng.standard_normal((M, N)).astype(np.float32)
    y0 = linear_ref(q, sa, qw, sw, bias, EPI_GATED_RESIDUAL, np.zeros(N, np.float32), res)
    assert np.array_equal(y0, res.astype(np.float64))
    y1 = linear_ref(q, sa, qw, sw, bias, EPI_GATED_RESIDUAL, np.ones(N, np.float32),
                    np.zeros((M, N), np.float32))
    assert np.array_equal(y1, linear_ref(q, sa, qw, sw, bias, EPI_BIAS))
    with pytest.raises(ValueError):
        linear_ref(q, sa, qw, sw, bias, EPI_GATED_RESIDUAL)


@pytest.mark.parametrize("epi", [EPI_BIAS, EPI_GELU_TANH, EPI_GATED_RESIDUAL])
@pytest.mark.parametrize("seed", [0, 1])
def test_whole_chain_matches_exact_rational_bruteforce(epi, seed):
    rng = np.random.default_rng(200 + seed)
    M, N, K = 5, 7, 24
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.integers(0, K)] *= 30
    x[1] *= np.float32(2.0 ** -125)          # a row with a subnormal scale
    x[2] = 0.0                               # an all-zero row
    w = rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02)
    bias = rng.standard_normal(N).astype(np.float32) * np.float32(0.01)
    gate = np.float32(1) + rng.standard_normal(N).astype(np.float32) * np.float32(0.1)
    res = rng.standard_normal((M, N)).astype(np.float32)
    x, w, bias, gate, res = (bf16_bits_to_f32(f32_to_bf16_bits(a)) for a in (x, w, bias, gate, res))
    bq, bsa, bqw, bsw, by = bruteforce_linear(x, w, bias, epi, gate, res)
    q, sa = quantize_rows(x)
    qw, sw = quantize_rows(w)
    assert np.array_equal(q, bq) and np.array_equal(qw, bqw)
    assert np.array_equal(sa.view(np.uint32), bsa.view(np.uint32))
    assert np.array_equal(sw.view(np.uint32), bsw.view(np.uint32))
    y = linear_ref(q, sa, qw, sw, bias, epi, gate, res)
    assert np.allclose(y, by, rtol=1e-13, atol=1e-300)


def test_round_to_bf16_vs_torch_on_float32_values():
    rng = np.random.default_rng(12)
    bits = rng.integers(0, 1 << 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.3e38)]
    ours = round_to_bf16(f.astype(np.float64))
    theirs = torch.from_numpy(f.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, theirs)
    assert np.array_equal(np.signbit(ours), np.signbit(theirs))


def test_round_to_bf16_hand_cases():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: tie to even (1.0)
    assert round_to_bf16(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: tie to even (1 + 2^-6)
    assert round_to_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    # just above a tie rounds up; fp64 inputs are rounded once, directly
    assert round_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7
    # subnormal grid 2^-133
    assert round_to_bf16(2.0 ** -134) == 0.0
    assert round_to_bf16(3 * 2.0 ** -134) == 2.0 ** -132
    assert round_to_bf16(-(2.0 ** -140)) == 0.0 and np.signbit(round_to_bf16(-(2.0 ** -140)))
    # overflow
    assert round_to_bf16((2 - 2.0 ** -8) * 2.0 ** 127) == np.inf
    assert round_to_bf16((2 - 2.0 ** -7) * 2.0 ** 127) == (2 - 2.0 ** -7) * 2.0 ** 127


def test_tiny_workload_sampled_against_bruteforce():
    """The tiny 64x256x512 workload: whole quantizer, and a sample of outputs, exactly."""
    w = workload("tiny-64x256x512")
    inp = make_linear_inputs(w.linears[0], w.seed)
    x = bf16_bits_to_f32(inp.x)
    wt = bf16_bits_to_f32(inp.w)
    bias = bf16_bits_to_f32(inp.bias)
    q, sa = quantize_rows(x)
    qw, sw = quantize_rows(wt)
    rows = [0, 17, 63]
    cols = [0, 5, 300, 511]
    bq, bsa, bqw, bsw, by = bruteforce_linear(x[rows], wt[cols], bias[cols], "bias")
    assert np.array_equal(q[rows], bq) and np.array_equal(qw[cols], bqw)
    assert np.array_equal(sa[rows], bsa) and np.array_equal(sw[cols], bsw)
    y = linear_ref(q, sa, qw, sw, bias, EPI_BIAS)
    assert np.allclose(y[np.ix_(rows, cols)], by, rtol=1e-13, atol=1e-300)
    # the outlier columns dominate amax, so every row's 448 sits in one of them
    idx = np.abs(x).argmax(axis=1)
    assert set(idx.tolist()) <= set(inp.outlier_cols.tolist())
