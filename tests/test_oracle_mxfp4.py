"""Pins of the MXFP4 (block-scaled E2M1) oracle, CPU only.

Each pin reaches the oracle's result by a route other than its own arithmetic: the element
encoding against a count of rounding thresholds (the midpoints of E2M1, strict or not by the
tie-to-even rule) over every bf16 value at scale 1; closed forms of the shared exponent; landmark
blocks worked by hand; exact round trips; invariance under powers of two; the nibble packing
against a hand-written byte; the layer against an integer matrix product (twice every E2M1 value
is an integer) and against permutation weights.
"""
import numpy as np

from oracle import EPI_BIAS, EPI_GELU_TANH, gelu_tanh
from oracle.mxfp4 import (MX_BLOCK, decode_fp4_table, dequantize_mxfp4, encode_fp4,
                          linear_mxfp4_ref, pack_fp4, quantize_mxfp4, shared_exponent4,
                          unpack_fp4)
from workloads import bf16_bits_to_f32, f32_to_bf16_bits


def _bf16(a):
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(a, np.float32)))


def _threshold_code(v):
    """E2M1 magnitude code by counting the midpoints below |v|: a midpoint whose lower neighbour
    has the even code is passed only strictly (the tie goes down), the others at equality too."""
    a = np.abs(np.asarray(v, np.float64))
    c = ((a > 0.25).astype(int) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5)
         + (a >= 3.5) + (a > 5.0))
    return (c + 8 * np.signbit(v)).astype(np.uint8)


def test_decode_table():
    t = decode_fp4_table()
    assert t[:8].tolist() == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert t[8:].tolist() == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    # E2M1 with exponent bias 1: code = 2 e + m, value (1 + m / 2) 2^(e - 1), subnormal 0.5 m
    for c in range(1, 8):
        e, m = c >> 1, c & 1
        want = 0.5 * m if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
        assert t[c] == want


def test_encode_every_bf16_value_at_scale_one():
    """Every finite bf16 value, positive and negative: the nearest-magnitude code with ties to
    even equals the threshold count."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bf16_bits_to_f32(bits)
    v = v[np.isfinite(v)]
    assert np.array_equal(encode_fp4(v), _threshold_code(v))


def test_midpoints_and_saturation():
    v = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 7.99, 0.2499, 0.2501,
                  -0.1, -0.75, -5.0, -7.5])
    want = [0, 2, 2, 4, 4, 6, 6, 7, 7, 7, 0, 1, 8, 10, 14, 15]
    assert encode_fp4(v).tolist() == want


def test_shared_exponent_closed_forms():
    amax = np.array([0.0, 1.0, 4.0, 6.0, 7.99, 8.0, 0.75, 2.0 ** -126, 2.0 ** -124, 2.0 ** -125,
                     3.0e38, 2.0 ** -130])
    # floor(log2 a) - 2, clamped to [-127, 127]
    want = [-127, -2, 0, 0, 0, 1, -3, -127, -126, -127, 125, -127]
    assert shared_exponent4(amax).tolist() == want


def test_landmark_blocks():
    rows = np.zeros((5, 32), np.float32)
    rows[0] = 1.0                              # amax 1: scale 2^-2, 1 / 2^-2 = 4 -> code 6
    rows[1, :4] = [6.0, 3.0, 1.0, 0.5]         # amax 6: scale 1: codes 7, 5, 2, 1; zeros 0
    rows[2, 0], rows[2, 1] = 7.0, -2.5         # amax 7: scale 1: 7 saturates to 6, -2.5 -> -2
    rows[3] = -0.0                             # all-zero block: scale 2^-127, signed zeros
    rows[4, 0], rows[4, 1] = 2.0 ** -130, 2.0 ** -131   # clamps at 2^-127: 2^-3 -> 0, 2^-4 -> 0
    q, s = quantize_mxfp4(rows)
    codes = unpack_fp4(q)
    assert s.ravel().tolist() == [125, 127, 127, 0, 0]
    assert np.all(codes[0] == 6)
    assert codes[1, :4].tolist() == [7, 5, 2, 1] and np.all(codes[1, 4:] == 0)
    assert codes[2, :2].tolist() == [7, 12] and np.all(codes[2, 2:] == 0)
    assert np.all(codes[3] == 8)
    assert codes[4, :2].tolist() == [0, 0]


def test_packing_order():
    codes = np.array([[1, 2, 3, 4, 15, 0] + [0] * 26], np.uint8)
    p = pack_fp4(codes)
    assert p[0, :3].tolist() == [0x21, 0x43, 0x0F]
    assert np.array_equal(unpack_fp4(p), codes)


def test_exact_round_trip():
    """Blocks of values dec(c) 2^j whose largest magnitude sits in the top binade [4, 8) come back
    as the same codes with scale byte j + 127."""
    rng = np.random.default_rng(7)
    R, K = 16, 128
    codes = rng.integers(0, 16, size=(R, K)).astype(np.uint8)
    codes[:, ::MX_BLOCK] = 6 + rng.integers(0, 2, size=(R, K // MX_BLOCK))   # 4 or 6 leads
    j = rng.integers(-100, 100, size=(R, K // MX_BLOCK))
    x = decode_fp4_table()[codes].reshape(R, K // MX_BLOCK, MX_BLOCK) * np.ldexp(1.0, j)[..., None]
    q, s = quantize_mxfp4(x.reshape(R, K).astype(np.float32))
    assert np.array_equal(unpack_fp4(q), codes)
    assert np.array_equal(s.astype(np.int64), j + 127)


def test_power_of_two_invariance_and_error_bound():
    rng = np.random.default_rng(8)
    x = _bf16(rng.standard_normal((8, 256)) * np.exp(rng.uniform(-8, 8, size=(8, 1))))
    q, s = quantize_mxfp4(x)
    for t in (-20, -1, 3, 40):
        q2, s2 = quantize_mxfp4((x * 2.0 ** t).astype(np.float32))
        assert np.array_equal(q2, q)
        assert np.array_equal(s2.astype(int), s.astype(int) + t)
    # each value within half the E2M1 spacing of its binade (x 2^shared), or saturated at 6
    dq = dequantize_mxfp4(q, s)
    e = s.astype(np.int64).repeat(MX_BLOCK, axis=1) - 127
    a = np.abs(x.astype(np.float64)) * np.ldexp(1.0, -e)
    half = np.where(a < 2.0, 0.25, np.where(a < 4.0, 0.5, 1.0))
    err = np.abs(dq - x) * np.ldexp(1.0, -e)
    assert np.all((err <= half) | ((a > 6.0) & (np.abs(err - (a - 6.0)) == 0)))


def test_layer_against_integer_product():
    """With every scale byte 127 the layer is the product of decoded values: twice each E2M1
    value is an integer, so the integer product / 4 is the exact result."""
    rng = np.random.default_rng(9)
    M, N, K = 7, 9, 96
    ca = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    cw = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    sa = np.full((M, K // MX_BLOCK), 127, np.uint8)
    sw = np.full((N, K // MX_BLOCK), 127, np.uint8)
    twice = np.array([0, 1, 2, 3, 4, 6, 8, 12], np.int64)
    ia = np.where(ca >= 8, -twice[ca & 7], twice[ca & 7])
    iw = np.where(cw >= 8, -twice[cw & 7], twice[cw & 7])
    want = (ia @ iw.T).astype(np.float64) / 4.0
    bias = _bf16(rng.standard_normal(N))
    got = linear_mxfp4_ref(pack_fp4(ca), sa, pack_fp4(cw), sw, bias, EPI_BIAS)
    assert np.array_equal(got, want + bias.astype(np.float64))
    g = linear_mxfp4_ref(pack_fp4(ca), sa, pack_fp4(cw), sw, None, EPI_GELU_TANH)
    assert np.allclose(g, gelu_tanh(want), rtol=0, atol=0)


def test_block_scales_and_permutation_weights():
    """One-hot weight rows pick a column of A, times the weight block's scale and 6 (code 7):
    out[m, n] = dec(a[m, p(n)]) 2^(ea[m, b] + ew[n, b]) 6, with b the block of p(n)."""
    rng = np.random.default_rng(10)
    M, N, K = 5, 64, 128
    ca = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    sa = rng.integers(120, 135, size=(M, K // MX_BLOCK)).astype(np.uint8)
    perm = rng.permutation(K)[:N]
    cw = np.zeros((N, K), np.uint8)
    cw[np.arange(N), perm] = 7
    sw = rng.integers(124, 131, size=(N, K // MX_BLOCK)).astype(np.uint8)
    got = linear_mxfp4_ref(pack_fp4(ca), sa, pack_fp4(cw), sw)
    b = perm // MX_BLOCK
    a_val = decode_fp4_table()[ca[:, perm]]
    scale = np.ldexp(1.0, sa[:, b].astype(int) - 127 + sw[np.arange(N), b].astype(int) - 127)
    assert np.array_equal(got, a_val * scale * 6.0)


def test_gated_residual_epilogue():
    """The gated epilogue against the bias one: gate 0 returns the residual exactly, gate 1 with
    a zero residual the bias epilogue's value, and a hand-worked row r + g (sum + bias)."""
    from oracle import EPI_GATED_RESIDUAL
    rng = np.random.default_rng(13)
    M, N, K = 6, 8, 64
    ca = rng.integers(0, 16, size=(M, K)).astype(np.uint8)
    cw = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    sa = rng.integers(124, 131, size=(M, K // MX_BLOCK)).astype(np.uint8)
    sw = rng.integers(124, 131, size=(N, K // MX_BLOCK)).astype(np.uint8)
    bias = _bf16(rng.standard_normal(N))
    res = _bf16(rng.standard_normal((M, N)))
    args = (pack_fp4(ca), sa, pack_fp4(cw), sw, bias)
    v = linear_mxfp4_ref(*args, EPI_BIAS)
    assert np.array_equal(linear_mxfp4_ref(*args, EPI_GATED_RESIDUAL, np.zeros(N), res), res)
    assert np.array_equal(linear_mxfp4_ref(*args, EPI_GATED_RESIDUAL, np.ones(N),
                                           np.zeros((M, N))), v)
    # one weight row of code 2 (1.0) at K position 0 only, unit scales: v = a[:, 0] + bias
    cw1 = np.zeros((1, K), np.uint8); cw1[0, 0] = 2
    ca1 = np.zeros((2, K), np.uint8); ca1[0, 0], ca1[1, 0] = 5, 14     # 3.0 and -4.0
    one = np.full((2, K // MX_BLOCK), 127, np.uint8)
    g = linear_mxfp4_ref(pack_fp4(ca1), one, pack_fp4(cw1), one[:1], np.array([0.5]),
                         EPI_GATED_RESIDUAL, np.array([2.0]), np.array([[1.0], [-1.0]]))
    assert g.ravel().tolist() == [1.0 + 2.0 * 3.5, -1.0 + 2.0 * (-3.5)]
