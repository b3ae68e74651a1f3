"""Pins of the MX (block-scaled FP8) oracle (CPU only): closed forms of the shared exponent, exact
round trips, a brute-force nearest search, scale invariance, and the block-scaled linear layer
against the per-row oracle, hand-computed blocks and permutation weights."""
import numpy as np
import pytest

from oracle import EPI_BIAS, EPI_GELU_TANH, decode_table, gelu_tanh, linear_ref
from oracle.mx import MX_BLOCK, dequantize_mx, linear_mx_ref, quantize_mx, shared_exponent
from workloads import bf16_bits_to_f32, f32_to_bf16_bits


def _bf16(a):
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(a, np.float32)))


def test_shared_exponent_closed_forms():
    amax = np.array([0.0, 1.0, 1.5, 255.9, 256.0, 448.0, 511.0, 512.0, 2.0 ** -126, 2.0 ** -133,
                     3.0e38, 2.0 ** -119])
    want = [-127, -8, -8, -1, 0, 0, 0, 1, -127, -127, 127 - 8, -127]
    # 2^-126 -> -134 and 2^-119 -> -127 clamp to -127; 3e38 = 1.76 * 2^127
    assert shared_exponent(amax).tolist() == want


def test_landmark_blocks():
    rows = np.zeros((5, 32), np.float32)
    rows[0] = 1.0                      # amax 1: scale 2^-8, every value 256 -> 0x78
    rows[1, 0] = 448.0                 # amax 448: scale 2^0, 0x7E; zeros stay 0x00
    rows[2, 0], rows[2, 1:] = 500.0, 1.0   # 500 / 1 saturates to 448; 1.0 -> 0x38
    rows[3] = -0.0                     # an all-zero block: smallest scale, signed zeros
    rows[4, 0] = 2.0 ** -130           # tiny block: scale clamps at 2^-127, 2^-3 -> 0x20
    q, s = quantize_mx(rows)
    assert s.ravel().tolist() == [119, 127, 127, 0, 0]
    assert np.all(q[0] == 0x78)
    assert q[1, 0] == 0x7E and np.all(q[1, 1:] == 0)
    assert q[2, 0] == 0x7E and np.all(q[2, 1:] == 0x38)
    assert np.all(q[3] == 0x80)
    assert q[4, 0] == 0x20


def test_exact_round_trip():
    """Values dec(c) 2^j whose block maximum sits in E4M3's top binade ([256, 448]) come back
    as the same codes with scale j."""
    rng = np.random.default_rng(1)
    R, K = 24, 128
    codes = rng.integers(0, 0x7F, size=(R, K), dtype=np.int64)
    codes[codes == 0x7F] = 0x7E
    codes |= rng.integers(0, 2, size=(R, K)) << 7
    blocks = codes.reshape(R, K // MX_BLOCK, MX_BLOCK)
    top = rng.integers(0x78, 0x7F, size=blocks.shape[:2])       # 256 .. 448
    blocks[:, :, 5] = top | (rng.integers(0, 2, size=top.shape) << 7)
    codes = blocks.reshape(R, K).astype(np.uint8)
    j = rng.integers(-100, 100, size=(R, K // MX_BLOCK))
    x = decode_table()[codes].reshape(R, K // MX_BLOCK, MX_BLOCK) * np.ldexp(1.0, j)[..., None]
    x = x.reshape(R, K).astype(np.float32)
    assert np.all(_bf16(x) == x)                    # 4-bit significands are bf16 values
    q, s = quantize_mx(x)
    zero = (codes & 0x7F) == 0                      # +-0 keep their sign bit
    assert np.array_equal(q[~zero], codes[~zero])
    assert np.array_equal(s.astype(np.int64) - 127, j)


def test_elements_are_the_nearest_e4m3_value():
    """Brute force: every code is the finite E4M3 value nearest to x / 2^shared (ties to the even
    code, saturating at 448), checked against all 254 finite magnitudes."""
    rng = np.random.default_rng(2)
    x = _bf16(rng.standard_normal((40, 64)) * np.exp(rng.uniform(-8, 8, (40, 1))))
    q, s = quantize_mx(x)
    table = decode_table()
    mags = np.array([table[c] for c in range(0x7F)])            # 0x00 .. 0x7E
    sh = (s.astype(np.int64) - 127).repeat(MX_BLOCK, axis=1)
    quot = x.astype(np.float64) * np.ldexp(1.0, -sh)
    for v, c in zip(quot.ravel(), q.ravel()):
        a = min(abs(v), 448.0)
        d = np.abs(mags - a)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else best[best % 2 == 0][0]
        assert (c & 0x7F) == want and (c >> 7) == (1 if np.signbit(v) else 0)


def test_scaling_by_powers_of_two():
    rng = np.random.default_rng(3)
    x = _bf16(rng.standard_normal((8, 96)))
    q0, s0 = quantize_mx(x)
    for t in (-20, -3, 5, 40):
        q1, s1 = quantize_mx((x * np.float32(2.0 ** t)).astype(np.float32))
        assert np.array_equal(q0, q1)
        assert np.array_equal(s1.astype(np.int64), s0.astype(np.int64) + t)


def test_dequantized_error_bound():
    """E4M3 keeps 3 mantissa bits: each element is off by at most 2^-4 of its value in the normal
    range, or by half the subnormal step 2^(shared - 10); saturated ones by less than 2^(shared+6)."""
    rng = np.random.default_rng(4)
    x = _bf16(rng.standard_normal((16, 128)) * 3.0)
    q, s = quantize_mx(x)
    xd = dequantize_mx(q, s)
    sh = (s.astype(np.int64) - 127).repeat(MX_BLOCK, axis=1).astype(np.float64)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, np.ldexp(1.0, (sh - 10).astype(np.int64)))
    bound = np.maximum(bound, np.where(np.abs(x) * np.ldexp(1.0, -sh.astype(np.int64)) > 448,
                                       np.ldexp(1.0, (sh + 6).astype(np.int64)), 0.0))
    assert np.all(np.abs(xd - x) <= bound)


def test_unit_scales_match_the_row_oracle():
    """All block scales 2^0: the block-scaled layer is the per-row oracle with unit scales."""
    rng = np.random.default_rng(5)
    M, N, K = 6, 5, 96
    qa = rng.integers(0, 256, size=(M, K), dtype=np.uint8)
    qw = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x01
    qw[(qw & 0x7F) == 0x7F] = 0x02
    ones_a = np.full((M, K // 32), 127, np.uint8)
    ones_w = np.full((N, K // 32), 127, np.uint8)
    bias = _bf16(rng.standard_normal(N))
    for epi in (EPI_BIAS, EPI_GELU_TANH):
        got = linear_mx_ref(qa, ones_a, qw, ones_w, bias, epi)
        want = linear_ref(qa, np.ones(M, np.float32), qw, np.ones(N, np.float32), bias, epi)
        assert np.allclose(got, want, rtol=1e-13, atol=1e-13)


def test_block_scales_by_hand():
    """One row against one weight row, two blocks: 2^(ea0 + ew0) * 32 * 1 * 1.5 +
    2^(ea1 + ew1) * 32 * 2 * (-0.5)."""
    qa = np.concatenate([np.full(32, 0x38), np.full(32, 0x40)]).astype(np.uint8)[None]   # 1, 2
    qw = np.concatenate([np.full(32, 0x3C), np.full(32, 0xB0)]).astype(np.uint8)[None]   # 1.5, -0.5
    sa = np.array([[127 + 3, 127 - 2]], np.uint8)
    sw = np.array([[127 - 1, 127 + 5]], np.uint8)
    want = 2.0 ** 2 * 32 * 1.5 + 2.0 ** 3 * 32 * 2 * (-0.5)
    assert linear_mx_ref(qa, sa, qw, sw)[0, 0] == want


def test_permutation_weights_pick_columns():
    """Weight row n is one code 1.0 (0x38) at column p[n] with block scale 2^t[n]: output n is
    the dequantized activation at column p[n] times 2^t[n]."""
    rng = np.random.default_rng(6)
    M, K, N = 7, 128, 9
    x = _bf16(rng.standard_normal((M, K)))
    qa, sa = quantize_mx(x)
    p = rng.choice(K, N, replace=False)
    t = rng.integers(-4, 5, N)
    qw = np.zeros((N, K), np.uint8)
    qw[np.arange(N), p] = 0x38
    sw = np.full((N, K // 32), 127, np.uint8)
    sw[np.arange(N), p // 32] = 127 + t
    got = linear_mx_ref(qa, sa, qw, sw)
    xd = dequantize_mx(qa, sa)
    assert np.array_equal(got, xd[:, p] * np.ldexp(1.0, t)[None, :])
    gl = linear_mx_ref(qa, sa, qw, sw, np.zeros(N, np.float32), EPI_GELU_TANH)
    assert np.allclose(gl, gelu_tanh(xd[:, p] * np.ldexp(1.0, t)[None, :]), rtol=0, atol=0)


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        quantize_mx(np.zeros((2, 40), np.float32))
