"""GPU parity of the block-scaled (MX) FP8 path (dq_quantize_mx_fp8, dq_linear_mx_fp8) against the
oracle.

Codes and scale bytes must equal the oracle's bit for bit. The linear layer's output is
compared with the oracle's float64 value of the layer on the same codes and scales within the
output tolerance of the FP8 linear layer, |out - ref| <= 4e-3 |ref| + 1e-3 rms(ref): the
accumulation is fp32 (each block product is exact in the matrix unit, the block sums carry a
few fp32 ulps) and the output is one bf16 rounding; on inputs whose sums are exact in fp32 the
output must equal the bf16 rounding of the exact value.
"""
import numpy as np
import pytest
import torch

import fp8_dynamic_quant_amd as dq
from oracle import EPI_BIAS, EPI_GELU_TANH, round_to_bf16
from oracle.mx import dequantize_mx, linear_mx_ref, quantize_mx
from gpu_util import (announce, assert_within_tolerance, bf16_to_dev, dev_to_bf16_bits, dev_to_f64,
                      require_gpu, u8_to_dev)
from workloads import bf16_bits_to_f32, f32_to_bf16_bits, make_rows

pytestmark = pytest.mark.gpu

EPI = {"bias": EPI_BIAS, "gelu_tanh": EPI_GELU_TANH}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _quant(x16):
    q, s = dq.dq_quantize_mx_fp8(bf16_to_dev(x16))
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def _check_quant(x16, what):
    announce(f"mx quantize {what} {x16.shape}")
    gq, gs = _quant(x16)
    q, s = quantize_mx(bf16_bits_to_f32(x16))
    assert np.array_equal(gs, s), f"{what}: scale bytes differ at {np.argwhere(gs != s)[:4]}"
    bad = np.argwhere(gq != q)
    assert bad.size == 0, f"{what}: codes differ at {bad[:4]}: {gq[tuple(bad[0])]:#x} vs {q[tuple(bad[0])]:#x}"
    return q, s


@pytest.mark.parametrize("M,K", [(1, 32), (3, 64), (17, 96), (64, 3072), (33, 1056)])
def test_quantize_random_rows(M, K):
    rng = np.random.default_rng([M, K])
    x = rng.standard_normal((M, K)).astype(np.float32) * np.exp(rng.uniform(-20, 20, (M, 1)))
    _check_quant(f32_to_bf16_bits(x.astype(np.float32)), "random")


def test_quantize_edge_blocks():
    """Zero blocks (+0 and -0), one nonzero, subnormal and huge amax, saturating blocks (the top
    binade past 448), values at every E4M3 rounding midpoint."""
    K = 32
    rows = []
    rows.append(np.zeros(K))
    rows.append(-np.zeros(K))
    r = np.zeros(K); r[7] = -3.0; rows.append(r)
    rows.append(np.full(K, 2.0 ** -133) * np.where(np.arange(K) % 2, 1, -1))   # bf16 subnormals
    rows.append(np.full(K, 2.0 ** 127) * 1.5)
    r = np.linspace(-500, 500, K); rows.append(r)                                 # 500 saturates
    r = np.full(K, 496.0); r[1::2] = 480.0; rows.append(r)                          # all past 448
    r = (np.arange(K) + 0.5) * 2.0 ** -9                  # E4M3 subnormal midpoints at scale 2^0
    r[0] = 256.0; rows.append(r)
    x = np.array(rows, dtype=np.float32)
    _check_quant(f32_to_bf16_bits(x), "edges")


def test_quantize_activations_full_size():
    x = make_rows(4608, 3072, seed=21)
    _check_quant(x, "flux hidden 4608x3072")


def _linear(q, s, qw, sw, bias16, epi):
    out = dq.dq_linear_mx_fp8(u8_to_dev(q), u8_to_dev(s), u8_to_dev(qw), u8_to_dev(sw),
                              None if bias16 is None else bf16_to_dev(bias16), epi)
    torch.cuda.synchronize()
    return out


def _end_to_end(M, K, N, epi, seed, bias=True, rows=None):
    rng = np.random.default_rng([seed, M, K, N])
    x = rng.standard_normal((M, K)).astype(np.float32)
    cols = rng.choice(K, max(1, K // 100), replace=False)
    x[:, cols] *= 30.0
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    b16 = f32_to_bf16_bits((rng.standard_normal(N) * 0.01).astype(np.float32)) if bias else None
    x16, w16 = f32_to_bf16_bits(x), f32_to_bf16_bits(w)
    announce(f"mx linear {M}x{K}x{N} {epi} bias={bias}")
    q, s = _check_quant(x16, "activations")
    qw, sw = _check_quant(w16, "weights")
    out = dev_to_f64(_linear(q, s, qw, sw, b16, epi))
    rows = np.arange(M) if rows is None else np.asarray(rows)
    ref = linear_mx_ref(q[rows], s[rows], qw, sw, None if b16 is None else bf16_bits_to_f32(b16),
                        EPI[epi])
    assert_within_tolerance(out[rows], ref, what=f"mx {M}x{K}x{N} {epi}")
    return out


@pytest.mark.parametrize("M,K,N", [(64, 128, 64), (1, 256, 192), (255, 384, 320), (257, 1024, 256),
                                   (300, 640, 512), (513, 128, 64), (300, 2048, 576),
                                   (40, 512, 128)])
@pytest.mark.parametrize("epi", ["bias", "gelu_tanh"])
def test_tiles_and_ragged_tails(M, K, N, epi):
    """K steps of 128 a multiple of 4 (K = 512, 1024, 2048) take the grouped scale copies, the
    others the per-step ones."""
    _end_to_end(M, K, N, epi, seed=1)


def test_without_bias():
    _end_to_end(96, 256, 128, "bias", seed=2, bias=False)


def test_mlp_up_full_size_sampled_rows():
    """4608 x 3072 -> 12288 with the GELU epilogue, 64 sampled rows against the oracle."""
    rows = np.unique(np.concatenate([[0, 255, 256, 4607],
                                     np.random.default_rng(5).choice(4608, 60, replace=False)]))
    _end_to_end(4608, 3072, 12288, "gelu_tanh", seed=3, rows=rows)


@pytest.mark.parametrize("K", [256, 512])
def test_more_tiles_than_compute_units_ragged(K):
    """4608 x 3648 (18 x 15 tiles, the last tile column 64 wide): more tiles than compute units,
    so the 14 tiles left after the first round run as narrow halves (per-step scale copies at
    K = 256, grouped at K = 512)."""
    rows = np.unique(np.concatenate([[0, 4095, 4096, 4607],
                                     np.random.default_rng(6).choice(4608, 44, replace=False)]))
    _end_to_end(4608, K, 3648, "bias", seed=4, rows=rows)


@pytest.mark.parametrize("steps", [131070, 131068])
def test_longest_k(steps):
    """M = 3, K = 16776960 (the longest the layer accepts: 131070 steps of 128; per-step scale
    copies) and 131068 steps (grouped scale copies), N = 64: random codes and scale bytes
    127 +- 6, against the oracle summed over K chunks of 131072."""
    rng = np.random.default_rng(32)
    M, K, N = 3, steps * 128, 64
    q = rng.integers(0, 256, size=(M, K), dtype=np.uint8)
    qw = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x01
    qw[(qw & 0x7F) == 0x7F] = 0x02
    s = (127 + rng.integers(-6, 7, (M, K // 32))).astype(np.uint8)
    sw = (127 + rng.integers(-6, 7, (N, K // 32))).astype(np.uint8)
    announce(f"mx longest K {M}x{K}x{N}")
    out = dev_to_f64(_linear(q, s, qw, sw, None, "bias"))
    ref = None
    for k0 in range(0, K, 131072):
        k1 = min(K, k0 + 131072)
        part = linear_mx_ref(q[:, k0:k1], s[:, k0 // 32:k1 // 32], qw[:, k0:k1],
                             sw[:, k0 // 32:k1 // 32])
        ref = part if ref is None else ref + part
    assert_within_tolerance(out, ref, what="mx longest K")


def _small_codes(rng, shape):
    """Codes of values in [1, 2) with random signs."""
    mant = rng.integers(0, 8, size=shape)
    sign = rng.integers(0, 2, size=shape) << 7
    return (sign | (7 << 3) | mant).astype(np.uint8)


def _one_per_half(rng, codes):
    """Keep one code per row in every 64-wide K half (one matrix instruction's reach): each
    instruction then adds a single exact product."""
    R, K = codes.shape
    keep = np.zeros_like(codes)
    pos = rng.integers(0, 64, size=(R, K // 64)) + 64 * np.arange(K // 64)[None, :]
    keep[np.arange(R)[:, None], pos] = codes[np.arange(R)[:, None], pos]
    return keep


@pytest.mark.parametrize("M,K,N", [(128, 256, 128), (300, 512, 320)])
def test_exact_inputs_are_bit_exact(M, K, N):
    """Activations with one nonzero code per 64-wide K half, block scales 2^(-3..3) per operand:
    each instruction adds one product, a multiple of 2^-12 below 2^8, so the fp32 sums (at most
    K / 64 terms, below 2^11) are exact and the output is the bf16 rounding of the exact value."""
    rng = np.random.default_rng(M + K + N)
    q, qw = _one_per_half(rng, _small_codes(rng, (M, K))), _small_codes(rng, (N, K))
    s = (127 + rng.integers(-3, 4, (M, K // 32))).astype(np.uint8)
    sw = (127 + rng.integers(-3, 4, (N, K // 32))).astype(np.uint8)
    b16 = f32_to_bf16_bits((rng.integers(-64, 64, N) * 2.0 ** -6).astype(np.float32))
    announce(f"mx exact {M}x{K}x{N}")
    out = _linear(q, s, qw, sw, b16, "bias")
    ref = linear_mx_ref(q, s, qw, sw, bf16_bits_to_f32(b16), EPI_BIAS)
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)
    want = f32_to_bf16_bits(round_to_bf16(ref).astype(np.float32))
    assert np.array_equal(dev_to_bf16_bits(out), want)


def test_permutation_weights_pick_columns():
    """One-hot weight rows (code 1.0 at column p[n], block scale 2^t[n]): output column n is the
    dequantized activation at p[n] times 2^t[n], rounded to bf16."""
    rng = np.random.default_rng(9)
    M, K, N = 200, 512, 192
    x16 = f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    q, s = _check_quant(x16, "activations")
    p = rng.choice(K, N, replace=False)
    t = rng.integers(-4, 5, N)
    qw = np.zeros((N, K), np.uint8)
    qw[np.arange(N), p] = 0x38
    sw = np.full((N, K // 32), 127, np.uint8)
    sw[np.arange(N), p // 32] = 127 + t
    announce("mx permutation weights")
    out = _linear(q, s, qw, sw, None, "bias")
    want = dequantize_mx(q, s)[:, p] * np.ldexp(1.0, t)[None, :]
    assert np.array_equal(dev_to_bf16_bits(out), f32_to_bf16_bits(round_to_bf16(want).astype(np.float32)))


def test_deterministic_and_m_zero():
    rng = np.random.default_rng(11)
    q = _small_codes(rng, (96, 256))
    qw = _small_codes(rng, (128, 256))
    s = np.full((96, 8), 120, np.uint8)
    sw = np.full((128, 8), 130, np.uint8)
    a = dev_to_bf16_bits(_linear(q, s, qw, sw, None, "gelu_tanh"))
    b = dev_to_bf16_bits(_linear(q, s, qw, sw, None, "gelu_tanh"))
    assert np.array_equal(a, b)
    e = dq.dq_linear_mx_fp8(torch.empty((0, 256), dtype=torch.uint8, device="cuda:0"),
                            torch.empty((0, 8), dtype=torch.uint8, device="cuda:0"),
                            u8_to_dev(qw), u8_to_dev(sw))
    assert e.shape == (0, 128)
