"""Pins of the oracle's LayerNorm + modulation + quantization step (CPU only).

Expected values come from closed forms (alternating, constant and arithmetic-progression rows,
whose mean and variance are known exactly), from a library LayerNorm evaluated in float64, and
from invariants of the normalization. A dropped "1 +" in the modulation, a swapped scale and
shift, the unbiased variance or a missing eps each fail at least one of them.
"""
import numpy as np
import pytest
import torch

from oracle import LN_EPS, layernorm_modulate, modulate_rows, quantize_rows
from workloads import bf16_bits_to_f32, f32_to_bf16_bits


def _vec(rng, K, sd):
    # bf16 values, as the modulation vectors are
    return bf16_bits_to_f32(f32_to_bf16_bits(rng.normal(0.0, sd, K).astype(np.float32)))


@pytest.mark.parametrize("K,c", [(2, 1.0), (64, 3.5), (3072, 0.25), (3072, 1e-3)])
def test_alternating_rows_closed_form(K, c):
    """x = (c, -c, c, -c, ...): mean 0, variance c^2, so y_k = +-c / sqrt(c^2 + eps) (1 + s_k) + t_k."""
    rng = np.random.default_rng(K)
    s, t = _vec(rng, K, 0.3), _vec(rng, K, 0.5)
    x = np.tile([c, -c], K // 2)[None, :]
    y = layernorm_modulate(x, s, t)
    sign = np.tile([1.0, -1.0], K // 2)
    want = sign * c / np.sqrt(c * c + LN_EPS) * (1.0 + s.astype(np.float64)) + t
    assert np.allclose(y[0], want, rtol=1e-13, atol=1e-13)


def test_constant_row_gives_the_shift():
    """Every deviation from the mean is exactly zero, so y = shift exactly."""
    rng = np.random.default_rng(2)
    K = 96
    s, t = _vec(rng, K, 0.3), _vec(rng, K, 0.5)
    for v in (0.0, 1.5, -7.25, 1e-20):
        y = layernorm_modulate(np.full((1, K), v), s, t)
        assert np.array_equal(y[0], t.astype(np.float64))


@pytest.mark.parametrize("K,a,d", [(16, 0.0, 1.0), (3072, -2.0, 0.001), (1000, 5.0, -0.03)])
def test_arithmetic_progression_closed_form(K, a, d):
    """x_k = a + d k: mean a + d (K - 1) / 2 and variance d^2 (K^2 - 1) / 12."""
    rng = np.random.default_rng(K)
    s, t = _vec(rng, K, 0.2), _vec(rng, K, 0.2)
    k = np.arange(K, dtype=np.float64)
    y = layernorm_modulate((a + d * k)[None, :], s, t)
    dev = d * (k - (K - 1) / 2.0)
    want = dev / np.sqrt(d * d * (K * K - 1) / 12.0 + LN_EPS) * (1.0 + s.astype(np.float64)) + t
    assert np.allclose(y[0], want, rtol=1e-10, atol=1e-12)


def test_matches_library_layernorm():
    """torch's LayerNorm (no affine) in float64, then the modulation."""
    rng = np.random.default_rng(5)
    R, K = 7, 3072
    x = rng.normal(0.0, 1.0, (R, K))
    x[:, rng.choice(K, 30, replace=False)] *= 30.0
    s, t = _vec(rng, K, 0.3), _vec(rng, K, 0.5)
    ln = torch.nn.functional.layer_norm(torch.from_numpy(x), (K,), eps=LN_EPS).numpy()
    want = ln * (1.0 + s.astype(np.float64)) + t
    assert np.allclose(layernorm_modulate(x, s, t), want, rtol=1e-12, atol=1e-12)


def test_invariant_to_affine_input_changes():
    """LayerNorm removes the mean and the scale: a x + b gives the same y when eps is negligible."""
    rng = np.random.default_rng(9)
    K = 512
    x = rng.normal(0.0, 1.0, (3, K))
    s, t = _vec(rng, K, 0.3), _vec(rng, K, 0.5)
    y0 = layernorm_modulate(x, s, t, eps=0.0)
    y1 = layernorm_modulate(4.0 * x - 11.0, s, t, eps=0.0)
    assert np.allclose(y0, y1, rtol=1e-12, atol=1e-12)


def test_rounds_to_bf16_then_quantizes_rows():
    """y is the nearest bf16 of the float64 value, and the codes are those of quantize_rows(y)."""
    rng = np.random.default_rng(13)
    R, K = 5, 256
    x = rng.normal(0.0, 2.0, (R, K))
    s, t = _vec(rng, K, 0.3), _vec(rng, K, 0.5)
    y, q, qs = modulate_rows(x, s, t)
    exact = layernorm_modulate(x, s, t)
    assert np.array_equal(bf16_bits_to_f32(f32_to_bf16_bits(y)), y)          # bf16 values
    assert np.all(np.abs(y - exact) <= np.abs(exact) * 2.0 ** -8 + 1e-40)     # half a bf16 step
    q2, s2 = quantize_rows(y)
    assert np.array_equal(q, q2) and np.array_equal(qs.view(np.uint32), s2.view(np.uint32))
