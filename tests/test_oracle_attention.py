"""Pins of the oracle's FP8 attention (CPU only): a library attention, closed forms and
invariants that do not reuse the oracle's formula."""
import numpy as np
import pytest
import torch

from oracle import decode_table, quantize_rows
from oracle.attention import HEAD_DIM, attention_fp8_ref, attention_ref, quantize_heads
from workloads import bf16_bits_to_f32, f32_to_bf16_bits

D = HEAD_DIM


def _bf16(a):
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(a, np.float32)))


def _qkv(H, S, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return tuple(_bf16(rng.standard_normal((H, S, D)) * scale) for _ in range(3))


def _dequant(codes, scales):
    return decode_table()[codes] * scales[..., None].astype(np.float64)


def test_quantize_heads_is_row_quantization():
    q, _, _ = _qkv(3, 5, 1)
    c, s = quantize_heads(q)
    c2, s2 = quantize_rows(q.reshape(15, D))
    assert np.array_equal(c.reshape(15, D), c2) and np.array_equal(s.reshape(15), s2)


def test_single_key_returns_its_value():
    q, k, v = _qkv(2, 1, 2)
    o, _, _, (v8, sv) = attention_fp8_ref(q, k, v)
    assert np.array_equal(o, _dequant(v8, sv))


def test_identical_keys_average_the_values():
    """Equal keys give equal logits: every weight is 1/S and o is the mean of the values."""
    H, S = 2, 37
    q, _, v = _qkv(H, S, 3)
    k = np.repeat(_qkv(H, 1, 4)[0], S, axis=1)
    o, _, _, (v8, sv) = attention_fp8_ref(q, k, v)
    want = _dequant(v8, sv).mean(axis=1, keepdims=True)
    assert np.allclose(o, np.broadcast_to(want, o.shape), rtol=1e-12, atol=1e-14)


def test_a_dominant_key_selects_its_value():
    """Key j* aligned with every query at 40 logit units above the others: o = v_j* to e^-40."""
    H, S = 1, 16
    rng = np.random.default_rng(5)
    v = _bf16(rng.standard_normal((H, S, D)))
    q = np.zeros((H, S, D), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((H, S, D), np.float32)
    k[0, 7, 0] = 40.0 * np.sqrt(D)             # logit 40 for key 7, 0 for the others
    o, _, _, (v8, sv) = attention_fp8_ref(q, k, _bf16(v))
    vd = _dequant(v8, sv)
    assert np.allclose(o, np.broadcast_to(vd[:, 7:8], o.shape), rtol=0, atol=1e-15 * S
                       + np.abs(vd).max() * S * np.exp(-40.0) * 2)


def test_matches_library_attention():
    H, S = 3, 50
    q, k, v = _qkv(H, S, 6, scale=3.0)
    o, (q8, sq), (k8, sk), (v8, sv) = attention_fp8_ref(q, k, v)
    lib = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(_dequant(q8, sq)), torch.from_numpy(_dequant(k8, sk)),
        torch.from_numpy(_dequant(v8, sv)))
    assert np.allclose(o, lib.numpy(), rtol=1e-11, atol=1e-13)


def test_permutation_invariance():
    H, S = 2, 23
    q, k, v = _qkv(H, S, 7)
    o = attention_fp8_ref(q, k, v)[0]
    perm = np.random.default_rng(8).permutation(S)
    o_kv = attention_fp8_ref(q, k[:, perm], v[:, perm])[0]
    assert np.allclose(o, o_kv, rtol=1e-12, atol=1e-14)       # keys and values together
    o_q = attention_fp8_ref(q[:, perm], k, v)[0]
    assert np.allclose(o[:, perm], o_q, rtol=1e-12, atol=1e-14)  # queries permute the output


def test_outputs_are_convex_combinations_of_values():
    H, S = 2, 41
    q, k, v = _qkv(H, S, 9, scale=4.0)
    o, _, _, (v8, sv) = attention_fp8_ref(q, k, v)
    vd = _dequant(v8, sv)
    lo, hi = vd.min(axis=1, keepdims=True), vd.max(axis=1, keepdims=True)
    assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)


def test_uses_the_quantized_operands():
    """The result is the attention of the decoded codes, not of the bf16 inputs: it differs from
    the unquantized attention, by no more than the quantization error allows."""
    H, S = 2, 30
    q, k, v = _qkv(H, S, 10)
    o = attention_fp8_ref(q, k, v)[0]
    exact = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(a.astype(np.float64)) for a in (q, k, v))).numpy()
    assert not np.allclose(o, exact, rtol=1e-6, atol=1e-9)
    # E4M3 rounds each operand by at most 2^-4 of its value
    assert np.max(np.abs(o - exact)) < 0.25 * np.max(np.abs(exact))
