"""QKV projection with query/key RMS normalization and rotary position embedding, fused into the
linear's epilogue. TEST INFRASTRUCTURE ONLY.

The page "Accelerarea generarii de imagini cu FLUX 3 Image Klein pe GPU-urile Blackwell NVIDIA"
(the paragraph on the PrimsTS GEMMs after "Tabelul 1") names, among the epilogues fused into the
quantized GEMMs, the query/key/value projection with query/key normalization and rotary position
embeddings. It gives no formula. The reading taken is the FLUX-style attention input:

  * the linear's output row v[m, :] (dequantized, plus bias, see `linear.py`) holds, in order,
    the query, key and value of H heads of D = 128 channels each: N = 3 H D;
  * query and key are each normalized per head by their root mean square, with a learned
    per-channel scale w of D entries (one for queries, one for keys) and eps = 1e-6:
        r = v_h / sqrt(mean_d(v_h[d]^2) + eps) * w[d]
  * then rotated pairwise: channels (2i, 2i + 1) of a head turn by the angle of token m and pair
    i, given as cos[m, i] and sin[m, i] (the model derives the angles from the token positions):
        out[2i]     = cos * r[2i] - sin * r[2i + 1]
        out[2i + 1] = sin * r[2i] + cos * r[2i + 1]
  * values pass through unchanged;
  * the outputs are laid out head-major, [H, M, D] each (the layout attention reads), and
    rounded once to bf16.

Everything after the contraction is evaluated in float64 here.
"""
import numpy as np

from .linear import EPI_BIAS, linear_ref, round_to_bf16

HEAD_DIM = 128
QK_NORM_EPS = 1e-6


def rms_norm(v, w, eps=QK_NORM_EPS):
    """v / sqrt(mean(v^2) + eps) * w over the last axis, float64. v: [..., D]; w: [D]."""
    v = np.asarray(v, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64).reshape(-1)
    if v.shape[-1] != w.shape[0]:
        raise ValueError("rms_norm: the scale needs one entry per channel")
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps) * w


def rope_pairs(v, cos, sin):
    """Turn channel pairs (2i, 2i + 1) of the last axis by the angle whose cosine and sine are
    cos[m, i], sin[m, i]. v: [M, ..., D] with the token on the first axis; cos, sin: [M, D/2]."""
    v = np.asarray(v, dtype=np.float64)
    M, D = v.shape[0], v.shape[-1]
    if D % 2:
        raise ValueError("rope_pairs: the channel count must be even")
    cos = np.asarray(cos, dtype=np.float64).reshape(M, D // 2)
    sin = np.asarray(sin, dtype=np.float64).reshape(M, D // 2)
    shape = (M,) + (1,) * (v.ndim - 2) + (D // 2,)
    c, s = cos.reshape(shape), sin.reshape(shape)
    a, b = v[..., 0::2], v[..., 1::2]
    out = np.empty_like(v)
    out[..., 0::2] = c * a - s * b
    out[..., 1::2] = s * a + c * b
    return out


def qkv_split_norm_rope(v, heads, norm_q, norm_k, cos, sin, eps=QK_NORM_EPS):
    """The epilogue on the linear's float64 output v [M, 3 H D]: returns (q, k, v) float64, each
    [H, M, D] (head-major)."""
    v = np.asarray(v, dtype=np.float64)
    M, N = v.shape
    D = HEAD_DIM
    if N != 3 * heads * D:
        raise ValueError("qkv_split_norm_rope: N must be 3 * heads * 128")
    t = v.reshape(M, 3, heads, D)
    q = rope_pairs(rms_norm(t[:, 0], norm_q, eps), cos, sin)
    k = rope_pairs(rms_norm(t[:, 1], norm_k, eps), cos, sin)
    vv = t[:, 2]
    return tuple(np.ascontiguousarray(a.transpose(1, 0, 2)) for a in (q, k, vv))


def linear_qkv_ref(q, sa, qw, sw, bias, heads, norm_q, norm_k, cos, sin, eps=QK_NORM_EPS):
    """The whole fused linear: exact contraction, dequant + bias, then the QKV epilogue.
    Returns float64 (q, k, v) [H, M, D] before the bf16 rounding."""
    v = linear_ref(q, sa, qw, sw, bias, EPI_BIAS)
    return qkv_split_norm_rope(v, heads, norm_q, norm_k, cos, sin, eps)


def linear_qkv_bf16(*args, **kwargs):
    """linear_qkv_ref rounded once to bf16 (returned as float32 values)."""
    return tuple(round_to_bf16(a).astype(np.float32) for a in linear_qkv_ref(*args, **kwargs))
