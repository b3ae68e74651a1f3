"""Attention over FP8-quantized queries, keys and values. TEST INFRASTRUCTURE ONLY.

The pages name FP8 attention as the second lever after the quantized GEMMs: page "Accelerarea
generarii de imagini cu FLUX 3 Image Klein pe GPU-urile Blackwell NVIDIA" (attention as the
main cost at high resolution, about 60 % of the DiT's GPU time at 2048 x 2048, and the quantized
cuDNN FP8 / VC-Attention FP8 options), and page "Optimizacion de la inferencia de FLUX 3 Image
Klein en GPUs NVIDIA Blackwell", section "Como funciona" (quantized attention keeps query, key
and value in FP8). Neither page writes the arithmetic out. The reading taken:

  * per head h, the query, key and value rows (one per token, 128 channels) are quantized per
    row exactly as the linear layer's activations (`quantize_rows`: scale = amax / 448, OCP
    E4M3, nearest even, saturating);
  * logits s[i, j] = (dec(q_i) sq_i) . (dec(k_j) sk_j) / sqrt(128), from the decoded values;
  * p = softmax over the keys j (all tokens attend to all tokens: the joint text + image
    attention of a FLUX block has no mask);
  * o_i = sum_j p[i, j] sv_j dec(v_j): the weights multiply the dequantized values.

Everything after the codes is evaluated in float64 here.
"""
import numpy as np

from .e4m3 import decode_table
from .quantize import quantize_rows

HEAD_DIM = 128


def quantize_heads(x):
    """Per (head, token) row quantization of x [H, S, D] (float32 holding bf16 values).
    Returns (codes uint8 [H, S, D], scales float32 [H, S])."""
    x = np.asarray(x, dtype=np.float32)
    H, S, D = x.shape
    q, s = quantize_rows(x.reshape(H * S, D))
    return q.reshape(H, S, D), s.reshape(H, S)


def attention_ref(q8, sq, k8, sk, v8, sv):
    """float64 attention output [H, S, D] from codes [H, S, D] and row scales [H, S]."""
    table = decode_table()
    q = table[np.asarray(q8, np.uint8)] * np.asarray(sq, np.float64)[..., None]
    k = table[np.asarray(k8, np.uint8)] * np.asarray(sk, np.float64)[..., None]
    v = table[np.asarray(v8, np.uint8)] * np.asarray(sv, np.float64)[..., None]
    D = q.shape[-1]
    logits = np.einsum("hid,hjd->hij", q, k) / np.sqrt(D)
    logits -= logits.max(axis=-1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=-1, keepdims=True)
    return np.einsum("hij,hjd->hid", p, v)


def attention_fp8_ref(q, k, v):
    """The whole step from bf16-valued float32 inputs [H, S, D]: quantize, then attention.
    Returns (o float64 [H, S, D], (q8, sq), (k8, sk), (v8, sv))."""
    qq, kk, vv = quantize_heads(q), quantize_heads(k), quantize_heads(v)
    return attention_ref(qq[0], qq[1], kk[0], kk[1], vv[0], vv[1]), qq, kk, vv
