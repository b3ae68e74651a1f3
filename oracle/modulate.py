"""LayerNorm + modulation + per-row FP8 quantization in one pass. TEST INFRASTRUCTURE ONLY.

The input of a DiT block's QKV, MLP-up and single-stream linears is the block's hidden state
after a normalization and a per-channel modulation. Folding that step into the quantizer is the
kernel fusion the pages count among the fixes for high per-image latency: page "Solucion de
WaveSpeed para Acelerar la Generacion de Imagenes FLUX.1-dev", the list of bottlenecks (no
kernel fusion) and the list of the engine's innovations (custom kernels and kernel fusion); the
model is FLUX-dev's hybrid of multimodal and parallel transformer blocks (same page, the model
description).

The pages do not write the normalization out. The reading taken is the one FLUX-style DiT blocks
use: LayerNorm over the hidden dimension without learned weight or bias, eps = 1e-6, followed by
y = n * (1 + scale) + shift with per-channel bf16 vectors scale and shift (the block's
modulation). The modulated value is a bf16 activation, as the unfused step would hand to the
quantizer, so y is rounded to bf16 (nearest, ties to even) and then quantized per row exactly as
`quantize_rows` does.

Precision: the statistics and y are evaluated in float64 here. A GPU kernel evaluates them in
fp32, so its bf16 y can differ from this one by one bf16 step where y lies next to a rounding
boundary; the codes are a function of the bf16 y, which is why `modulate_rows` returns it.
"""
import numpy as np

from .linear import round_to_bf16
from .quantize import quantize_rows

LN_EPS = 1e-6


def layernorm_modulate(x, scale, shift, eps=LN_EPS):
    """y[r, k] = (x[r, k] - mean_r) / sqrt(var_r + eps) * (1 + scale[k]) + shift[k], float64.

    mean_r = (1/K) sum_k x[r, k];  var_r = (1/K) sum_k (x[r, k] - mean_r)^2  (the biased variance
    LayerNorm uses). x: [R, K]; scale, shift: [K].
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] == 0:
        raise ValueError("layernorm_modulate: expected a 2-D array with K >= 1")
    scale = np.asarray(scale, dtype=np.float64).reshape(-1)
    shift = np.asarray(shift, dtype=np.float64).reshape(-1)
    if scale.shape[0] != x.shape[1] or shift.shape[0] != x.shape[1]:
        raise ValueError("layernorm_modulate: scale and shift need K entries")
    mean = x.mean(axis=1, keepdims=True)
    d = x - mean
    var = (d * d).mean(axis=1, keepdims=True)
    n = d / np.sqrt(var + eps)
    return n * (1.0 + scale[None, :]) + shift[None, :]


def modulate_rows(x, scale, shift, eps=LN_EPS):
    """The fused step: bf16 y (as float32 values) and its per-row FP8 codes and scales.

    Returns (y_bf16 float32 [R, K], q uint8 [R, K], qscale float32 [R]).
    """
    y = round_to_bf16(layernorm_modulate(x, scale, shift, eps)).astype(np.float32)
    if not np.all(np.isfinite(y)):
        raise ValueError("modulate_rows: the modulated values overflow bf16")
    q, s = quantize_rows(y)
    return y, q, s
