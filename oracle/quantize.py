"""Per-row dynamic FP8 quantization (one scale per row). TEST INFRASTRUCTURE ONLY.

Dynamic FP8 quantization of weights and activations follows the page "Solucion de WaveSpeed
para Acelerar la Generacion de Imagenes FLUX.1-dev", section "Cuantizacion Dinamica FP8".
The same routine serves activations (a row is a token, scales recomputed on every call) and
weights (a row is an output channel, quantized once when the weight is loaded).
"""
import numpy as np

from .e4m3 import E4M3_MAX, encode_e4m3


def quantize_rows(x):
    """Quantize each row of a float32 [R, K] array holding bf16 values.

    Steps, all in IEEE fp32 (NumPy float32 division is correctly rounded and keeps subnormals):
      1. amax[r] = max_k |x[r, k]|                      (exact)
      2. scale[r] = fl32(amax[r] / 448)
      3. if amax[r] == 0: scale[r] = 0 and every code is the sign bit of x (0x00 or 0x80);
         otherwise q[r, k] = E4M3_RNE_SAT(fl32(x[r, k] / scale[r])).
    Returns (q uint8 [R, K], scale float32 [R]).
    """
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] == 0:
        raise ValueError("quantize_rows: expected a 2-D array with K >= 1")
    if not np.all(np.isfinite(x)):
        raise ValueError("quantize_rows: inputs must be finite")
    amax = np.max(np.abs(x), axis=1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    q = np.empty(x.shape, dtype=np.uint8)
    zero = amax == 0
    if zero.any():
        q[zero] = np.where(np.signbit(x[zero]), 0x80, 0x00).astype(np.uint8)
    live = ~zero
    if live.any():
        quot = (x[live] / scale[live][:, None]).astype(np.float32)
        q[live] = encode_e4m3(quot)
    return q, scale
