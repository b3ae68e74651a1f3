"""W8A8 linear with the dequant / bias / activation epilogue. TEST INFRASTRUCTURE ONLY.

The FP8 GEMM with a fused epilogue follows the page "Accelerarea generarii de imagini cu FLUX 3
Image Klein pe GPU-urile Blackwell NVIDIA" (the paragraph after "Tabelul 1": optimized GEMMs
with fused epilogues) and the page "Solucion de WaveSpeed para Acelerar la Generacion de
Imagenes FLUX.1-dev", section "Cuantizacion Dinamica FP8" (8-bit matrix units fed with
dynamically quantized weights and activations).

Readings taken where the pages are silent:
  * acc[m, n] = sum_k dec(q[m, k]) * dec(qw[n, k])
  * v = acc * sa[m] * sw[n] + bias[n]           (bias absent = 0)
  * bias:           y = v
  * gelu_tanh:      y = 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3)))
  * gated_residual: y = residual[m, n] + gate[n] * v
The output is y; the GPU stores bf16(y), rounded once to nearest even.

Exactness of the contraction in float64: every decoded value is a multiple of 2^-9 with
magnitude <= 448, so every product is a multiple of 2^-18 with magnitude < 2^17.7, and any
partial sum over K <= 131072 terms is a multiple of 2^-18 below 2^34.7. Such numbers need at
most 53 significant bits, so float64 holds every partial sum exactly, in any summation order:
`acc` is the exact mathematical value whatever blocking the BLAS library uses.
"""
import numpy as np

from .e4m3 import decode_table

EPI_BIAS = "bias"
EPI_GELU_TANH = "gelu_tanh"
EPI_GATED_RESIDUAL = "gated_residual"

_SQRT_2_OVER_PI = 0.7978845608028654
_GELU_CUBIC = 0.044715
_K_EXACT = 131072


def gelu_tanh(v):
    """0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))), in float64."""
    v = np.asarray(v, dtype=np.float64)
    return 0.5 * v * (1.0 + np.tanh(_SQRT_2_OVER_PI * (v + _GELU_CUBIC * v * v * v)))


def contract(q, qw):
    """Exact acc = dec(q) @ dec(qw)^T in float64 (q: uint8 [M,K], qw: uint8 [N,K])."""
    q = np.asarray(q, dtype=np.uint8)
    qw = np.asarray(qw, dtype=np.uint8)
    if q.ndim != 2 or qw.ndim != 2 or q.shape[1] != qw.shape[1]:
        raise ValueError("contract: shapes must be [M,K] and [N,K]")
    if q.shape[1] > _K_EXACT:
        raise ValueError("contract: K too large for an exact float64 contraction")
    table = decode_table()
    a = table[q]
    b = table[qw]
    if np.isnan(a).any() or np.isnan(b).any():
        raise ValueError("contract: NaN codes in the operands")
    return a @ b.T


def linear_ref(q, sa, qw, sw, bias=None, epilogue=EPI_BIAS, gate=None, residual=None):
    """float64 [M,N] value y of the epilogue applied to the exact contraction (before bf16).

    q uint8 [M,K], sa float32 [M], qw uint8 [N,K], sw float32 [N]; bias, gate float [N];
    residual float [M,N]. Floats may be float32 arrays holding bf16 values.
    """
    acc = contract(q, qw)
    M, N = acc.shape
    sa = np.asarray(sa, dtype=np.float64).reshape(M)
    sw = np.asarray(sw, dtype=np.float64).reshape(N)
    v = (acc * sa[:, None]) * sw[None, :]
    if bias is not None:
        v = v + np.asarray(bias, dtype=np.float64).reshape(N)[None, :]
    if epilogue == EPI_BIAS:
        return v
    if epilogue == EPI_GELU_TANH:
        return gelu_tanh(v)
    if epilogue == EPI_GATED_RESIDUAL:
        if gate is None or residual is None:
            raise ValueError("gated_residual needs gate and residual")
        g = np.asarray(gate, dtype=np.float64).reshape(N)
        r = np.asarray(residual, dtype=np.float64).reshape(M, N)
        return r + g[None, :] * v
    raise ValueError(f"unknown epilogue {epilogue!r}")


def round_to_bf16(y):
    """Nearest bf16 value (ties to even) of finite float64 values, returned as float64.

    bf16 keeps 8 significant bits and fp32's exponent range: below 2^-126 the grid is the
    subnormal one with spacing 2^-133. Values that round past the largest finite bf16 become
    infinities.
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    _, ex = np.frexp(a)
    e = np.where(a > 0, ex.astype(np.int64) - 1, -126)
    e = np.maximum(e, -126)
    r = np.ldexp(np.rint(np.ldexp(a, 7 - e)), e - 7)
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    return np.copysign(r, y)
