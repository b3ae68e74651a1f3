"""Block-scaled (MX) FP8 quantization and the block-scaled linear layer. TEST INFRASTRUCTURE ONLY.

The pages run FLUX 3 Image Klein's linears in NVFP4 on Blackwell: weights and activations in 4
bits with a shared scale per small block of values, up to 1.62x faster text-to-image than BF16
(page "Accelerarea generarii de imagini cu FLUX 3 Image Klein pe GPU-urile Blackwell NVIDIA", its
paragraph on NVFP4 against BF16; page "Optimizacion de la inferencia de FLUX 3 Image Klein en GPUs
NVIDIA Blackwell", section "Como funciona"). Neither page defines the block format, and NVFP4 is
NVIDIA's own. The block-scaled format that gfx950's matrix units execute is the OCP Microscaling
(MX) one; the reading taken is its definition, with E4M3 elements (MXFP8):

  * a block is 32 consecutive values of a row along K (K a multiple of 32);
  * the block's shared exponent is floor(log2(amax)) - 8, where 8 is the exponent of E4M3's
    largest binade, clamped to the E8M0 range [-127, 127]; an all-zero block takes -127;
  * each element is the E4M3 value nearest to x / 2^shared (ties to even; magnitudes past 448,
    which the top binade reaches since x / 2^shared < 512, saturate to 448);
  * the scale is kept as its E8M0 byte, shared + 127.

The block-scaled linear layer: y[m, n] = epilogue(sum_b 2^(ea[m, b] + ew[n, b])
sum_{k in b} dec(a[m, k]) dec(w[n, k]) + bias[n]), evaluated here as the product of the
dequantized matrices in float64.
"""
import numpy as np

from .e4m3 import decode_table, encode_e4m3
from .linear import EPI_BIAS, EPI_GELU_TANH, gelu_tanh

MX_BLOCK = 32
E4M3_EMAX = 8          # 448 = 1.75 * 2^8
E8M0_BIAS = 127


def shared_exponent(amax):
    """floor(log2(amax)) - 8 clamped to [-127, 127]; -127 for amax == 0 (int64 array)."""
    a = np.asarray(amax, dtype=np.float64)
    e = np.full(a.shape, -E8M0_BIAS, dtype=np.int64)
    nz = a > 0
    _, ex = np.frexp(a[nz])                    # a = f * 2^ex, f in [0.5, 1)
    e[nz] = np.clip(ex.astype(np.int64) - 1 - E4M3_EMAX, -E8M0_BIAS, E8M0_BIAS)
    return e


def quantize_mx(x):
    """MX quantization of each row of a float32 [R, K] array holding bf16 values.

    Returns (codes uint8 [R, K], scales uint8 [R, K / 32], the E8M0 bytes)."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % MX_BLOCK != 0:
        raise ValueError("quantize_mx: expected [R, K] with K a multiple of 32")
    if not np.all(np.isfinite(x)):
        raise ValueError("quantize_mx: inputs must be finite")
    R, K = x.shape
    xb = x.reshape(R, K // MX_BLOCK, MX_BLOCK).astype(np.float64)
    e = shared_exponent(np.max(np.abs(xb), axis=2))
    # x / 2^e is exact in float64; it is a float32 value unless it falls below 2^-126, where
    # the float32 rounding cannot move it past half of E4M3's smallest step (2^-10)
    quot = (xb * np.ldexp(1.0, -e)[..., None]).astype(np.float32)
    codes = encode_e4m3(quot).reshape(R, K)
    return codes, (e + E8M0_BIAS).astype(np.uint8)


def dequantize_mx(codes, scales):
    """float64 [R, K]: dec(code) * 2^(scale - 127) per block of 32 along K."""
    codes = np.asarray(codes, dtype=np.uint8)
    R, K = codes.shape
    s = np.asarray(scales, dtype=np.int64).reshape(R, K // MX_BLOCK) - E8M0_BIAS
    vals = decode_table()[codes].reshape(R, K // MX_BLOCK, MX_BLOCK)
    return (vals * np.ldexp(1.0, s)[..., None]).reshape(R, K)


def linear_mx_ref(qa, sa, qw, sw, bias=None, epilogue=EPI_BIAS):
    """float64 [M, N] value of the block-scaled linear layer before the bf16 rounding.

    qa uint8 [M, K] and sa uint8 [M, K / 32]; qw uint8 [N, K] and sw uint8 [N, K / 32];
    bias float [N] (bf16 values) or None."""
    a = dequantize_mx(qa, sa)
    w = dequantize_mx(qw, sw)
    v = a @ w.T
    if bias is not None:
        v = v + np.asarray(bias, dtype=np.float64).reshape(1, -1)
    if epilogue == EPI_BIAS:
        return v
    if epilogue == EPI_GELU_TANH:
        return gelu_tanh(v)
    raise ValueError(f"linear_mx_ref: unsupported epilogue {epilogue!r}")
