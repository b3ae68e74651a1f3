"""Block-scaled FP4 (MXFP4) quantization and the MXFP4 linear layer. TEST INFRASTRUCTURE ONLY.

The pages run FLUX 3 Image Klein's linears with 4-bit weights and activations and a shared scale
per small block of values (NVFP4), up to 1.62x faster text-to-image than BF16 (page "Accelerarea
generarii de imagini cu FLUX 3 Image Klein pe GPU-urile Blackwell NVIDIA", its paragraph on NVFP4
against BF16; page "Optimizacion de la inferencia de FLUX 3 Image Klein en GPUs NVIDIA
Blackwell", section "Como funciona"). The pages define no 4-bit format, and NVFP4 is NVIDIA's.
The 4-bit block format gfx950's matrix units execute is the OCP Microscaling one with E2M1
elements (MXFP4); the reading taken is its definition:

  * E2M1 element: sign, two exponent bits (bias 1), one mantissa bit; the magnitudes are
    0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7, the sign is bit 3 (so -0 is code 8);
  * a block is 32 consecutive values of a row along K (K a multiple of 32);
  * the block's shared exponent is floor(log2(amax)) - 2, where 2 is the exponent of E2M1's
    largest binade (6 = 1.5 * 2^2), clamped to the E8M0 range [-127, 127]; an all-zero block
    takes -127;
  * each element is the E2M1 value nearest to x / 2^shared, ties to the even code (mantissa bit
    0); magnitudes past 6, which x / 2^shared < 8 can reach, saturate to 6; the sign of x is kept
    (also for values that round to zero);
  * the scale is kept as its E8M0 byte, shared + 127;
  * two elements per byte: element 2j of a row in the low nibble of byte j, element 2j + 1 in
    the high nibble.

The MXFP4 linear layer: y[m, n] = epilogue(sum_b 2^(ea[m, b] + ew[n, b])
sum_{k in b} dec(a[m, k]) dec(w[n, k]) + bias[n]), evaluated here as the product of the
dequantized matrices in float64.
"""
import numpy as np

from .linear import EPI_BIAS, EPI_GATED_RESIDUAL, EPI_GELU_TANH, gelu_tanh

MX_BLOCK = 32
FP4_EMAX = 2           # 6 = 1.5 * 2^2
E8M0_BIAS = 127
FP4_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def decode_fp4_table():
    """float64 [16]: the value of every E2M1 code (bit 3 the sign)."""
    return np.concatenate([FP4_MAGNITUDES, -FP4_MAGNITUDES])


def encode_fp4(v):
    """E2M1 codes (uint8, 0..15) of float values: the nearest magnitude, ties to the even code,
    saturating at 6; the sign bit of v is kept."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    d = np.abs(a[..., None] - FP4_MAGNITUDES)           # distance to each magnitude
    best = np.min(d, axis=-1, keepdims=True)
    ties = d == best
    # among the nearest magnitudes (one, or two at a midpoint) take the even code
    even = ties & (np.arange(8) % 2 == 0)
    code = np.where(np.any(even, axis=-1), np.argmax(even, axis=-1), np.argmax(ties, axis=-1))
    code = np.where(a > 6.0, 7, code)
    return (code + 8 * np.signbit(v)).astype(np.uint8)


def shared_exponent4(amax):
    """floor(log2(amax)) - 2 clamped to [-127, 127]; -127 for amax == 0 (int64 array)."""
    a = np.asarray(amax, dtype=np.float64)
    e = np.full(a.shape, -E8M0_BIAS, dtype=np.int64)
    nz = a > 0
    _, ex = np.frexp(a[nz])                    # a = f * 2^ex, f in [0.5, 1)
    e[nz] = np.clip(ex.astype(np.int64) - 1 - FP4_EMAX, -E8M0_BIAS, E8M0_BIAS)
    return e


def pack_fp4(codes):
    """uint8 [R, K] codes (0..15) -> uint8 [R, K / 2]: element 2j low nibble, 2j + 1 high."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_fp4(packed):
    """uint8 [R, K / 2] -> uint8 [R, K] codes."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], 2 * p.shape[1]), dtype=np.uint8)
    out[:, 0::2] = p & 0x0F
    out[:, 1::2] = p >> 4
    return out


def quantize_mxfp4(x):
    """MXFP4 quantization of each row of a float32 [R, K] array holding bf16 values.

    Returns (packed codes uint8 [R, K / 2], scales uint8 [R, K / 32], the E8M0 bytes)."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2 or x.shape[1] % MX_BLOCK != 0:
        raise ValueError("quantize_mxfp4: expected [R, K] with K a multiple of 32")
    if not np.all(np.isfinite(x)):
        raise ValueError("quantize_mxfp4: inputs must be finite")
    R, K = x.shape
    xb = x.reshape(R, K // MX_BLOCK, MX_BLOCK).astype(np.float64)
    e = shared_exponent4(np.max(np.abs(xb), axis=2))
    quot = xb * np.ldexp(1.0, -e)[..., None]          # exact in float64
    codes = encode_fp4(quot).reshape(R, K)
    return pack_fp4(codes), (e + E8M0_BIAS).astype(np.uint8)


def dequantize_mxfp4(packed, scales):
    """float64 [R, K]: dec(code) * 2^(scale - 127) per block of 32 along K."""
    codes = unpack_fp4(packed)
    R, K = codes.shape
    s = np.asarray(scales, dtype=np.int64).reshape(R, K // MX_BLOCK) - E8M0_BIAS
    vals = decode_fp4_table()[codes].reshape(R, K // MX_BLOCK, MX_BLOCK)
    return (vals * np.ldexp(1.0, s)[..., None]).reshape(R, K)


def linear_mxfp4_ref(qa, sa, qw, sw, bias=None, epilogue=EPI_BIAS, gate=None, residual=None):
    """float64 [M, N] value of the MXFP4 linear layer before the bf16 rounding.

    qa uint8 [M, K / 2] and sa uint8 [M, K / 32]; qw uint8 [N, K / 2] and sw uint8 [N, K / 32];
    bias float [N] (bf16 values) or None. The epilogues are the per-row layer's: v itself,
    gelu_tanh(v), or residual + gate v (gate [N], residual [M, N], bf16 values)."""
    a = dequantize_mxfp4(qa, sa)
    w = dequantize_mxfp4(qw, sw)
    v = a @ w.T
    if bias is not None:
        v = v + np.asarray(bias, dtype=np.float64).reshape(1, -1)
    if epilogue == EPI_BIAS:
        return v
    if epilogue == EPI_GELU_TANH:
        return gelu_tanh(v)
    if epilogue == EPI_GATED_RESIDUAL:
        if gate is None or residual is None:
            raise ValueError("linear_mxfp4_ref: the gated epilogue needs gate and residual")
        return (np.asarray(residual, dtype=np.float64)
                + np.asarray(gate, dtype=np.float64).reshape(1, -1) * v)
    raise ValueError(f"linear_mxfp4_ref: unsupported epilogue {epilogue!r}")
