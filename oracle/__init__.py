"""CPU oracle for the FP8 dynamic-quant linear layer. TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this package.
The GPU library never calls into it, and it never calls into the GPU library: the two share no
code. The only thing both sides take from a common place is the seeded input generator
(`workloads.py`), which holds none of the method's arithmetic.

What it computes, and where the pages say so:
  * FP8 dynamic quantization of weights and activations, so that 8-bit matrix units do the
    work: page "Solucion de WaveSpeed para Acelerar la Generacion de Imagenes FLUX.1-dev",
    section "Cuantizacion Dinamica FP8".
  * bf16 model tensors with FP8 compute (mixed precision): page "WaveSpeedAI X DataCrunch:
    Inferencia de Imagenes FLUX en Tiempo Real en B200", section "Marco de Inferencia
    Propietario".
  * a GEMM whose epilogue is fused (bias, activation, gated residual): page "Accelerarea
    generarii de imagini cu FLUX 3 Image Klein pe GPU-urile Blackwell NVIDIA", the paragraph
    after "Tabelul 1" on the PrimsTS GEMMs with fused epilogues.
  * the block's LayerNorm and modulation folded into the activation quantizer (kernel fusion):
    page "Solucion de WaveSpeed para Acelerar la Generacion de Imagenes FLUX.1-dev", its lists
    of bottlenecks and of the engine's innovations (see `modulate.py` for the reading taken).
  * the QKV projection with query/key normalization and rotary position embedding fused into
    the GEMM's epilogue: page "Accelerarea generarii de imagini cu FLUX 3 Image Klein pe
    GPU-urile Blackwell NVIDIA", the paragraph on the PrimsTS GEMMs (see `qkv.py`).
  * attention over FP8 queries, keys and values (see `attention.py`) and the block-scaled
    (MX) linear layers with FP8 and FP4 elements, the gfx950 analogue of the pages' NVFP4 (see
    `mx.py` and `mxfp4.py`).

The pages do not fix the granularity, the FP8 flavour, the scale formula or the rounding. The
readings taken are: one scale per token (row of x) and per output channel (row of W); OCP E4M3
with largest finite value 448; scale = amax / 448 and quotient x / scale, each a correctly
rounded fp32 division; round to nearest, ties to the even code, saturating at 448; an all-zero
row gets scale 0 and signed-zero codes.

Precision: the FP8 codes are decided in fp32, the precision the GPU kernel decides them in.
The contraction of decoded values is done in float64, where it is exact (see `linear.py`), and
the epilogue is evaluated in float64.

Parity status: every function here is pinned by tests that do not reuse its arithmetic
(exhaustive brute-force nearest search, exact rational evaluation on tiny shapes, integer
matrix products, closed-form rows, permutation weights, library routines). The pages print no
worked example, so nothing here is pinned to a number printed on the pages.
"""
from .e4m3 import E4M3_MAX, decode_table, encode_e4m3
from .quantize import quantize_rows
from .linear import EPI_BIAS, EPI_GELU_TANH, EPI_GATED_RESIDUAL, gelu_tanh, linear_ref, round_to_bf16
from .modulate import LN_EPS, layernorm_modulate, modulate_rows
from .qkv import (HEAD_DIM, QK_NORM_EPS, linear_qkv_bf16, linear_qkv_ref, qkv_split_norm_rope,
                  rms_norm, rope_pairs)
from .mx import MX_BLOCK, dequantize_mx, linear_mx_ref, quantize_mx, shared_exponent

__all__ = [
    "E4M3_MAX", "decode_table", "encode_e4m3", "quantize_rows",
    "EPI_BIAS", "EPI_GELU_TANH", "EPI_GATED_RESIDUAL", "gelu_tanh", "linear_ref", "round_to_bf16",
    "LN_EPS", "layernorm_modulate", "modulate_rows",
    "HEAD_DIM", "QK_NORM_EPS", "linear_qkv_bf16", "linear_qkv_ref", "qkv_split_norm_rope",
    "rms_norm", "rope_pairs",
    "MX_BLOCK", "dequantize_mx", "linear_mx_ref", "quantize_mx", "shared_exponent",
]
