"""GPU test of dq_linear_fp8_noalloc, the linear layer on the library's own device scratch.

Three calls in a row, each smaller than the one before, each checked against dq_linear_fp8 with
a workspace of the size its preferred schedule asks for:
  1. 2048 x 16384 -> 2048: 64 tiles of 128 steps; the preferred schedule cuts each into 4 parts
     (256 partial tiles), more than the scratch holds, so the allocation-free call runs another
     schedule: both results within the tolerance of the oracle;
  2. 600 x 5120 -> 448, gated residual in place: 24 parts, in the scratch: the same schedule,
     so the same bits;
  3. 256 x 8192 -> 256: one tile in 4 parts: the same bits, and the scratch's arrival counters
     (left by call 2) serve again.
"""
import numpy as np
import pytest
import torch

import fp8_dynamic_quant_amd as dq
from gpu_util import announce, assert_within_tolerance, bf16_to_dev, dev_to_f64, require_gpu
from oracle import linear_ref, quantize_rows
from workloads import LinearShape, bf16_bits_to_f32, make_linear_inputs

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 4096 + 128 * 256 * 256 * 4

CASES = [
    (LinearShape("noalloc-a", 2048, 16384, 2048, "gelu_tanh", 164, 30.0), 7101),
    (LinearShape("noalloc-b", 600, 5120, 448, "gated_residual", 51, 30.0), 7102),
    (LinearShape("noalloc-c", 256, 8192, 256, "bias", 82, 30.0), 7103),
]


def test_noalloc_matches_linear_on_calls_in_a_row():
    require_gpu()
    for shape, seed in CASES:
        M, K, N = shape.M, shape.K, shape.N
        need = dq.dq_linear_fp8_workspace_size(M, K, N)
        announce(f"noalloc linear {M}x{K}x{N} {shape.epilogue}: preferred workspace {need} bytes")
        inp = make_linear_inputs(shape, seed)
        q, sa = dq.dq_quantize_fp8(bf16_to_dev(inp.x))
        qw, sw = dq.dq_quantize_weight_fp8(bf16_to_dev(inp.w))
        b = bf16_to_dev(inp.bias)
        gated = shape.epilogue == "gated_residual"
        g = bf16_to_dev(inp.gate) if gated else None
        ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
        if gated:   # in place on two copies of the residual stream
            r_ref, r_got = bf16_to_dev(inp.residual), bf16_to_dev(inp.residual)
            ref = dq.dq_linear_fp8(q, sa, qw, sw, b, shape.epilogue, g, r_ref, out=r_ref,
                                   workspace=ws if need else None)
            got = dq.dq_linear_fp8_noalloc(q, sa, qw, sw, b, shape.epilogue, g, r_got, out=r_got)
        else:
            ref = dq.dq_linear_fp8(q, sa, qw, sw, b, shape.epilogue,
                                   workspace=ws if need else None)
            got = dq.dq_linear_fp8_noalloc(q, sa, qw, sw, b, shape.epilogue)
        torch.cuda.synchronize()
        if need <= SCRATCH_BYTES:
            assert torch.equal(got, ref), f"{shape.name}: not the bits of dq_linear_fp8"
        oq, osa = quantize_rows(bf16_bits_to_f32(inp.x))
        oqw, osw = quantize_rows(bf16_bits_to_f32(inp.w))
        want = linear_ref(oq, osa, oqw, osw, bf16_bits_to_f32(inp.bias), shape.epilogue,
                          None if not gated else bf16_bits_to_f32(inp.gate),
                          None if not gated else bf16_bits_to_f32(inp.residual))
        rms = float(np.sqrt(np.mean(want * want)))
        assert_within_tolerance(dev_to_f64(got), want, rms, what=f"{shape.name} noalloc")
        assert_within_tolerance(dev_to_f64(ref), want, rms, what=f"{shape.name} workspace")
        assert int(ws[:4096].view(torch.int32).abs().sum().item()) == 0
        del q, qw, ws, ref, got
        torch.cuda.empty_cache()
