"""GPU parity on the full DiT step exactly as the benchmark builds it.

The benchmark draws the 228 linears of a 1024^2 FLUX-dev denoising step on the device (distinct
weights per block). Here the first and last double-stream blocks (image and text streams, all
four linears each) and the first and last single-stream blocks (both linears) are drawn with
the same seeds, run through dq_quantize_weight_fp8 / dq_quantize_fp8 / dq_linear_fp8 as in
the step (gated linears in place on their residual stream), copied back, and checked: every
code and scale bit-exact against the oracle, and the outputs of 32 sampled rows within
|out - ref| <= 4e-3 |ref| + 1e-3 rms(ref).
"""
import numpy as np
import pytest
import torch

import fp8_dynamic_quant_amd as dq
from oracle import linear_ref, quantize_rows
from gpu_util import announce, assert_within_tolerance, dev_to_bf16_bits, require_gpu
from workloads import bf16_bits_to_f32, dit_step_device_inputs, dit_step_plan, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _selected(plan_list):
    """Plan indices of double blocks 0 and 18 (8 linears each) and single blocks 0 and 37."""
    picks = set()
    for idx, (shape, sub, stream) in enumerate(plan_list):
        block = sub // 100 - (19 if stream == "single" else 0)
        if stream == "single":
            if block in (0, 37):
                picks.add(idx)
        elif block in (0, 18):
            picks.add(idx)
    return picks


def test_dit_step_sampled_blocks():
    w = workload("flux-dit-step-1024")
    plan_list = dit_step_plan(w)
    only = _selected(plan_list)
    assert len(only) == 2 * 8 + 2 * 2
    dev = torch.device("cuda:0")
    announce(f"DiT step: drawing {len(only)} linears on the device")
    plan, acts, residuals = dit_step_device_inputs(w, dev, dq.dq_quantize_weight_fp8, only=only,
                                                   keep_weights=True)
    rng = np.random.default_rng(1234)
    host_x = {k: dev_to_bf16_bits(v) for k, v in acts.items()}
    for lin in plan:
        M, K, N, epi = lin["M"], lin["K"], lin["N"], lin["epilogue"]
        announce(f"DiT linear #{lin['plan_index']} {lin['name']} {M}x{K}->{N} {epi}")
        x = acts[lin["act"]]
        q, sa = dq.dq_quantize_fp8(x)
        res_before = None
        if epi == "gated_residual":
            r = residuals[lin["residual"]]
            res_before = dev_to_bf16_bits(r)
            out = dq.dq_linear_fp8(q, sa, lin["qw"], lin["sw"], lin["bias"], epi, lin["gate"], r,
                                   out=r)
        else:
            out = dq.dq_linear_fp8(q, sa, lin["qw"], lin["sw"], lin["bias"], epi)
        torch.cuda.synchronize()
        # weights: codes and scales of every output channel
        wq, ws = quantize_rows(bf16_bits_to_f32(dev_to_bf16_bits(lin["w"])))
        assert np.array_equal(lin["qw"].cpu().numpy(), wq), "weight codes differ"
        assert np.array_equal(lin["sw"].cpu().numpy().view(np.uint32), ws.view(np.uint32))
        # activations: every row
        xq, xs = quantize_rows(bf16_bits_to_f32(host_x[lin["act"]]))
        assert np.array_equal(q.cpu().numpy(), xq), "activation codes differ"
        assert np.array_equal(sa.cpu().numpy().view(np.uint32), xs.view(np.uint32))
        # outputs: sampled rows
        rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 30, replace=False)]))
        bias = bf16_bits_to_f32(dev_to_bf16_bits(lin["bias"]))
        gate = res = None
        if epi == "gated_residual":
            gate = bf16_bits_to_f32(dev_to_bf16_bits(lin["gate"]))
            res = bf16_bits_to_f32(res_before[rows])
        ref = linear_ref(xq[rows], xs[rows], wq, ws, bias, epi, gate, res)
        got = bf16_bits_to_f32(dev_to_bf16_bits(out)[rows]).astype(np.float64)
        assert_within_tolerance(got, ref, what=f"{lin['name']} #{lin['plan_index']}")
        del lin["w"]
