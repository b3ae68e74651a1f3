"""GPU parity on the full DiT step exactly as the benchmark builds it.

The benchmark draws the 228 weights of a 1024^2 FLUX-dev denoising step on the device (distinct
weights per block) and runs the step as 152 quantize + linear pairs: each double-stream linear is
one segmented call over the joint sequence (512 text rows, then 4096 image rows, with the text and
the image weight), each single-stream linear a plain call over the 4608 rows. Here the first,
middle and last double-stream blocks (all four calls each) and the first, middle and last
single-stream blocks (both calls) are drawn with the same seeds, run through
dq_quantize_weight_fp8 / dq_quantize_fp8 / dq_linear_fp8_segmented or dq_linear_fp8 as in the
step (gated linears in place on their residual stream), copied back, and checked: every code and
scale bit-exact against the oracle, and the outputs of sampled rows of every segment within
|out - ref| <= 4e-3 |ref| + 1e-3 rms(ref).
"""
import numpy as np
import pytest
import torch

import fp8_dynamic_quant_amd as dq
from oracle import linear_ref, quantize_rows
from gpu_util import announce, assert_within_tolerance, dev_to_bf16_bits, require_gpu
from workloads import bf16_bits_to_f32, dit_step_calls, dit_step_device_inputs, workload

pytestmark = pytest.mark.gpu

DOUBLE_BLOCKS = (0, 9, 18)
SINGLE_BLOCKS = (0, 19, 37)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _selected(calls):
    picks = set()
    for i, c in enumerate(calls):
        blocks = DOUBLE_BLOCKS if c["name"].startswith("double") else SINGLE_BLOCKS
        if c["block"] in blocks:
            picks.add(i)
    return picks


def test_dit_step_sampled_blocks():
    w = workload("flux-dit-step-1024")
    only = _selected(dit_step_calls(w))
    assert len(only) == 3 * 4 + 3 * 2
    dev = torch.device("cuda:0")
    announce(f"DiT step: drawing the weights of {len(only)} calls on the device")
    calls, acts, residuals = dit_step_device_inputs(w, dev, dq.dq_quantize_weight_fp8, only=only,
                                                    keep_weights=True)
    rng = np.random.default_rng(1234)
    host_x = {k: dev_to_bf16_bits(v) for k, v in acts.items()}
    for c in calls:
        M, K, N, epi = c["M"], c["K"], c["N"], c["epilogue"]
        segs = c["segments"]
        announce(f"DiT call #{c['call_index']} {c['name']} block {c['block']} {M}x{K}->{N} {epi} "
                 f"segments {[g['rows'] for g in segs]}")
        q, sa = dq.dq_quantize_fp8(acts[c["act"]])
        gated = epi == "gated_residual"
        res_before = None
        if gated:
            r = residuals[c["residual"]]
            res_before = dev_to_bf16_bits(r)
        if len(segs) == 1:
            g0 = segs[0]
            out = dq.dq_linear_fp8(q, sa, g0["qw"], g0["sw"], g0["bias"], epi, g0["gate"],
                                   r if gated else None, out=r if gated else None)
        else:
            out = dq.dq_linear_fp8_segmented(
                q, sa, [g["rows"] for g in segs], [g["qw"] for g in segs],
                [g["sw"] for g in segs], [g["bias"] for g in segs], epi,
                [g["gate"] for g in segs] if gated else None, r if gated else None,
                out=r if gated else None)
        torch.cuda.synchronize()
        # activations: every row of the joint sequence
        xq, xs = quantize_rows(bf16_bits_to_f32(host_x[c["act"]]))
        assert np.array_equal(q.cpu().numpy(), xq), "activation codes differ"
        assert np.array_equal(sa.cpu().numpy().view(np.uint32), xs.view(np.uint32))
        got_all = dev_to_bf16_bits(out)
        r0 = 0
        for g in segs:
            n = g["rows"]
            # weights: codes and scales of every output channel
            wq, ws = quantize_rows(bf16_bits_to_f32(dev_to_bf16_bits(g["w"])))
            assert np.array_equal(g["qw"].cpu().numpy(), wq), f"{g['name']}: weight codes differ"
            assert np.array_equal(g["sw"].cpu().numpy().view(np.uint32), ws.view(np.uint32))
            # outputs: the segment's first and last rows and 30 sampled ones
            rows = r0 + np.unique(np.concatenate([[0, n - 1], rng.choice(n, 30, replace=False)]))
            bias = bf16_bits_to_f32(dev_to_bf16_bits(g["bias"]))
            gate = res = None
            if gated:
                gate = bf16_bits_to_f32(dev_to_bf16_bits(g["gate"]))
                res = bf16_bits_to_f32(res_before[rows])
            ref = linear_ref(xq[rows], xs[rows], wq, ws, bias, epi, gate, res)
            got = bf16_bits_to_f32(got_all[rows]).astype(np.float64)
            assert_within_tolerance(got, ref, what=f"{g['name']} #{g['plan_index']}")
            del g["w"]
            r0 += n
