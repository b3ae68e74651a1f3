"""GPU parity of the DiT step's MXFP4 variant exactly as the benchmark builds it.

The benchmark's MXFP4 step draws the same 228 weights as the FP8 step (distinct per block) and
quantizes them with dq_quantize_mxfp4; each call quantizes its bf16 activation with
dq_quantize_mxfp4 and runs dq_linear_mxfp4_segmented (double-stream blocks: 512 text rows, then
4096 image rows, two weights) or dq_linear_mxfp4 (single-stream blocks), gated linears in place on
their residual stream. Here the middle double-stream block (all four calls) and the last
single-stream block (both calls) are drawn with the same seeds and run that way. Per segment, 32
rows (first, last, random) and 64 output channels (first, last, random) are sampled: the codes
and scale bytes of those activation rows and weight rows must equal the oracle's, and the outputs
at the sampled rows and channels must satisfy |out - ref| <= 4e-3 |ref| + 1e-3 rms(ref), ref
being the oracle's MXFP4 layer on the oracle's codes. (The oracle's E2M1 encoder holds a float64
distance to every magnitude per value: quantizing whole weights of up to 66 M values would take
minutes; the full-size codes are checked in the MXFP4 tests.)
"""
import numpy as np
import pytest
import torch

import fp8_dynamic_quant_amd as dq
from oracle.mxfp4 import linear_mxfp4_ref, quantize_mxfp4
from gpu_util import announce, assert_within_tolerance, dev_to_bf16_bits, require_gpu
from workloads import bf16_bits_to_f32, dit_step_calls, dit_step_device_inputs, workload

pytestmark = pytest.mark.gpu

DOUBLE_BLOCKS = (9,)
SINGLE_BLOCKS = (37,)


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


def test_dit_step_mxfp4_sampled_blocks():
    w = workload("flux-dit-step-1024")
    only = _selected(dit_step_calls(w))
    assert len(only) == 4 + 2
    dev = torch.device("cuda:0")
    announce(f"DiT step, MXFP4: drawing the weights of {len(only)} calls on the device")
    calls, acts, residuals = dit_step_device_inputs(w, dev, dq.dq_quantize_mxfp4, only=only,
                                                    keep_weights=True)
    rng = np.random.default_rng(4321)
    host_x = {k: dev_to_bf16_bits(v) for k, v in acts.items()}
    for c in calls:
        M, K, N, epi = c["M"], c["K"], c["N"], c["epilogue"]
        segs = c["segments"]
        announce(f"DiT MXFP4 call #{c['call_index']} {c['name']} block {c['block']} "
                 f"{M}x{K}->{N} {epi} segments {[g['rows'] for g in segs]}")
        q, sa = dq.dq_quantize_mxfp4(acts[c["act"]])
        gated = epi == "gated_residual"
        res_before = None
        r = None
        if gated:
            r = residuals[c["residual"]]
            res_before = dev_to_bf16_bits(r)
        if len(segs) == 1:
            g0 = segs[0]
            out = dq.dq_linear_mxfp4(q, sa, g0["qw"], g0["sw"], g0["bias"], epi, g0["gate"], r,
                                     out=r)
        else:
            out = dq.dq_linear_mxfp4_segmented(
                q, sa, [g["rows"] for g in segs], [g["qw"] for g in segs],
                [g["sw"] for g in segs], [g["bias"] for g in segs], epi,
                [g["gate"] for g in segs] if gated else None, r, out=r)
        torch.cuda.synchronize()
        gq, gs = q.cpu().numpy(), sa.cpu().numpy()
        got_all = dev_to_bf16_bits(out)
        r0 = 0
        for g in segs:
            n = g["rows"]
            rows = r0 + np.unique(np.concatenate([[0, n - 1], rng.choice(n, 30, replace=False)]))
            cols = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 62, replace=False)]))
            wq, ws = quantize_mxfp4(bf16_bits_to_f32(dev_to_bf16_bits(g["w"])[cols]))
            assert np.array_equal(g["qw"].cpu().numpy()[cols], wq), f"{g['name']}: weight codes differ"
            assert np.array_equal(g["sw"].cpu().numpy()[cols], ws), f"{g['name']}: weight scales differ"
            xq, xs = quantize_mxfp4(bf16_bits_to_f32(host_x[c["act"]][rows]))
            assert np.array_equal(gq[rows], xq), f"{g['name']}: activation codes differ"
            assert np.array_equal(gs[rows], xs), f"{g['name']}: activation scales differ"
            bias = bf16_bits_to_f32(dev_to_bf16_bits(g["bias"]))[cols]
            gate = res = None
            if gated:
                gate = bf16_bits_to_f32(dev_to_bf16_bits(g["gate"]))[cols]
                res = bf16_bits_to_f32(res_before[rows][:, cols])
            ref = linear_mxfp4_ref(xq, xs, wq, ws, bias, epi, gate, res)
            got = bf16_bits_to_f32(got_all[rows][:, cols]).astype(np.float64)
            assert_within_tolerance(got, ref, what=f"MXFP4 {g['name']} #{g['plan_index']}")
            del g["w"]
            r0 += n
