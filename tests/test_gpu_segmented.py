"""GPU parity of dq_linear_fp8_segmented: one launch over row segments with one weight each.

The reference for segment s is the oracle's linear layer on that segment's rows with that
segment's weight (the segmented call is defined as exactly that, row by row). Each case also
checks the call against one dq_linear_fp8 per segment on the same codes: without a workspace both
run whole (or narrow) tiles over the same K steps, so the outputs must be the same bits.
"""
import numpy as np
import pytest
import torch

import fp8_dynamic_quant_amd as dq
from gpu_util import announce, assert_within_tolerance, bf16_to_dev, dev_to_f64, require_gpu
from oracle import linear_ref, quantize_rows
from workloads import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _inputs(seg_rows, K, N, epi, seed):
    """bf16 bit patterns: x [M, K] (N(0,1), a few outlier columns x30), per segment W [N, K]
    (0.02 N(0,1)), bias and gate [N]; residual [M, N]."""
    rng = np.random.default_rng(seed)
    M = sum(seg_rows)
    x = rng.standard_normal((M, K), dtype=np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= np.float32(30.0)
    segs = []
    for _ in seg_rows:
        w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
        b = rng.standard_normal(N, dtype=np.float32) * np.float32(0.01)
        g = np.float32(1.0) + rng.standard_normal(N, dtype=np.float32) * np.float32(0.1)
        segs.append((f32_to_bf16_bits(w), f32_to_bf16_bits(b), f32_to_bf16_bits(g)))
    res = f32_to_bf16_bits(rng.standard_normal((M, N), dtype=np.float32))
    return f32_to_bf16_bits(x), segs, res


def _check(seg_rows, K, N, epi, seed, ws=None, sample=None):
    announce(f"segmented linear rows {seg_rows} K={K} N={N} {epi} workspace={ws}")
    x, segs, res = _inputs(seg_rows, K, N, epi, seed)
    gated = epi == "gated_residual"
    q, sa = dq.dq_quantize_fp8(bf16_to_dev(x))
    qws, sws, bs, gs = [], [], [], []
    for w, b, g in segs:
        qw, sw = dq.dq_quantize_weight_fp8(bf16_to_dev(w))
        qws.append(qw)
        sws.append(sw)
        bs.append(bf16_to_dev(b))
        gs.append(bf16_to_dev(g))
    r = bf16_to_dev(res) if gated else None
    out = dq.dq_linear_fp8_segmented(q, sa, seg_rows, qws, sws, bs, epi,
                                     gs if gated else None, r, out=r, workspace=ws)
    # one dq_linear_fp8 per segment on the same codes
    parts = []
    r0 = 0
    for i, n in enumerate(seg_rows):
        if n == 0:
            continue
        rr = bf16_to_dev(res[r0:r0 + n]) if gated else None
        # own (aligned) copies of the segment's codes and scales
        parts.append((r0, n, dq.dq_linear_fp8(q[r0:r0 + n].clone(), sa[r0:r0 + n].clone(),
                                              qws[i], sws[i], bs[i], epi, gs[i] if gated else None,
                                              rr, out=rr, workspace=ws)))
        r0 += n
    torch.cuda.synchronize()
    if ws is None:
        for r0, n, o in parts:
            assert torch.equal(out[r0:r0 + n], o), f"rows {r0}..{r0 + n}: not the bits of dq_linear_fp8"
    got = dev_to_f64(out)
    oq, osa = quantize_rows(bf16_bits_to_f32(x))
    r0 = 0
    for i, n in enumerate(seg_rows):
        rows = np.arange(r0, r0 + n)
        if sample is not None and n > sample:
            rows = np.unique(np.concatenate([rows[:8], rows[-8:],
                                             np.random.default_rng(i).choice(rows, sample)]))
        r0 += n
        if rows.size == 0:
            continue
        w, b, g = segs[i]
        oqw, osw = quantize_rows(bf16_bits_to_f32(w))
        ref = linear_ref(oq[rows], osa[rows], oqw, osw, bf16_bits_to_f32(b), epi,
                         bf16_bits_to_f32(g) if gated else None,
                         bf16_bits_to_f32(res[rows]) if gated else None)
        assert_within_tolerance(got[rows], ref, what=f"segment {i} rows {rows[0]}..{rows[-1]}")


@pytest.mark.parametrize("epi", ["bias", "gelu_tanh", "gated_residual"])
def test_two_segments(epi):
    _check([300, 77], 384, 320, epi, seed=11)


@pytest.mark.parametrize("ws", [None, "auto"])
def test_ragged_and_empty_segments(ws):
    """Four segments, one of them empty, none a multiple of 256 rows: each has its own tile rows
    (rows of the next segment are never computed with this one's weight)."""
    _check([1, 255, 0, 257], 256, 192, "gated_residual", seed=12, ws=ws)


def test_single_segment_equals_linear():
    _check([513], 640, 576, "gelu_tanh", seed=13)


@pytest.mark.parametrize("K,N,epi", [(3072, 3072, "bias"), (12288, 3072, "gated_residual")])
def test_flux_joint_sequence(K, N, epi):
    """The 1024^2 double-stream shapes: 4096 image and 512 text tokens in one launch (sampled
    rows of the image segment, every text row)."""
    _check([4096, 512], K, N, epi, seed=14, ws="auto", sample=48)
