"""GPU parity of dq_linear_qkv_fp8_attn: the QKV projection whose outputs leave as the FP8
operands of dq_attention_fp8 (E4M3 codes, one scale per head row; queries and keys
[heads, M, 128], values transposed [heads, 128, M]).

The entry point is defined as the unfused path, exactly: dq_linear_qkv_fp8 (tested against the
float64 oracle in test_gpu_qkv.py) followed by the per-row quantization of its outputs. So, on the
same inputs:
  * the codes and scales equal the oracle's quantization (quantize_rows) of the bf16 queries,
    keys and values that dq_linear_qkv_fp8 gives: the oracle decides every code from the same
    bf16 values;
  * they equal dq_quantize_fp8 of the query and key outputs and dq_quantize_v_fp8 of the value
    output, bit for bit;
  * attention over the fused operands equals attention over the unfused ones.
"""
import numpy as np
import pytest
import torch

import fp8_dynamic_quant_amd as dq
from oracle import quantize_rows
from gpu_util import announce, bf16_to_dev, dev_to_bf16_bits, f32_to_dev, require_gpu
from workloads import LinearShape, bf16_bits_to_f32, make_linear_inputs, make_qk_norm, make_rope

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _inputs(M, K, heads, seed, n_text):
    N = 3 * heads * D
    shape = LinearShape(f"qkv8 {M}x{K}x{heads}h", M, K, N, "bias", max(1, K // 100), 30.0)
    inp = make_linear_inputs(shape, seed)
    cos, sin = make_rope(M, n_text=min(n_text, M))
    q, sa = dq.dq_quantize_fp8(bf16_to_dev(inp.x))
    qw, sw = dq.dq_quantize_weight_fp8(bf16_to_dev(inp.w))
    return (q, sa, qw, sw, heads, bf16_to_dev(inp.bias), bf16_to_dev(make_qk_norm(seed)),
            f32_to_dev(cos), f32_to_dev(sin))


def _check(M, K, heads, seed, ws="auto", n_text=0, oracle_rows=None):
    announce(f"qkv fp8 handoff M={M} K={K} heads={heads} workspace={ws}")
    args = _inputs(M, K, heads, seed, n_text)
    out = dq.dq_linear_qkv_fp8_attn(*args, workspace=ws)
    q8, sq, k8, sk, vt, sv = out
    oq, ok, ov = dq.dq_linear_qkv_fp8(*args, workspace=ws)
    rvt, rsv = dq.dq_quantize_v_fp8(ov)
    torch.cuda.synchronize()
    assert np.array_equal(vt.cpu().numpy(), rvt.cpu().numpy()), "value codes differ"
    assert np.array_equal(sv.cpu().numpy().view(np.uint32), rsv.cpu().numpy().view(np.uint32)), \
        "value scales differ from dq_quantize_v_fp8"
    vt_rows = vt.cpu().numpy().transpose(0, 2, 1).reshape(heads * M, D)   # [head row][channel]
    for what, gc, scales, bf in (("query", q8.cpu().numpy().reshape(heads * M, D), sq, oq),
                                 ("key", k8.cpu().numpy().reshape(heads * M, D), sk, ok),
                                 ("value", vt_rows, sv, ov)):
        rows_bf = dev_to_bf16_bits(bf).reshape(heads * M, D)
        gs = scales.cpu().numpy().reshape(heads * M)
        if what != "value":
            # the library's own quantizer on the bf16 outputs: every row
            rq, rs = dq.dq_quantize_fp8(bf.reshape(heads * M, D))
            torch.cuda.synchronize()
            assert np.array_equal(gc, rq.cpu().numpy()), f"{what} codes differ from dq_quantize_fp8"
            assert np.array_equal(gs.view(np.uint32), rs.cpu().numpy().view(np.uint32)), \
                f"{what} scales differ from dq_quantize_fp8"
        # the oracle's quantization of the same bf16 rows
        rows = np.arange(heads * M) if oracle_rows is None else np.asarray(oracle_rows)
        xq, xs = quantize_rows(bf16_bits_to_f32(rows_bf[rows]))
        assert np.array_equal(gc[rows], xq), f"{what} codes differ from the oracle's"
        assert np.array_equal(gs[rows].view(np.uint32), xs.view(np.uint32)), \
            f"{what} scales differ from the oracle's"
    return out


@pytest.mark.parametrize("ws", ("auto", None))
@pytest.mark.parametrize("M,K,heads", [(64, 256, 1), (304, 384, 2), (272, 128, 3), (16, 128, 1),
                                       (528, 640, 2), (144, 1024, 5)])
def test_tiles_heads_and_ragged_rows(M, K, heads, ws):
    """Whole tiles, the narrow halves of left-over tiles (a head over four waves), tiles cut
    along K, an odd head count, rows past M (M a multiple of 16, as the entry point asks)."""
    _check(M, K, heads, seed=3600 + M + K + heads, ws=ws, n_text=M // 3)


def test_few_tiles_long_k_cut_along_k():
    _check(256, 8192, 1, seed=3700)


def test_all_zero_rows():
    """A zero weight block and a zero bias make every row of the first query head zero (signed
    zeros after the norm and the rotation): those rows take the quantizer's all-zero path."""
    M, K, heads = 128, 256, 2
    args = list(_inputs(M, K, heads, 3750, 0))
    qw = args[2].clone()
    qw[: D] = 0                    # the first query head's rows of W: those outputs are the bias
    args[2] = qw
    zero_bias = torch.zeros_like(args[5])
    args[5] = zero_bias            # and the bias is zero: all-zero query rows (signs only)
    announce("qkv fp8 handoff all-zero rows")
    q8, sq, k8, sk, vt, sv = dq.dq_linear_qkv_fp8_attn(*args)
    oq, ok, ov = dq.dq_linear_qkv_fp8(*args)
    torch.cuda.synchronize()
    assert float(sq[0].abs().max()) == 0.0
    for codes, scales, bf in ((q8, sq, oq), (k8, sk, ok)):
        rq, rs = dq.dq_quantize_fp8(bf.reshape(heads * M, D))
        torch.cuda.synchronize()
        assert torch.equal(codes.reshape(heads * M, D), rq)
        assert torch.equal(scales.reshape(heads * M).view(torch.int32), rs.view(torch.int32))
    rvt, rsv = dq.dq_quantize_v_fp8(ov)
    torch.cuda.synchronize()
    assert torch.equal(vt, rvt) and torch.equal(sv.view(torch.int32), rsv.view(torch.int32))


def test_flux_image_stream_1024px():
    """The image stream's projection at 1024 x 1024: 4096 tokens, 3072 -> 9216 (24 heads); every
    row against dq_quantize_fp8, 96 sampled head rows against the oracle."""
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 4095, 4096, 24 * 4096 - 1],
                                     rng.choice(24 * 4096, 92, replace=False)]))
    _check(4096, 3072, 24, seed=3800, oracle_rows=rows)


def test_flux_text_stream():
    _check(512, 3072, 24, seed=3900, n_text=512)


def test_attention_over_the_handoff():
    """The fused operands drive dq_attention_fp8 to the same output as the unfused ones."""
    M, K, heads = 272, 384, 2
    q8, sq, k8, sk, vt, sv = _check(M, K, heads, seed=3950, n_text=M)
    args = _inputs(M, K, heads, 3950, M)
    oq, ok, ov = dq.dq_linear_qkv_fp8(*args)
    a = dq.quantize_qkv_heads_fp8(oq, ok, ov)
    fused = dq.dq_attention_fp8(q8, sq, k8, sk, vt, sv)
    unfused = dq.dq_attention_fp8(*a)
    torch.cuda.synchronize()
    assert torch.equal(fused.view(torch.int16), unfused.view(torch.int16))


def test_deterministic_and_empty():
    a = _check(304, 384, 2, seed=3990)
    b = _check(304, 384, 2, seed=3990)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    q = torch.empty((0, 256), dtype=torch.uint8, device="cuda:0")
    e = dq.dq_linear_qkv_fp8_attn(q, torch.empty(0, device="cuda:0"),
                                  torch.zeros((384, 256), dtype=torch.uint8, device="cuda:0"),
                                  torch.ones(384, device="cuda:0"), 1, None,
                                  torch.ones((2, 128), dtype=torch.bfloat16, device="cuda:0"),
                                  torch.ones((0, 64), device="cuda:0"),
                                  torch.zeros((0, 64), device="cuda:0"))
    assert e[0].shape == (1, 0, 128) and e[1].shape == (1, 0) and e[4].shape == (1, 128, 0)
    with pytest.raises(dq.DQError):   # M must be a multiple of 16
        dq.dq_linear_qkv_fp8_attn(*_inputs(40, 256, 1, 3991, 0))
