"""GPU parity of dq_linear_qkv_fp8 (FP8 GEMM with the QKV / query-key RMS norm / rotary
epilogue) against the oracle.

x and W are quantized on the GPU and their codes and scales checked bit for bit against the
oracle's own quantization; the oracle then evaluates the whole projection from its codes in
float64 and every output must satisfy |out - ref| <= 4e-3 |ref| + 1e-3 rms(ref) per output
tensor, ref being the oracle's value before bf16 rounding. The value third does the same
arithmetic as the plain bias epilogue, so it must equal dq_linear_fp8's bias output bit for bit.
"""
import numpy as np
import pytest
import torch

import fp8_dynamic_quant_amd as dq
from oracle import linear_ref, linear_qkv_ref, quantize_rows
from gpu_util import (announce, assert_within_tolerance, bf16_to_dev, dev_to_bf16_bits,
                      dev_to_f64, f32_to_dev, require_gpu)
from workloads import (LinearShape, bf16_bits_to_f32, make_linear_inputs, make_qk_norm,
                       make_rope)

pytestmark = pytest.mark.gpu

D = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _run(M, K, heads, seed, ws="auto", rows=None, check_v_against_bias=True, n_text=512):
    N = 3 * heads * D
    shape = LinearShape(f"qkv{M}x{K}x{heads}h", M, K, N, "bias", max(1, K // 100), 30.0)
    inp = make_linear_inputs(shape, seed)
    nqk = make_qk_norm(seed)
    cos, sin = make_rope(M, n_text=min(n_text, M))
    announce(f"qkv M={M} K={K} heads={heads} workspace={ws}")
    q, sa = dq.dq_quantize_fp8(bf16_to_dev(inp.x))
    qw, sw = dq.dq_quantize_weight_fp8(bf16_to_dev(inp.w))
    tb = bf16_to_dev(inp.bias)
    oq, ok, ov = dq.dq_linear_qkv_fp8(q, sa, qw, sw, heads, tb, bf16_to_dev(nqk), f32_to_dev(cos),
                                      f32_to_dev(sin), workspace=ws)
    torch.cuda.synchronize()
    rows = np.arange(M) if rows is None else np.asarray(rows)
    # codes and scales against the oracle's own quantization
    xq, xs = quantize_rows(bf16_bits_to_f32(inp.x[rows]))
    wq, ws_ = quantize_rows(bf16_bits_to_f32(inp.w))
    assert np.array_equal(q.cpu().numpy()[rows], xq), "activation codes differ"
    assert np.array_equal(sa.cpu().numpy()[rows].view(np.uint32), xs.view(np.uint32))
    assert np.array_equal(qw.cpu().numpy(), wq), "weight codes differ"
    assert np.array_equal(sw.cpu().numpy().view(np.uint32), ws_.view(np.uint32))
    ref = linear_qkv_ref(xq, xs, wq, ws_, bf16_bits_to_f32(inp.bias), heads,
                         bf16_bits_to_f32(nqk[0]), bf16_bits_to_f32(nqk[1]), cos[rows], sin[rows])
    worst = []
    for name, got, r in zip("qkv", (oq, ok, ov), ref):
        g = dev_to_f64(got)[:, rows, :]
        worst.append(assert_within_tolerance(g, r, what=f"{shape.name} {name}"))
    if check_v_against_bias:
        # the value third through the plain bias epilogue: the same arithmetic, the same bits
        plain = dq.dq_linear_fp8(q, sa, qw[2 * heads * D:], sw[2 * heads * D:], tb[2 * heads * D:],
                                 "bias", workspace=ws)
        torch.cuda.synchronize()
        pv = dev_to_bf16_bits(plain).reshape(M, heads, D).transpose(1, 0, 2)
        assert np.array_equal(dev_to_bf16_bits(ov), pv), "value third differs from the bias epilogue"
    print(f"[{shape.name} ws={ws}] worst err/bound q {worst[0]:.3f} k {worst[1]:.3f} "
          f"v {worst[2]:.3f}")
    return oq, ok, ov


WS = ("auto", None)


@pytest.mark.parametrize("ws", WS)
@pytest.mark.parametrize("M,K,heads", [(64, 256, 1), (300, 384, 2), (257, 128, 3), (1, 128, 1),
                                       (513, 640, 2), (130, 1024, 5)])
def test_tiles_heads_and_ragged_rows(M, K, heads, ws):
    """An odd head count leaves the last 256-column tile half past N; rows past M, a single
    row, and tiles whose work is cut along K (with a workspace)."""
    _run(M, K, heads, seed=3000 + M + K + heads, ws=ws, n_text=M // 3)


def test_few_tiles_long_k_cut_along_k():
    """2 tiles of 64 steps: with a workspace each is cut into parts summed before the epilogue."""
    _run(256, 8192, 1, seed=3100, ws="auto")


@pytest.mark.parametrize("ws", WS)
def test_flux_image_stream_qkv_1024px(ws):
    """The image stream's QKV projection at 1024 x 1024: 4096 tokens, 3072 -> 9216 (24 heads).
    576 tiles: two full rounds, then 64 left-over tiles run as narrow halves (no workspace) or
    cut along K. 64 sampled rows are compared element by element."""
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 4095],
                                     np.random.default_rng(5).choice(4096, 59, replace=False)]))
    _run(4096, 3072, 24, seed=3200, ws=ws, rows=rows, n_text=0)


def test_flux_text_stream_qkv():
    """The text stream's QKV projection: 512 tokens at position 0 (no rotation)."""
    _run(512, 3072, 24, seed=3300, ws="auto", n_text=512)


def test_rotation_by_a_quarter_turn_swaps_pairs():
    """cos = 0, sin = 1 turns (a, b) into (-b, a): the outputs are exact bf16 negations and
    swaps of the unrotated ones."""
    M, K, heads = 96, 256, 2
    shape = LinearShape("quarter", M, K, 3 * heads * D, "bias", 3, 30.0)
    inp = make_linear_inputs(shape, 3400)
    q, sa = dq.dq_quantize_fp8(bf16_to_dev(inp.x))
    qw, sw = dq.dq_quantize_weight_fp8(bf16_to_dev(inp.w))
    tb, tn = bf16_to_dev(inp.bias), bf16_to_dev(make_qk_norm(3400))
    one = torch.ones((M, 64), dtype=torch.float32, device="cuda:0")
    zero = torch.zeros((M, 64), dtype=torch.float32, device="cuda:0")
    announce("qkv quarter turn")
    a = dq.dq_linear_qkv_fp8(q, sa, qw, sw, heads, tb, tn, one, zero)
    b = dq.dq_linear_qkv_fp8(q, sa, qw, sw, heads, tb, tn, zero, one)
    torch.cuda.synchronize()
    for x, y in zip(a[:2], b[:2]):
        xb, yb = dev_to_bf16_bits(x), dev_to_bf16_bits(y)
        assert np.array_equal(yb[..., 0::2], xb[..., 1::2] ^ np.uint16(0x8000))
        assert np.array_equal(yb[..., 1::2], xb[..., 0::2])
    assert np.array_equal(dev_to_bf16_bits(a[2]), dev_to_bf16_bits(b[2]))


def test_deterministic_and_empty():
    outs = [_run(300, 384, 2, seed=3500, check_v_against_bias=False) for _ in range(2)]
    for a, b in zip(*outs):
        assert torch.equal(a, b)
    q = torch.empty((0, 256), dtype=torch.uint8, device="cuda:0")
    e = dq.dq_linear_qkv_fp8(q, torch.empty(0, device="cuda:0"),
                             torch.zeros((384, 256), dtype=torch.uint8, device="cuda:0"),
                             torch.ones(384, device="cuda:0"), 1, None,
                             torch.ones((2, 128), dtype=torch.bfloat16, device="cuda:0"),
                             torch.ones((0, 64), device="cuda:0"),
                             torch.zeros((0, 64), device="cuda:0"))
    assert all(t.shape == (1, 0, 128) for t in e)
