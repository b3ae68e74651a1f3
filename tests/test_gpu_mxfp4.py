"""GPU parity of the MXFP4 path (dq_quantize_mxfp4, dq_linear_mxfp4, its segmented form) against
the oracle.

Packed codes and scale bytes must equal the oracle's bit for bit. The linear layer's output is
compared with the oracle's float64 value of the layer on the same codes and scales within the
output tolerance of the FP8 linear layer, |out - ref| <= 4e-3 |ref| + 1e-3 rms(ref): every
product of two E2M1 values is exact, the accumulation is fp32 and the output is one bf16
rounding. On inputs whose sums are exact in fp32 the output must equal the bf16 rounding of the
exact value.
"""
import numpy as np
import pytest
import torch

import fp8_dynamic_quant_amd as dq
from oracle import EPI_BIAS, EPI_GATED_RESIDUAL, EPI_GELU_TANH, round_to_bf16
from oracle.mxfp4 import (decode_fp4_table, dequantize_mxfp4, linear_mxfp4_ref, pack_fp4,
                          quantize_mxfp4)
from gpu_util import (announce, assert_within_tolerance, bf16_to_dev, dev_to_bf16_bits, dev_to_f64,
                      require_gpu, u8_to_dev)
from workloads import bf16_bits_to_f32, f32_to_bf16_bits, make_rows

pytestmark = pytest.mark.gpu

EPI = {"bias": EPI_BIAS, "gelu_tanh": EPI_GELU_TANH, "gated_residual": EPI_GATED_RESIDUAL}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _check_quant(x16, what):
    announce(f"mxfp4 quantize {what} {x16.shape}")
    gq, gs = dq.dq_quantize_mxfp4(bf16_to_dev(x16))
    torch.cuda.synchronize()
    gq, gs = gq.cpu().numpy(), gs.cpu().numpy()
    q, s = quantize_mxfp4(bf16_bits_to_f32(x16))
    assert np.array_equal(gs, s), f"{what}: scale bytes differ at {np.argwhere(gs != s)[:4]}"
    bad = np.argwhere(gq != q)
    assert bad.size == 0, \
        f"{what}: code bytes differ at {bad[:4]}: {gq[tuple(bad[0])]:#x} vs {q[tuple(bad[0])]:#x}"
    return q, s


@pytest.mark.parametrize("M,K", [(1, 32), (3, 64), (17, 96), (64, 3072), (33, 1056)])
def test_quantize_random_rows(M, K):
    rng = np.random.default_rng([M, K, 4])
    x = rng.standard_normal((M, K)).astype(np.float32) * np.exp(rng.uniform(-20, 20, (M, 1)))
    _check_quant(f32_to_bf16_bits(x.astype(np.float32)), "random")


def test_quantize_every_bf16_value_at_scale_one():
    """Every bf16 value below 7.5 in magnitude (both signs), 31 to a block whose first value 7.5
    sets the shared exponent to 0: each code is the E2M1 rounding of the value itself."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bf16_bits_to_f32(bits)
    v = v[np.isfinite(v) & (np.abs(v) < 7.5)]
    n = -(-v.size // 31)
    n += -n % 8                                   # whole rows of 8 blocks
    blocks = np.zeros((n, 32), np.float32)
    blocks[:, 0] = 7.5
    flat = np.zeros(n * 31, np.float32)
    flat[:v.size] = v
    blocks[:, 1:] = flat.reshape(n, 31)
    _check_quant(f32_to_bf16_bits(blocks.reshape(-1, 256)), "every bf16 value at scale 1")


def test_quantize_edge_blocks():
    """Zero blocks (+0 and -0), one nonzero, bf16 subnormal and huge amax, saturating blocks (the
    top binade past 6), negative values that round to zero."""
    K = 32
    rows = [np.zeros(K), -np.zeros(K)]
    r = np.zeros(K); r[7] = -3.0; rows.append(r)
    rows.append(np.full(K, 2.0 ** -133) * np.where(np.arange(K) % 2, 1, -1))
    rows.append(np.full(K, 2.0 ** 127) * 1.5)
    rows.append(np.linspace(-7.9, 7.9, K))                        # 7.9 / 1 saturates to 6
    r = np.full(K, 7.0); r[1::2] = 6.5; rows.append(r)           # all past 6
    r = -np.linspace(0.0, 0.24, K); r[0] = 4.0; rows.append(r)   # negative values to -0
    r = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] * 4 + [4.0] * 4); rows.append(r)
    x = np.array(rows, dtype=np.float32)
    _check_quant(f32_to_bf16_bits(x), "edges")


def test_quantize_activations_full_size():
    _check_quant(make_rows(4608, 3072, seed=22), "flux hidden 4608x3072")


def _linear(q, s, qw, sw, bias16, epi):
    out = dq.dq_linear_mxfp4(u8_to_dev(q), u8_to_dev(s), u8_to_dev(qw), u8_to_dev(sw),
                             None if bias16 is None else bf16_to_dev(bias16), epi)
    torch.cuda.synchronize()
    return out


def _end_to_end(M, K, N, epi, seed, bias=True, rows=None):
    rng = np.random.default_rng([seed, M, K, N, 4])
    x = rng.standard_normal((M, K)).astype(np.float32)
    cols = rng.choice(K, max(1, K // 100), replace=False)
    x[:, cols] *= 30.0
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    b16 = f32_to_bf16_bits((rng.standard_normal(N) * 0.01).astype(np.float32)) if bias else None
    x16, w16 = f32_to_bf16_bits(x), f32_to_bf16_bits(w)
    announce(f"mxfp4 linear {M}x{K}x{N} {epi} bias={bias}")
    q, s = _check_quant(x16, "activations")
    qw, sw = _check_quant(w16, "weights")
    out = dev_to_f64(_linear(q, s, qw, sw, b16, epi))
    rows = np.arange(M) if rows is None else np.asarray(rows)
    ref = linear_mxfp4_ref(q[rows], s[rows], qw, sw,
                           None if b16 is None else bf16_bits_to_f32(b16), EPI[epi])
    assert_within_tolerance(out[rows], ref, what=f"mxfp4 {M}x{K}x{N} {epi}")
    return out


@pytest.mark.parametrize("M,K,N", [(64, 256, 64), (1, 256, 192), (255, 512, 320),
                                   (257, 1024, 256), (300, 768, 512), (513, 256, 64)])
@pytest.mark.parametrize("epi", ["bias", "gelu_tanh"])
def test_tiles_and_ragged_tails(M, K, N, epi):
    _end_to_end(M, K, N, epi, seed=1)


def test_without_bias():
    _end_to_end(96, 512, 128, "bias", seed=2, bias=False)


def test_mlp_up_full_size_sampled_rows():
    """4608 x 3072 -> 12288 with the GELU epilogue (three full rounds of 256 x 256 tiles, then the
    left-over tiles as narrow halves), 64 sampled rows against the oracle."""
    rows = np.unique(np.concatenate([[0, 255, 256, 4607],
                                     np.random.default_rng(5).choice(4608, 60, replace=False)]))
    _end_to_end(4608, 3072, 12288, "gelu_tanh", seed=3, rows=rows)


@pytest.mark.parametrize("K", [256, 512])
def test_more_tiles_than_compute_units_ragged(K):
    """4608 x K -> 3648 (18 x 15 tiles, the last tile column 64 wide; the 14 tiles left after the
    first round run as narrow halves): per-step scale copies at K = 256, grouped at K = 512."""
    rows = np.unique(np.concatenate([[0, 4095, 4096, 4607],
                                     np.random.default_rng(6).choice(4608, 44, replace=False)]))
    _end_to_end(4608, K, 3648, "bias", seed=4, rows=rows)


@pytest.mark.parametrize("steps", [65535, 65534])
def test_longest_k(steps):
    """M = 3, K = 16776960 (the longest the layer accepts: 65535 steps of 256 values; per-step
    scale copies) and 65534 steps (grouped scale copies), N = 64: random codes and scale bytes
    127 +- 6, against the oracle summed over K chunks of 131072."""
    rng = np.random.default_rng(33)
    M, K, N = 3, steps * 256, 64
    q = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    qw = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s = (127 + rng.integers(-6, 7, (M, K // 32))).astype(np.uint8)
    sw = (127 + rng.integers(-6, 7, (N, K // 32))).astype(np.uint8)
    announce(f"mxfp4 longest K {M}x{K}x{N}")
    out = dev_to_f64(_linear(q, s, qw, sw, None, "bias"))
    ref = None
    for k0 in range(0, K, 131072):
        k1 = min(K, k0 + 131072)
        part = linear_mxfp4_ref(q[:, k0 // 2:k1 // 2], s[:, k0 // 32:k1 // 32],
                                qw[:, k0 // 2:k1 // 2], sw[:, k0 // 32:k1 // 32])
        ref = part if ref is None else ref + part
    assert_within_tolerance(out, ref, what="mxfp4 longest K")


def _small_codes(rng, shape):
    """E2M1 codes of 0, 0.5, 1 or 1.5 with random signs."""
    return (rng.integers(0, 4, size=shape) | (rng.integers(0, 2, size=shape) << 3)).astype(np.uint8)


@pytest.mark.parametrize("M,K,N", [(128, 512, 128), (300, 1024, 320)])
def test_exact_inputs_are_bit_exact(M, K, N):
    """Codes of magnitude at most 1.5 and block scales 2^(-1..1): every product is a multiple of
    2^-4 of magnitude at most 9, so every fp32 sum (at most K terms, below 2^14) is exact and the
    output is the bf16 rounding of the exact value."""
    rng = np.random.default_rng(M + K + N + 4)
    q, qw = pack_fp4(_small_codes(rng, (M, K))), pack_fp4(_small_codes(rng, (N, K)))
    s = (127 + rng.integers(-1, 2, (M, K // 32))).astype(np.uint8)
    sw = (127 + rng.integers(-1, 2, (N, K // 32))).astype(np.uint8)
    b16 = f32_to_bf16_bits((rng.integers(-64, 64, N) * 2.0 ** -6).astype(np.float32))
    announce(f"mxfp4 exact {M}x{K}x{N}")
    out = _linear(q, s, qw, sw, b16, "bias")
    ref = linear_mxfp4_ref(q, s, qw, sw, bf16_bits_to_f32(b16), EPI_BIAS)
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)
    want = f32_to_bf16_bits(round_to_bf16(ref).astype(np.float32))
    assert np.array_equal(dev_to_bf16_bits(out), want)


def test_permutation_weights_pick_columns():
    """One-hot weight rows (code 1.0 at column p[n], that block's scale 2^t[n]): output column n is
    the dequantized activation at p[n] times 2^t[n], rounded to bf16. This fixes which K position
    every nibble of both operands lands on, and which scale byte applies to it."""
    rng = np.random.default_rng(9)
    M, K, N = 200, 512, 192
    x16 = f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    q, s = _check_quant(x16, "activations")
    p = rng.choice(K, N, replace=False)
    t = rng.integers(-4, 5, N)
    cw = np.zeros((N, K), np.uint8)
    cw[np.arange(N), p] = 2
    sw = np.full((N, K // 32), 127, np.uint8)
    sw[np.arange(N), p // 32] = 127 + t
    announce("mxfp4 permutation weights")
    out = _linear(q, s, pack_fp4(cw), sw, None, "bias")
    # a sum of products is +0 where the picked value is -0 (E2M1 keeps the sign of values that
    # round to zero; the other products are +0 or -0 too)
    want = dequantize_mxfp4(q, s)[:, p] * np.ldexp(1.0, t)[None, :] + 0.0
    assert np.array_equal(dev_to_bf16_bits(out),
                          f32_to_bf16_bits(round_to_bf16(want).astype(np.float32)))


def test_one_hot_decodes_every_code():
    """Weight rows with a single code c at one K position and activations holding 1.0 there:
    output column n is dec(c) exactly, for all 16 codes, at every position of a 256-value step."""
    M, K, N = 64, 256, 256
    pos = np.arange(N) % K
    codes = np.arange(N) % 16
    cw = np.zeros((N, K), np.uint8)
    cw[np.arange(N), pos] = codes
    ca = np.zeros((M, K), np.uint8)
    ca[:, :] = 2                                                  # every activation 1.0
    s = np.full((M, K // 32), 127, np.uint8)
    sw = np.full((N, K // 32), 127, np.uint8)
    announce("mxfp4 one-hot codes")
    out = dev_to_f64(_linear(pack_fp4(ca), s, pack_fp4(cw), sw, None, "bias"))
    want = np.broadcast_to(decode_fp4_table()[codes][None, :], (M, N))
    assert np.array_equal(out, want)


def test_deterministic_and_m_zero():
    rng = np.random.default_rng(11)
    q = pack_fp4(_small_codes(rng, (96, 512)))
    qw = pack_fp4(_small_codes(rng, (128, 512)))
    s = np.full((96, 16), 120, np.uint8)
    sw = np.full((128, 16), 130, np.uint8)
    a = dev_to_bf16_bits(_linear(q, s, qw, sw, None, "gelu_tanh"))
    b = dev_to_bf16_bits(_linear(q, s, qw, sw, None, "gelu_tanh"))
    assert np.array_equal(a, b)
    e = dq.dq_linear_mxfp4(torch.empty((0, 256), dtype=torch.uint8, device="cuda:0"),
                           torch.empty((0, 16), dtype=torch.uint8, device="cuda:0"),
                           u8_to_dev(qw), u8_to_dev(sw))
    assert e.shape == (0, 128)


def _seg_inputs(seg_rows, K, N, seed):
    """bf16 bit patterns: x [M, K] (N(0,1), a few outlier columns x30), per segment W [N, K]
    (0.02 N(0,1)), bias (0.01 N(0,1)) and gate (1 + 0.1 N(0,1)) [N]; residual [M, N] N(0,1)."""
    rng = np.random.default_rng(seed)
    M = sum(seg_rows)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 30.0
    segs = []
    for _ in seg_rows:
        w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        b = (rng.standard_normal(N) * 0.01).astype(np.float32)
        g = (1.0 + rng.standard_normal(N) * 0.1).astype(np.float32)
        segs.append((f32_to_bf16_bits(w), f32_to_bf16_bits(b), f32_to_bf16_bits(g)))
    res = f32_to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    return f32_to_bf16_bits(x), segs, res


def _check_segments(seg_rows, K, N, epi, seed, sample=None):
    """dq_linear_mxfp4_segmented against one dq_linear_mxfp4 per segment on the same codes (the
    same tiles over the same K steps: the same bits) and against the oracle per segment. The
    gated epilogue runs in place (out is the residual)."""
    announce(f"mxfp4 segmented rows {seg_rows} K={K} N={N} {epi}")
    x, segs, res = _seg_inputs(seg_rows, K, N, seed)
    gated = epi == "gated_residual"
    q, s = dq.dq_quantize_mxfp4(bf16_to_dev(x))
    qws, sws, bs, gs, oracle_w = [], [], [], [], []
    for w, b, g in segs:
        qw, sw = dq.dq_quantize_mxfp4(bf16_to_dev(w))
        qws.append(qw)
        sws.append(sw)
        bs.append(bf16_to_dev(b))
        gs.append(bf16_to_dev(g))
        oracle_w.append(quantize_mxfp4(bf16_bits_to_f32(w)))
    r = bf16_to_dev(res) if gated else None
    out = dq.dq_linear_mxfp4_segmented(q, s, seg_rows, qws, sws, bs, epi,
                                       gs if gated else None, r, out=r)
    parts, r0 = [], 0
    for i, n in enumerate(seg_rows):
        if n:
            rr = bf16_to_dev(res[r0:r0 + n]) if gated else None
            parts.append((r0, n, dq.dq_linear_mxfp4(q[r0:r0 + n].clone(), s[r0:r0 + n].clone(),
                                                    qws[i], sws[i], bs[i], epi,
                                                    gs[i] if gated else None, rr, out=rr)))
        r0 += n
    torch.cuda.synchronize()
    for r0, n, o in parts:
        assert torch.equal(out[r0:r0 + n], o), f"rows {r0}..{r0 + n}: not the bits of one call"
    got = dev_to_f64(out)
    gq, gsc = q.cpu().numpy(), s.cpu().numpy()
    for i, (oqw, osw) in enumerate(oracle_w):
        assert np.array_equal(qws[i].cpu().numpy(), oqw) and np.array_equal(sws[i].cpu().numpy(), osw)
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
        oq, osc = quantize_mxfp4(bf16_bits_to_f32(x[rows]))
        assert np.array_equal(gq[rows], oq) and np.array_equal(gsc[rows], osc)
        ref = linear_mxfp4_ref(oq, osc, *oracle_w[i], bf16_bits_to_f32(b), EPI[epi],
                               bf16_bits_to_f32(g) if gated else None,
                               bf16_bits_to_f32(res[rows]) if gated else None)
        assert_within_tolerance(got[rows], ref, what=f"mxfp4 segment {i} rows {rows[0]}..")


@pytest.mark.parametrize("M,K,N", [(64, 256, 64), (300, 768, 320), (513, 512, 192)])
def test_gated_residual_in_place(M, K, N):
    _check_segments([M], K, N, "gated_residual", seed=20)


def test_gated_residual_separate_output():
    """The gated epilogue with an output other than the residual: the residual is left as it
    was."""
    M, K, N = 200, 512, 128
    x, segs, res = _seg_inputs([M], K, N, seed=21)
    w, b, g = segs[0]
    announce("mxfp4 gated, separate output")
    q, s = dq.dq_quantize_mxfp4(bf16_to_dev(x))
    qw, sw = dq.dq_quantize_mxfp4(bf16_to_dev(w))
    r = bf16_to_dev(res)
    out = dq.dq_linear_mxfp4(q, s, qw, sw, bf16_to_dev(b), "gated_residual", bf16_to_dev(g), r)
    torch.cuda.synchronize()
    assert np.array_equal(dev_to_bf16_bits(r), res)
    oq, osc = quantize_mxfp4(bf16_bits_to_f32(x))
    ref = linear_mxfp4_ref(oq, osc, *quantize_mxfp4(bf16_bits_to_f32(w)), bf16_bits_to_f32(b),
                           EPI_GATED_RESIDUAL, bf16_bits_to_f32(g), bf16_bits_to_f32(res))
    assert_within_tolerance(dev_to_f64(out), ref, what="mxfp4 gated separate output")


@pytest.mark.parametrize("epi", ["bias", "gelu_tanh", "gated_residual"])
def test_segments_two(epi):
    _check_segments([300, 77], 512, 320, epi, seed=22)


def test_segments_ragged_and_empty():
    """Four segments, one empty, none a multiple of 256 rows: each has its own tile rows."""
    _check_segments([1, 255, 0, 257], 256, 192, "gated_residual", seed=23)


@pytest.mark.parametrize("K,N,epi", [(3072, 3072, "bias"), (12288, 3072, "gated_residual")])
def test_segments_flux_joint_sequence(K, N, epi):
    """The 1024^2 double-stream shapes: 4096 image and 512 text tokens in one launch (sampled
    rows of the image segment, every text row)."""
    _check_segments([4096, 512], K, N, epi, seed=24, sample=48)
