"""GPU parity of dq_linear_fp8 (FP8 GEMM + fused epilogue) against the oracle.

Where the arithmetic is exact on both sides (codes of narrow dynamic range, power-of-two
scales, permutation and one-hot weights) the bf16 outputs must match bit for bit. Elsewhere every
output must satisfy |out - ref| <= 4e-3 |ref| + 1e-3 rms(ref), ref being the oracle's value
before bf16 rounding.

The FP8 matrix instruction sums each group of 8 products in a fixed-point window about 13 bits
wide below the group's largest product (measured on gfx950), so "exact" cases keep every group's
products within that window.
"""
import numpy as np
import pytest
import torch

import fp8_dynamic_quant_amd as dq
from oracle import decode_table, linear_ref, quantize_rows, round_to_bf16
from gpu_util import (announce, assert_within_tolerance, bf16_to_dev, dev_to_bf16_bits,
                      dev_to_f64, f32_to_dev, require_gpu, u8_to_dev)
from workloads import (LinearShape, bf16_bits_to_f32, f32_to_bf16_bits, make_linear_inputs,
                       workload)

pytestmark = pytest.mark.gpu

EPIS = ("bias", "gelu_tanh", "gated_residual")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _bits_of(ref64):
    """bf16 bit patterns of the nearest-even bf16 of float64 values."""
    return (round_to_bf16(ref64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


WS = ("auto", None)   # tile-sharing schedule through a workspace, and whole tiles only


def _run_linear(q, sa, qw, sw, bias, epi, gate=None, residual=None, inplace=False, ws="auto"):
    """q, qw uint8; sa, sw float32; bias/gate/residual bf16 bit patterns (or None)."""
    tq, tsa, tqw, tsw = u8_to_dev(q), f32_to_dev(sa), u8_to_dev(qw), f32_to_dev(sw)
    tb = None if bias is None else bf16_to_dev(bias)
    tg = None if gate is None else bf16_to_dev(gate)
    tr = None if residual is None else bf16_to_dev(residual)
    out = tr if inplace else None
    o = dq.dq_linear_fp8(tq, tsa, tqw, tsw, tb, epi, tg, tr, out=out, workspace=ws)
    torch.cuda.synchronize()
    return o


def _end_to_end(shape: LinearShape, seed, index=0, rows=None, inplace=False, ws="auto"):
    """Quantize x and W on the GPU, run the linear on the GPU; compare codes/scales exactly and
    the outputs (all rows, or the sampled `rows`) within tolerance."""
    inp = make_linear_inputs(shape, seed, index)
    announce(f"linear {shape.name} M={shape.M} K={shape.K} N={shape.N} epi={shape.epilogue} "
             f"workspace={ws}")
    tx, tw = bf16_to_dev(inp.x), bf16_to_dev(inp.w)
    q, sa = dq.dq_quantize_fp8(tx)
    qw, sw = dq.dq_quantize_weight_fp8(tw)
    tb = bf16_to_dev(inp.bias)
    tg = tr = None
    if shape.epilogue == "gated_residual":
        tg, tr = bf16_to_dev(inp.gate), bf16_to_dev(inp.residual)
    out = dq.dq_linear_fp8(q, sa, qw, sw, tb, shape.epilogue, tg, tr,
                           out=tr if inplace else None, workspace=ws)
    torch.cuda.synchronize()
    del tx, tw
    rows = np.arange(shape.M) if rows is None else np.asarray(rows)
    xs = bf16_bits_to_f32(inp.x[rows])
    oq, osa = quantize_rows(xs)
    oqw, osw = quantize_rows(bf16_bits_to_f32(inp.w))
    gq = q.cpu().numpy()[rows]
    assert np.array_equal(gq, oq), "activation codes differ"
    assert np.array_equal(sa.cpu().numpy()[rows].view(np.uint32), osa.view(np.uint32))
    assert np.array_equal(qw.cpu().numpy(), oqw), "weight codes differ"
    assert np.array_equal(sw.cpu().numpy().view(np.uint32), osw.view(np.uint32))
    gate = None if inp.gate is None else bf16_bits_to_f32(inp.gate)
    res = None if inp.residual is None else bf16_bits_to_f32(inp.residual[rows])
    ref = linear_ref(oq, osa, oqw, osw, bf16_bits_to_f32(inp.bias), shape.epilogue, gate, res)
    got = dev_to_f64(out)[rows]
    return assert_within_tolerance(got, ref, what=f"{shape.name} {shape.epilogue}")


@pytest.mark.parametrize("ws", WS)
@pytest.mark.parametrize("epi", EPIS)
def test_tiny_workload_all_epilogues(epi, ws):
    w = workload("tiny-64x256x512")
    base = w.linears[0]
    shape = LinearShape(base.name, base.M, base.K, base.N, epi, base.n_outliers,
                        base.outlier_factor)
    _end_to_end(shape, w.seed, ws=ws)


@pytest.mark.parametrize("M,K,N", [(300, 384, 320), (257, 128, 64), (1, 128, 64), (5, 256, 192),
                                   (513, 640, 576), (64, 3072, 512), (700, 1152, 1088)])
@pytest.mark.parametrize("epi", EPIS)
@pytest.mark.parametrize("ws", WS)
def test_tiles_and_ragged_tails(M, K, N, epi, ws):
    shape = LinearShape(f"ragged{M}x{K}x{N}", M, K, N, epi, max(1, K // 100), 30.0)
    _end_to_end(shape, seed=1000 + M + K + N, ws=ws)


@pytest.mark.parametrize("M,K,N", [(256, 8192, 256), (40, 4096, 192), (600, 5120, 448),
                                   (256, 6400, 768), (2304, 3072, 2560)])
def test_tiles_shared_by_many_workgroups(M, K, N):
    """Few tiles and a long K: with a workspace each tile is cut along K into up to 8 parts
    (8 for one tile of 64 steps, 5 for three tiles of 50 steps) that the last arriving part
    sums."""
    shape = LinearShape(f"split{M}x{K}x{N}", M, K, N, "gated_residual", K // 100, 30.0)
    _end_to_end(shape, seed=2000 + M + K + N, ws="auto")


def test_gated_in_place_equals_out_of_place():
    shape = LinearShape("inplace", 300, 512, 320, "gated_residual", 5, 30.0)
    inp = make_linear_inputs(shape, 77)
    announce("gated in place vs out of place")
    q, sa = dq.dq_quantize_fp8(bf16_to_dev(inp.x))
    qw, sw = dq.dq_quantize_weight_fp8(bf16_to_dev(inp.w))
    b, g = bf16_to_dev(inp.bias), bf16_to_dev(inp.gate)
    r1 = bf16_to_dev(inp.residual)
    r2 = bf16_to_dev(inp.residual)
    o1 = dq.dq_linear_fp8(q, sa, qw, sw, b, "gated_residual", g, r1)
    o2 = dq.dq_linear_fp8(q, sa, qw, sw, b, "gated_residual", g, r2, out=r2)
    torch.cuda.synchronize()
    assert o2.data_ptr() == r2.data_ptr()
    assert torch.equal(o1, r2)
    assert torch.equal(r1, bf16_to_dev(inp.residual))   # out-of-place left residual untouched


def _narrow_codes(rng, shape):
    """Codes of values in [1, 2) and [2, 4) with random signs: every product lies in [1, 16)
    and is a multiple of 2^-6, so a group of 8 spans < 2^7 / 2^-6 = 2^13: exact in the MFMA."""
    mant = rng.integers(0, 8, size=shape)
    exp_field = rng.integers(7, 9, size=shape)           # 2^0 or 2^1
    sign = rng.integers(0, 2, size=shape) << 7
    return (sign | (exp_field << 3) | mant).astype(np.uint8)


@pytest.mark.parametrize("ws", WS)
@pytest.mark.parametrize("epi,M,K,N", [(e, M, K, N) for e in ("bias", "gated_residual")
                                       for M, K, N in ((256, 256, 256), (300, 1024, 320),
                                                       (64, 128, 64))]
                         + [("bias", 256, 8192, 256), ("bias", 96, 6144, 320)])
def test_exact_inputs_are_bit_exact(M, K, N, epi, ws):
    rng = np.random.default_rng(M + K + N)
    q = _narrow_codes(rng, (M, K))
    qw = _narrow_codes(rng, (N, K))
    # acc = A 2^-6 with |A| < 2^10 K; sa sw = 2^e, e in [-10, -6]; bias = B 2^-6, |B| <= 64;
    # gate = 2^g, g in [-1, 1]; residual = R 2^-4, |R| <= 64. Then every intermediate is an
    # integer below 2^24 times 2^(e - 6 + g): exact in fp32 for K <= 4096.
    sa = np.ldexp(1.0, rng.integers(-5, -2, M)).astype(np.float32)
    sw = np.ldexp(1.0, rng.integers(-5, -2, N)).astype(np.float32)
    bias = f32_to_bf16_bits((rng.integers(-64, 64, N) * 2.0 ** -6).astype(np.float32))
    gate = res = None
    if epi == "gated_residual":
        gate = f32_to_bf16_bits(np.ldexp(1.0, rng.integers(-1, 2, N)).astype(np.float32))
        res = f32_to_bf16_bits((rng.integers(-64, 64, (M, N)) * 2.0 ** -4).astype(np.float32))
    announce(f"exact linear {M}x{K}x{N} {epi} workspace={ws}")
    out = _run_linear(q, sa, qw, sw, bias, epi, gate, res, ws=ws)
    ref = linear_ref(q, sa, qw, sw, bf16_bits_to_f32(bias), epi,
                     None if gate is None else bf16_bits_to_f32(gate),
                     None if res is None else bf16_bits_to_f32(res))
    # the exact value is a float32 here, so one rounding to bf16 is what both sides do
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)
    assert np.array_equal(dev_to_bf16_bits(out), _bits_of(ref))


# Shapes of more than 128 tiles (too many for narrow halves) whose last round runs whole (no
# workspace): every tile is a whole 256 x 256 tile, including ragged last tile rows and columns.
WHOLE_TILES = [(2500, 1024, 3520), (2560, 512, 3584), (4608, 3072, 3072)]


@pytest.mark.parametrize("epi", EPIS)
def test_whole_tiles_ragged(epi):
    """2500 x 1024 -> 3520: 10 x 14 tiles, the last tile row 196 rows and the last tile column
    192 columns wide; every output against the oracle."""
    M, K, N = WHOLE_TILES[0]
    shape = LinearShape(f"whole_{M}x{K}x{N}", M, K, N, epi, K // 100, 30.0)
    _end_to_end(shape, seed=4000 + len(epi), ws=None)


@pytest.mark.parametrize("epi", ["bias", "gated_residual"])
@pytest.mark.parametrize("M,K,N", [WHOLE_TILES[1], (2500, 512, 3520)])
def test_whole_tiles_exact_inputs_are_bit_exact(M, K, N, epi):
    """The exact-input construction of test_exact_inputs_are_bit_exact on whole-tile shapes."""
    rng = np.random.default_rng(M + K + N + 7)
    q = _narrow_codes(rng, (M, K))
    qw = _narrow_codes(rng, (N, K))
    sa = np.ldexp(1.0, rng.integers(-5, -2, M)).astype(np.float32)
    sw = np.ldexp(1.0, rng.integers(-5, -2, N)).astype(np.float32)
    bias = f32_to_bf16_bits((rng.integers(-64, 64, N) * 2.0 ** -6).astype(np.float32))
    gate = res = None
    if epi == "gated_residual":
        gate = f32_to_bf16_bits(np.ldexp(1.0, rng.integers(-1, 2, N)).astype(np.float32))
        res = f32_to_bf16_bits((rng.integers(-64, 64, (M, N)) * 2.0 ** -4).astype(np.float32))
    announce(f"whole-tile exact linear {M}x{K}x{N} {epi}")
    out = _run_linear(q, sa, qw, sw, bias, epi, gate, res, ws=None)
    ref = linear_ref(q, sa, qw, sw, bf16_bits_to_f32(bias), epi,
                     None if gate is None else bf16_bits_to_f32(gate),
                     None if res is None else bf16_bits_to_f32(res))
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)
    assert np.array_equal(dev_to_bf16_bits(out), _bits_of(ref))


def test_whole_tiles_gated_in_place_and_deterministic():
    """4608 x 3072 -> 3072 (one round of 216 tiles): in place equals out of place, the residual
    of the out-of-place call is untouched, and a second call gives the same bits."""
    M, K, N = WHOLE_TILES[2]
    shape = LinearShape("whole_inplace", M, K, N, "gated_residual", K // 100, 30.0)
    inp = make_linear_inputs(shape, 78)
    announce("whole-tile gated in place vs out of place")
    q, sa = dq.dq_quantize_fp8(bf16_to_dev(inp.x))
    qw, sw = dq.dq_quantize_weight_fp8(bf16_to_dev(inp.w))
    b, g = bf16_to_dev(inp.bias), bf16_to_dev(inp.gate)
    r1 = bf16_to_dev(inp.residual)
    r2 = bf16_to_dev(inp.residual)
    o1 = dq.dq_linear_fp8(q, sa, qw, sw, b, "gated_residual", g, r1, workspace=None)
    o3 = dq.dq_linear_fp8(q, sa, qw, sw, b, "gated_residual", g, r1, workspace=None)
    o2 = dq.dq_linear_fp8(q, sa, qw, sw, b, "gated_residual", g, r2, out=r2, workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(o1, r2) and torch.equal(o1, o3)
    assert torch.equal(r1, bf16_to_dev(inp.residual))


def test_permutation_weights_are_bit_exact():
    """W = 448 P: sw = 1, qw = 0x7E at pi(n): out[:, n] = bf16(448 dec(q[:, pi(n)]) sa + b[n])."""
    rng = np.random.default_rng(3)
    M, K = 320, 512
    N = K
    perm = rng.permutation(K)
    W = np.zeros((N, K), np.float32)
    W[np.arange(N), perm] = 448.0
    x = f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    bias = f32_to_bf16_bits((rng.standard_normal(N) * 0.01).astype(np.float32))
    announce("permutation weights")
    q, sa = dq.dq_quantize_fp8(bf16_to_dev(x))
    qw, sw = dq.dq_quantize_weight_fp8(bf16_to_dev(f32_to_bf16_bits(W)))
    out = dq.dq_linear_fp8(q, sa, qw, sw, bf16_to_dev(bias), "bias")
    torch.cuda.synchronize()
    oq, osa = quantize_rows(bf16_bits_to_f32(x))
    assert np.all(sw.cpu().numpy() == 1.0)
    t = decode_table()
    acc = 448.0 * t[oq[:, perm]]
    # acc * sa is one rounding in fp32 on the GPU; adding the bias is a second
    want = (acc.astype(np.float32) * osa[:, None]).astype(np.float32) + bf16_bits_to_f32(bias)[None, :]
    assert np.array_equal(dev_to_bf16_bits(out), _bits_of(want.astype(np.float64)))


def test_one_hot_weights_decode_every_code():
    """Activation codes run through all 254 finite E4M3 bytes; one-hot weights (1.0 at k == n)
    with unit scales give out[m, n] = dec(q[m, n]) exactly: the matrix units read OCP E4M3."""
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    M, K = 4, 256
    N = K
    q = np.zeros((M, K), np.uint8)
    q[0, :254] = finite
    q[1, :254] = finite[::-1]
    q[2] = np.roll(q[0], 17)
    q[3] = 0x38
    qw = np.zeros((N, K), np.uint8)
    qw[np.arange(N), np.arange(N)] = 0x38
    ones_m, ones_n = np.ones(M, np.float32), np.ones(N, np.float32)
    announce("one-hot weights over every code")
    out = _run_linear(q, ones_m, qw, ones_n, None, "bias")
    t = decode_table()
    want = t[q]
    got = dev_to_f64(out)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got[0, :254]), np.signbit(want[0, :254]) & (want[0, :254] != 0))


@pytest.mark.parametrize("name,index,inplace", [
    ("flux-mlp-up-1024", 0, False),
    ("flux-single-block-1024", 0, False),
    ("flux-single-block-1024", 1, True),
    ("flux-mlp-up-2048", 0, False),
    ("flux-dit-step-1024", 3, True),     # image-stream fc2: 4096 x 12288 -> 3072, 192 tiles
    ("flux-dit-step-1024", 7, True),     # text-stream fc2: 512 x 12288 -> 3072, 24 tiles
    ("flux-dit-step-1024", 6, False),    # text-stream fc1: 512 x 3072 -> 12288
])
def test_full_size_workloads_sampled_rows(name, index, inplace):
    """Full-size launch exactly as the benchmark runs it; every code and scale is compared, and
    all outputs of 64 sampled rows (first, last, random) against the oracle."""
    w = workload(name)
    shape = w.linears[index]
    rng = np.random.default_rng(99)
    rows = np.unique(np.concatenate([[0, shape.M - 1], rng.choice(shape.M, 62, replace=False)]))
    _end_to_end(shape, w.seed, index, rows=rows, inplace=inplace)


@pytest.mark.parametrize("M,K,N,epi", [(5120, 3072, 3584, "gelu_tanh"),
                                       (4608, 3072, 12288, "bias")])
def test_full_rounds_then_cut_tiles_sampled_rows(M, K, N, epi):
    """More tiles than compute units: whole tiles for the full rounds, then the left-over tiles
    (24 of 280; 96 of 864) cut along K; sampled rows against the oracle, both schedules."""
    shape = LinearShape(f"rounds{M}x{K}x{N}", M, K, N, epi, K // 100, 30.0)
    rng = np.random.default_rng(M + N)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 62, replace=False)]))
    for ws in WS:
        _end_to_end(shape, seed=3000 + M + N, rows=rows, ws=ws)


# The longest K the linear layer accepts is below 2^24 (a 256-row operand tile stays within one
# 32-bit buffer range); 131070 K steps of 128 (= 2 3 5 17 257) also let a tile be cut into 2, 3,
# 5 or 6 parts.
K_LONGEST = 131070 * 128


def _chunked_ref(contract_chunk, K, chunk):
    """Sum of the oracle's float64 values over K chunks (the layer is linear in each K range; the
    oracle's exact contraction takes at most 131072 terms per call)."""
    ref = None
    for k0 in range(0, K, chunk):
        part = contract_chunk(k0, min(K, k0 + chunk))
        ref = part if ref is None else ref + part
    return ref


def test_longest_k():
    """M = 3, K = 16776960, N = 64 (one tile, 131070 K steps): whole tile and cut into parts,
    random codes, power-of-two scales, against the oracle summed over K chunks."""
    rng = np.random.default_rng(31)
    M, K, N = 3, K_LONGEST, 64
    q = rng.integers(0, 256, size=(M, K), dtype=np.uint8)
    qw = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x01
    qw[(qw & 0x7F) == 0x7F] = 0x02
    sa = np.ldexp(1.0, rng.integers(-12, -6, M)).astype(np.float32)
    sw = np.ldexp(1.0, rng.integers(-12, -6, N)).astype(np.float32)
    announce(f"linear longest K {M}x{K}x{N}")
    ref = _chunked_ref(lambda a, b: linear_ref(q[:, a:b], sa, qw[:, a:b], sw), K, 131072)
    for ws in WS:
        got = dev_to_f64(_run_linear(q, sa, qw, sw, None, "bias", ws=ws))
        assert_within_tolerance(got, ref, what=f"longest K workspace={ws}")


def test_deterministic_and_m_zero():
    shape = LinearShape("det", 513, 768, 640, "gelu_tanh", 8, 30.0)
    inp = make_linear_inputs(shape, 5)
    q, sa = dq.dq_quantize_fp8(bf16_to_dev(inp.x))
    qw, sw = dq.dq_quantize_weight_fp8(bf16_to_dev(inp.w))
    b = bf16_to_dev(inp.bias)
    o1 = dq.dq_linear_fp8(q, sa, qw, sw, b, "gelu_tanh")
    o2 = dq.dq_linear_fp8(q, sa, qw, sw, b, "gelu_tanh")
    e = dq.dq_linear_fp8(q[:0], sa[:0], qw, sw, b, "gelu_tanh")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert e.shape == (0, 640)


def test_workspace_is_left_zeroed_and_reusable():
    """An explicit workspace: after every completed call its arrival counters are zero again, so
    back-to-back calls of different sizes can share it; results equal the whole-tile schedule
    on exact inputs."""
    rng = np.random.default_rng(11)
    shapes = [(256, 8192, 256), (520, 2048, 640), (64, 128, 64)]
    need = max(dq.dq_linear_fp8_workspace_size(M, K, N) for M, K, N in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for M, K, N in shapes:
        announce(f"explicit workspace {M}x{K}x{N}")
        q, qw = _narrow_codes(rng, (M, K)), _narrow_codes(rng, (N, K))
        sa = np.ldexp(1.0, rng.integers(-5, -2, M)).astype(np.float32)
        sw = np.ldexp(1.0, rng.integers(-5, -2, N)).astype(np.float32)
        a = _run_linear(q, sa, qw, sw, None, "bias", ws=ws)
        b = _run_linear(q, sa, qw, sw, None, "bias", ws=None)
        assert torch.equal(a, b)
        counters = ws[:4096].view(torch.int32)            # one per cut tile, first in the layout
        assert int(counters.abs().sum().item()) == 0
