"""GPU parity of dq_quantize_fp8 / dq_quantize_weight_fp8 against the oracle: codes and scales
must be bit-identical."""
import numpy as np
import pytest
import torch

import fp8_dynamic_quant_amd as dq
from oracle import quantize_rows
from gpu_util import announce, bf16_to_dev, require_gpu
from workloads import (bf16_bits_to_f32, f32_to_bf16_bits, make_linear_inputs, make_rows,
                       workload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _gpu_quantize(u16, weight=False):
    x = bf16_to_dev(u16)
    fn = dq.dq_quantize_weight_fp8 if weight else dq.dq_quantize_fp8
    q, s = fn(x)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def _assert_same(u16, what, weight=False):
    announce(f"quantize {what} shape={u16.shape} weight={weight}")
    q, s = _gpu_quantize(u16, weight)
    oq, os_ = quantize_rows(bf16_bits_to_f32(u16))
    assert np.array_equal(s.view(np.uint32), os_.view(np.uint32)), \
        f"{what}: {int(np.sum(s.view(np.uint32) != os_.view(np.uint32)))} scales differ"
    if not np.array_equal(q, oq):
        bad = np.argwhere(q != oq)
        r, c = bad[0]
        raise AssertionError(f"{what}: {len(bad)} codes differ; first at {(r, c)}: "
                             f"x={bf16_bits_to_f32(u16)[r, c]!r} gpu={q[r, c]:#04x} "
                             f"oracle={oq[r, c]:#04x} scale={os_[r]!r}")


def test_tiny_workload_activation_and_weight():
    w = workload("tiny-64x256x512")
    inp = make_linear_inputs(w.linears[0], w.seed)
    _assert_same(inp.x, "tiny x")
    _assert_same(inp.w, "tiny w", weight=True)


def test_every_bf16_pattern_at_scale_one():
    """Rows whose amax is 448 have scale exactly 1: the codes are the encoder applied to every
    finite bf16 value with |v| <= 448."""
    u = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = bf16_bits_to_f32(u)
    keep = np.isfinite(f) & (np.abs(f) <= 448.0)
    vals = u[keep]
    K = 4096
    n = (vals.size + K - 2) // (K - 1)
    pad = np.full(n * (K - 1) - vals.size, 0, dtype=np.uint16)
    body = np.concatenate([vals, pad]).reshape(n, K - 1)
    col448 = np.full((n, 1), f32_to_bf16_bits(np.array([448.0], np.float32))[0], np.uint16)
    rows = np.concatenate([col448, body], axis=1)
    _, s = quantize_rows(bf16_bits_to_f32(rows))
    assert np.all(s == 1.0)
    _assert_same(rows, "all bf16 |v|<=448 at scale 1")


def _rows_below(amax_bits, K):
    """Rows of length K that all hold amax (bf16 bits amax_bits) and, between them, every bf16
    value of magnitude <= amax with both signs."""
    mags = np.arange(0, int(amax_bits) + 1, dtype=np.uint32).astype(np.uint16)
    vals = np.concatenate([mags, mags | np.uint16(0x8000)])
    n = (vals.size + K - 2) // (K - 1)
    pad = np.zeros(n * (K - 1) - vals.size, dtype=np.uint16)
    body = np.concatenate([vals, pad]).reshape(n, K - 1)
    return np.concatenate([np.full((n, 1), amax_bits, np.uint16), body], axis=1)


@pytest.mark.parametrize("K", [3072, 16384])
def test_every_value_below_many_scales(K):
    """For amax spread over the whole bf16 range -- a subnormal scale (amax below 448 2^-126),
    rows below 2^-60 (quotient formed from x 2^64 and scale 2^64), ordinary and huge ones --
    every bf16 value with |x| <= amax, through the register-resident kernel (K = 3072) and the
    two-pass one (K = 16384)."""
    picks = [0x0001, 0x0080, 0x0300, 0x05A0, 0x0B40, 0x0C00, 0x0D07, 0x1A3C, 0x2180,
             0x2199, 0x21A0, 0x2F11, 0x3B80, 0x3F80, 0x4080, 0x42F3, 0x43E0, 0x47AB,
             0x5C01, 0x7F7F]
    rng = np.random.default_rng(5)
    picks += [int(v) for v in rng.integers(0x0100, 0x7F7F, 12)]
    for a in picks:
        _assert_same(_rows_below(np.uint16(a), K), f"every value below {a:#06x}, K={K}")


def test_random_amax_rows_spanning_all_magnitudes():
    """2048 rows; row r holds its amax a_r (any positive finite bf16, subnormals included) and
    4095 random bf16 values with |v| <= a_r."""
    rng = np.random.default_rng(17)
    R, K = 2048, 4096
    pos = np.arange(1, 0x7F80, dtype=np.uint16)        # every positive finite bf16
    amax = rng.choice(pos, size=R)
    vals = rng.integers(0, 1 << 16, size=(R, K), dtype=np.uint64).astype(np.uint16)
    mag = vals & 0x7FFF
    mag = np.where(mag > 0x7F7F, mag & 0x3FFF, mag)     # keep finite
    mag = np.minimum(mag, amax[:, None])
    vals = (vals & 0x8000) | mag
    vals[np.arange(R), rng.integers(0, K, R)] = amax
    _assert_same(vals.astype(np.uint16), "random-amax rows")


def test_edge_rows():
    K = 64
    rows = []
    rows.append(np.zeros(K, np.float32))
    z = np.zeros(K, np.float32)
    z[::3] = -0.0
    rows.append(z)
    r = np.zeros(K, np.float32)
    r[[1, 5, 9]] = [2.0 ** -133, -(2.0 ** -133), 2.0 ** -133]      # smallest bf16 subnormal
    rows.append(r)
    r = np.zeros(K, np.float32)
    r[[0, 7]] = [3 * 2.0 ** -128, -(2.0 ** -126)]                   # subnormal scale
    rows.append(r)
    r = np.full(K, 5.0, np.float32)
    r[::2] = -5.0
    rows.append(r)
    r = np.zeros(K, np.float32)
    r[40] = -7.0
    rows.append(r)
    r = np.linspace(-3e38, 3e38, K).astype(np.float32)
    rows.append(r)
    r = np.ones(K, np.float32) * 2.0 ** -100
    r[3] = 1e30
    rows.append(r)
    # ties: amax = 7 * 2^k gives power-of-two scales and exact quotients on E4M3 midpoints
    r = np.arange(K, dtype=np.float32) * np.float32(0.25) - np.float32(8.0)
    r[0] = 7.0 * 2 ** 3
    rows.append(r)
    x = f32_to_bf16_bits(np.array(rows, np.float32))
    _assert_same(x, "edge rows")


# every row layout of the kernel: four rows per wave (K <= 128), one wave per row (K <= 2048),
# two (K <= 8192), four (K <= 32768), and two passes beyond; at and just past each boundary
@pytest.mark.parametrize("M,K", [(1, 8), (3, 24), (5, 520), (7, 1000), (4, 4104), (9, 512),
                                 (13, 16392), (2, 24576), (33, 12288), (2, (1 << 24) + 8),
                                 (5, 2048), (6, 2056), (3, 3072), (7, 3080), (6, 8192), (3, 8200),
                                 (5, 15360), (2, 32768), (3, 32776)])
def test_ragged_shapes(M, K):
    x = make_rows(M, K, seed=M * 7 + K, n_outliers=max(1, K // 100))
    _assert_same(x, f"ragged {M}x{K}")


def test_empty_input():
    x = torch.zeros(0, 64, dtype=torch.bfloat16, device="cuda:0")
    q, s = dq.dq_quantize_fp8(x)
    torch.cuda.synchronize()
    assert q.shape == (0, 64) and s.shape == (0,)


@pytest.mark.parametrize("name,index", [("flux-mlp-up-1024", 0), ("flux-single-block-1024", 0),
                                        ("flux-single-block-1024", 1), ("flux-mlp-up-2048", 0)])
def test_full_size_workloads(name, index):
    w = workload(name)
    shape = w.linears[index]
    inp = make_linear_inputs(shape, w.seed, index)
    _assert_same(inp.x, f"{name}[{index}] x {shape.M}x{shape.K}")
    _assert_same(inp.w, f"{name}[{index}] w {shape.N}x{shape.K}", weight=True)


def test_more_row_groups_than_workgroups():
    """4 * 2^20 + 5 rows of 136 values: one wave per row, four rows per workgroup, and at most
    2^20 workgroups, so the last two row groups are taken by workgroups 0 and 1 on their second
    pass. The first rows, the rows around the wrap and the last rows are checked exactly."""
    M, K = 4 * (1 << 20) + 5, 136
    announce(f"quantize {M}x{K}: more row groups than workgroups")
    g = torch.Generator(device="cuda:0")
    g.manual_seed(77)
    x = torch.randn((M, K), generator=g, device="cuda:0").to(torch.bfloat16)
    q, sc = dq.dq_quantize_fp8(x)
    torch.cuda.synchronize()
    wrap = 4 * (1 << 20)
    rows = np.concatenate([np.arange(8), np.arange(wrap - 8, M),
                           np.random.default_rng(3).choice(M, 64, replace=False)])
    xs = x[torch.from_numpy(rows).to("cuda:0")].contiguous().view(torch.int16).cpu().numpy()
    oq, osc = quantize_rows(bf16_bits_to_f32(xs.view(np.uint16)))
    assert np.array_equal(q.cpu().numpy()[rows], oq)
    assert np.array_equal(sc.cpu().numpy()[rows].view(np.uint32), osc.view(np.uint32))


def test_deterministic():
    x = make_rows(256, 3072, seed=5)
    a = _gpu_quantize(x)
    b = _gpu_quantize(x)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
