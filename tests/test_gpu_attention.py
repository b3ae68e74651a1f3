"""GPU parity of the FP8 attention path (dq_quantize_v_fp8, dq_attention_fp8) against the oracle.

Codes and scales of queries, keys and values must be bit-identical to the oracle's per-row
quantization (values transposed). The attention output is compared with the oracle's float64
attention of the decoded operands within a bound that follows the kernel's arithmetic:
  * a logit t_ij (base 2, t = s log2(e) / sqrt(128)) comes from the FP8 matrix instruction,
    which sums products in fp32 inside a window about 13 bits wide per group: it is off by at
    most 2^-11 of the sum of the absolute products, eps_ij = 2^-11 c sq_i sk_j sum_d |q_id k_jd|;
    the normalized weights then differ by at most a factor 2^(+-2 eps_i), eps_i = max_j eps_ij;
  * each weight times its value scale is rounded to bf16 (2^-9), the bf16 products are summed
    in fp32 with the same windowing, the sum of weights is fp32;
  * the output is rounded to bf16 (half a step, 2^-9 relative).
So |o - ref| <= (2^-8 + 2 ln2 eps_i) A_id + 2^-8 |ref| with A_id = sum_j w_ij |v_jd| (the
weights and dequantized values of the oracle).
"""
import math

import numpy as np
import pytest
import torch

import fp8_dynamic_quant_amd as dq
from oracle import decode_table
from oracle.attention import HEAD_DIM, attention_ref, quantize_heads
from gpu_util import announce, bf16_to_dev, dev_to_f64, require_gpu
from workloads import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

D = HEAD_DIM
C = math.log2(math.e) / math.sqrt(D)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _inputs(H, S, seed, scale=1.0, outlier=0.0):
    """bf16 bit patterns of q, k, v [H, S, D]; `outlier` adds a few large channels."""
    rng = np.random.default_rng([seed, H, S])
    out = []
    for _ in range(3):
        x = rng.standard_normal((H, S, D), dtype=np.float32) * np.float32(scale)
        if outlier:
            x[..., :3] *= np.float32(outlier)
        out.append(f32_to_bf16_bits(x))
    return out


def _run(q16, k16, v16, **kw):
    H, S, _ = q16.shape
    q8, sq, k8, sk, vt, sv = dq.quantize_qkv_heads_fp8(bf16_to_dev(q16), bf16_to_dev(k16),
                                                       bf16_to_dev(v16))
    o = dq.dq_attention_fp8(q8, sq, k8, sk, vt, sv, **kw)
    torch.cuda.synchronize()
    return (q8.cpu().numpy(), sq.cpu().numpy(), k8.cpu().numpy(), sk.cpu().numpy(),
            vt.cpu().numpy(), sv.cpu().numpy(), dev_to_f64(o))


def _check(q16, k16, v16, what, rows=None, **kw):
    H, S, _ = q16.shape
    announce(f"attention {what} H={H} S={S} {kw}")
    gq8, gsq, gk8, gsk, gvt, gsv, o = _run(q16, k16, v16, **kw)
    # codes and scales against the oracle's own quantization
    (q8, sq), (k8, sk), (v8, sv) = (quantize_heads(bf16_bits_to_f32(x)) for x in (q16, k16, v16))
    assert np.array_equal(gq8, q8) and np.array_equal(gsq.view(np.uint32), sq.view(np.uint32))
    assert np.array_equal(gk8, k8) and np.array_equal(gsk.view(np.uint32), sk.view(np.uint32))
    assert np.array_equal(gvt, v8.transpose(0, 2, 1)), "value codes differ"
    assert np.array_equal(gsv.view(np.uint32), sv.view(np.uint32))
    rows = np.arange(S) if rows is None else np.asarray(rows)
    _assert_attention(o[rows].transpose(1, 0, 2), q8, sq, k8, sk, v8, sv, rows, what)
    return o


def _assert_attention(got, q8, sq, k8, sk, v8, sv, rows, what):
    """got [H, n, D]: the outputs of queries `rows` against the oracle's attention of the oracle's
    codes (q8, sq, k8, sk, v8, sv of those H heads), within the bound of the module docstring."""
    ref = attention_ref(q8[:, rows], sq[:, rows], k8, sk, v8, sv)        # [H, n, D]
    table = decode_table()
    qd = table[q8[:, rows]] * sq[:, rows, None].astype(np.float64)
    kd = table[k8] * sk[..., None].astype(np.float64)
    vd = table[v8] * sv[..., None].astype(np.float64)
    logits = np.einsum("hid,hjd->hij", qd, kd) / math.sqrt(D)
    w = np.exp(logits - logits.max(-1, keepdims=True))
    w /= w.sum(-1, keepdims=True)
    A = np.einsum("hij,hjd->hid", w, np.abs(vd))
    eps = 2.0 ** -11 * C * np.einsum("hid,hjd->hij", np.abs(qd), np.abs(kd)).max(-1)  # [H, n]
    bound = (2.0 ** -8 + 2 * math.log(2) * eps[..., None]) * A + 2.0 ** -8 * np.abs(ref) + 1e-30
    err = np.abs(got - ref)
    if not np.all(err <= bound):
        idx = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(f"{what}: {int(np.sum(err > bound))} outputs off; worst {idx}: "
                             f"got {got[idx]!r} ref {ref[idx]!r} bound {bound[idx]:.3g}")
    rel = np.sqrt(np.mean((got - ref) ** 2) / np.mean(ref ** 2))
    print(f"[{what}] worst err/bound {np.max(err / bound):.3f}, rms error / rms output {rel:.2e}, "
          f"max eps {eps.max():.2e}")


def test_offsets_past_two_gigabytes():
    """256 heads x 65536 tokens: the codes of the last head start 2^31 - 2^23 bytes in, so its
    key, value and output addresses pass 2^31. Inputs drawn on the device from a seeded
    generator; the first and last heads' codes and scales against the oracle's quantization of
    those heads, and 6 sampled queries of each against the oracle's attention."""
    H, S = 256, 65536
    announce(f"attention offsets past 2 GiB H={H} S={S}")
    g = torch.Generator(device="cuda:0")
    g.manual_seed(77)
    x16 = [torch.randn((H, S, D), generator=g, device="cuda:0").to(torch.bfloat16)
           for _ in range(3)]
    q8, sq, k8, sk, vt, sv = dq.quantize_qkv_heads_fp8(*x16)
    o = dq.dq_attention_fp8(q8, sq, k8, sk, vt, sv)
    torch.cuda.synchronize()
    heads = [0, H - 1]
    rows = np.array([0, 1, 4095, 32768, S - 385, S - 1])
    got = o[torch.as_tensor(rows, device="cuda:0")][:, heads].float().cpu().numpy()
    got = got.astype(np.float64).transpose(1, 0, 2)                      # [2, n, D]
    bits = [x[heads].view(torch.int16).cpu().numpy().view(np.uint16) for x in x16]
    (oq, osq), (ok, osk), (ov, osv) = (quantize_heads(bf16_bits_to_f32(b)) for b in bits)
    assert np.array_equal(q8[heads].cpu().numpy(), oq)
    assert np.array_equal(sq[heads].cpu().numpy().view(np.uint32), osq.view(np.uint32))
    assert np.array_equal(k8[heads].cpu().numpy(), ok)
    assert np.array_equal(sk[heads].cpu().numpy().view(np.uint32), osk.view(np.uint32))
    assert np.array_equal(vt[heads].cpu().numpy(), ov.transpose(0, 2, 1)), "value codes differ"
    assert np.array_equal(sv[heads].cpu().numpy().view(np.uint32), osv.view(np.uint32))
    _assert_attention(got, oq, osq, ok, osk, ov, osv, rows, "offsets past 2 GiB")


@pytest.mark.parametrize("H,S", [(1, 16), (2, 48), (1, 64), (2, 80), (3, 128), (2, 144),
                                 (1, 272), (2, 512)])
def test_ragged_sequences(H, S):
    """Sequences that end inside a 64-key block and inside a 128-query workgroup."""
    q, k, v = _inputs(H, S, 1)
    _check(q, k, v, f"ragged {H}x{S}")


@pytest.mark.parametrize("scale,outlier", [(3.0, 0.0), (0.05, 0.0), (1.0, 20.0)])
def test_sharp_flat_and_outlier_logits(scale, outlier):
    """Peaked weights (logits of spread ~9), nearly uniform ones, and a few large channels that
    dominate the row scales."""
    q, k, v = _inputs(2, 320, 2, scale, outlier)
    _check(q, k, v, f"scale {scale} outlier {outlier}")


def test_flux_joint_attention_1024px():
    """24 heads over 4608 tokens (4096 image + 512 text), 64 sampled queries per head."""
    q, k, v = _inputs(24, 4608, 3)
    rows = np.unique(np.concatenate([[0, 127, 128, 4095, 4607],
                                     np.random.default_rng(4).choice(4608, 59, replace=False)]))
    _check(q, k, v, "flux 24x4608", rows=rows)


def test_single_dominant_key():
    """One key far above the rest in every row: the output is that key's value row."""
    H, S = 1, 96
    rng = np.random.default_rng(5)
    q = np.zeros((H, S, D), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((H, S, D), np.float32)
    k[0, 41, 0] = 200.0
    v = rng.standard_normal((H, S, D)).astype(np.float32)
    q16, k16, v16 = (f32_to_bf16_bits(x) for x in (q, k, v))
    o = _check(q16, k16, v16, "dominant key")
    vd = decode_table()[quantize_heads(bf16_bits_to_f32(v16))[0]] * \
        quantize_heads(bf16_bits_to_f32(v16))[1][..., None]
    # two bf16 roundings (the weight times its value scale, then the output): 2^-8 + a little
    assert np.allclose(o[:, 0, :], vd[0, 41][None, :], rtol=2 ** -7, atol=1e-6)


def test_zero_queries_average_the_values():
    """A zero query row has zero logits: its output is the mean of the values."""
    H, S = 2, 64
    q, k, v = _inputs(H, S, 6)
    q = np.zeros_like(q)
    _check(q, k, v, "zero queries")


def test_deterministic_and_empty():
    q, k, v = _inputs(2, 80, 7)
    a = _run(q, k, v)[-1]
    b = _run(q, k, v)[-1]
    assert np.array_equal(a, b)
    e = dq.dq_attention_fp8(torch.empty((3, 0, D), dtype=torch.uint8, device="cuda:0"),
                            torch.empty((3, 0), device="cuda:0"),
                            torch.empty((3, 0, D), dtype=torch.uint8, device="cuda:0"),
                            torch.empty((3, 0), device="cuda:0"),
                            torch.empty((3, D, 0), dtype=torch.uint8, device="cuda:0"),
                            torch.empty((3, 0), device="cuda:0"))
    assert e.shape == (0, 3, D)


# (H, S, max_workgroups): tiles = H ceil(S / 384) above the cap cut tiles between neighbouring
# workgroups; caps that are multiples of 8 also renumber workgroups by XCD.
SPLIT_CASES = [(3, 128, 2), (3, 272, 2), (4, 1040, 5), (3, 1040, 8), (2, 4608, 16), (5, 400, 7),
               (4, 512, 8)]


@pytest.mark.parametrize("H,S,cap", SPLIT_CASES)
def test_cut_tiles(H, S, cap):
    """Runs of key blocks that start and end inside tiles (two parts merged through the
    workspace), ragged last blocks, and one tile per workgroup (4 x 512 with 8)."""
    q, k, v = _inputs(H, S, 12)
    ws = torch.zeros(dq.dq_attention_fp8_workspace_size(H, S), dtype=torch.uint8,
                     device="cuda:0")
    o = _check(q, k, v, f"cut {H}x{S} cap {cap}", workspace=ws, max_workgroups=cap)
    assert int(ws[:4096].count_nonzero()) == 0, "arrival counters left non-zero"
    again = _run(q, k, v, workspace=ws, max_workgroups=cap)[-1]
    assert np.array_equal(o, again), "cut tiles: result depends on the run"
    assert int(ws[:4096].count_nonzero()) == 0


@pytest.mark.parametrize("H,S,cap", [(3, 128, 2), (4, 1040, 5), (3, 1040, 8)])
def test_whole_tile_runs_without_workspace(H, S, cap):
    """More tiles than workgroups and no workspace: each workgroup takes whole tiles."""
    q, k, v = _inputs(H, S, 13)
    _check(q, k, v, f"whole runs {H}x{S} cap {cap}", workspace=None, max_workgroups=cap)


def test_flux_attention_cut_and_uncut_agree():
    """The default schedule on 24 x 4608 (tiles cut between workgroups) against whole tiles per
    workgroup: both within the bound of the oracle (sampled), and close to each other."""
    q, k, v = _inputs(24, 4608, 14)
    a = _run(q, k, v)[-1]
    b = _run(q, k, v, workspace=None)[-1]
    d = np.abs(a - b)
    assert np.max(d) <= 2.0 ** -7 * np.max(np.abs(b)), np.max(d)
