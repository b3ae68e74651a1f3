"""Seeded synthetic inputs for the FP8 dynamic-quant linear layers of a FLUX-dev-shaped DiT.

This module only draws random numbers and rounds them to bf16 storage. It holds none of the
method's arithmetic (no amax, no scale, no FP8 encoding, no contraction), so both the CPU oracle
and the GPU path may take their inputs from it without sharing any code of the method.

Shapes are those of FLUX-dev's linear layers at 1024x1024 and 2048x2048 (3072-wide hidden state,
4096 / 16384 image tokens plus 512 text tokens, MLP ratio 4, single-stream blocks that fuse the
QKV and MLP projections). The model and its hybrid double-stream / single-stream design are
described on the page "WaveSpeedAI X DataCrunch: Inferencia de Imagenes FLUX en Tiempo Real en
B200", section "FLUX-Dev"; the pages print no tensor data, so every value here is synthetic.

Recipe (host side, NumPy PCG64, one generator per linear seeded with [seed, linear_index]):
  1. outlier columns: rng.choice(K, n_outliers, replace=False)
  2. x = N(0,1) [M,K] float32, outlier columns multiplied by the outlier factor
  3. W = 0.02 * N(0,1) [N,K]
  4. bias = 0.01 * N(0,1) [N]
  5. gate = 1 + 0.1 * N(0,1) [N]          (gated-residual linears only)
  6. residual = N(0,1) [M,N]              (gated-residual linears only)
Every float32 draw is rounded to the nearest bf16 (ties to even) for storage.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

EPILOGUES = ("bias", "gelu_tanh", "gated_residual")


@dataclass(frozen=True)
class LinearShape:
    """One dynamically quantized linear: x[M,K] -> out[M,N]."""
    name: str
    M: int
    K: int
    N: int
    epilogue: str            # one of EPILOGUES
    n_outliers: int
    outlier_factor: float

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


def _n_outliers(K: int) -> int:
    return int(round(0.01 * K))


def _lin(name, M, K, N, epi, n_out=None, factor=30.0) -> LinearShape:
    return LinearShape(name, M, K, N, epi, _n_outliers(K) if n_out is None else n_out, factor)


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    linears: List[LinearShape] = field(default_factory=list)
    repeat: Optional[List[int]] = None   # multiplicity of each linear in a step (DiT step only)
    description: str = ""

    @property
    def flops_per_step(self) -> int:
        rep = self.repeat or [1] * len(self.linears)
        return sum(r * l.flops for r, l in zip(rep, self.linears))


def _dit_step_linears() -> (List[LinearShape], List[int]):
    """Distinct linear shapes of one 1024x1024 FLUX-dev denoising step, with multiplicities.

    19 double-stream blocks x {image M=4096, text M=512} x {QKV, proj, fc1, fc2}, then 38
    single-stream blocks on M=4608 running linear1 and linear2.
    """
    lins, rep = [], []
    for stream, M in (("img", 4096), ("txt", 512)):
        lins += [
            _lin(f"double.{stream}.qkv", M, 3072, 9216, "bias"),
            _lin(f"double.{stream}.proj", M, 3072, 3072, "bias"),
            _lin(f"double.{stream}.fc1", M, 3072, 12288, "gelu_tanh"),
            _lin(f"double.{stream}.fc2", M, 12288, 3072, "gated_residual"),
        ]
        rep += [19] * 4
    lins += [
        _lin("single.linear1", 4608, 3072, 21504, "bias"),
        _lin("single.linear2", 4608, 15360, 3072, "gated_residual"),
    ]
    rep += [38, 38]
    return lins, rep


def workloads() -> List[Workload]:
    dit, rep = _dit_step_linears()
    return [
        Workload("tiny-64x256x512", 0,
                 [_lin("tiny", 64, 256, 512, "bias", n_out=4, factor=20.0)],
                 description="tiny W8A8 linear, bias epilogue"),
        Workload("flux-mlp-up-1024", 1,
                 [_lin("mlp.fc1", 4608, 3072, 12288, "gelu_tanh")],
                 description="FLUX-dev MLP up-projection at 1024^2 (4096 image + 512 text tokens), GELU-tanh"),
        Workload("flux-single-block-1024", 2,
                 [_lin("single.linear1", 4608, 3072, 21504, "bias"),
                  _lin("single.linear2", 4608, 15360, 3072, "gated_residual")],
                 description="FLUX-dev single-stream block pair at 1024^2: linear1 (bias), linear2 (gated residual)"),
        Workload("flux-mlp-up-2048", 3,
                 [_lin("mlp.fc1", 16896, 3072, 12288, "gelu_tanh")],
                 description="MLP up-projection at 2048^2 (16384 image + 512 text tokens), GELU-tanh"),
        Workload("flux-dit-step-1024", 4, dit, rep,
                 description="all linears of one FLUX-dev denoising step at 1024^2, batch 1"),
    ]


def workload(name: str) -> Workload:
    for w in workloads():
        if w.name == name:
            return w
    raise KeyError(name)


# ---------------------------------------------------------------------------------------------
# bf16 storage (input generation only)
# ---------------------------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Nearest bf16 (ties to even) of finite float32 values, as uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("inputs must be finite")
    b = a.view(np.uint32).astype(np.uint64)
    b = b + 0x7FFF + ((b >> 16) & 1)
    return (b >> 16).astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Exact float32 value of bf16 bit patterns."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32)


@dataclass
class LinearInputs:
    """bf16 tensors of one linear, as uint16 bit patterns (host memory)."""
    shape: LinearShape
    x: np.ndarray                      # [M,K]
    w: np.ndarray                      # [N,K]
    bias: np.ndarray                   # [N]
    gate: Optional[np.ndarray] = None  # [N]
    residual: Optional[np.ndarray] = None  # [M,N]
    outlier_cols: Optional[np.ndarray] = None


def make_linear_inputs(shape: LinearShape, seed: int, index: int = 0) -> LinearInputs:
    """Draw the inputs of one linear from NumPy PCG64 seeded with [seed, index] (whole tensors,
    so that every consumer sees the same values)."""
    rng = np.random.default_rng([seed, index])
    M, K, N = shape.M, shape.K, shape.N
    cols = rng.choice(K, shape.n_outliers, replace=False) if shape.n_outliers else np.zeros(0, np.int64)
    x = rng.standard_normal((M, K), dtype=np.float32)
    if cols.size:
        x[:, cols] *= np.float32(shape.outlier_factor)
    w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    bias = rng.standard_normal(N, dtype=np.float32) * np.float32(0.01)
    gate = residual = None
    if shape.epilogue == "gated_residual":
        gate = np.float32(1.0) + rng.standard_normal(N, dtype=np.float32) * np.float32(0.1)
        residual = rng.standard_normal((M, N), dtype=np.float32)
    return LinearInputs(
        shape=shape,
        x=f32_to_bf16_bits(x),
        w=f32_to_bf16_bits(w),
        bias=f32_to_bf16_bits(bias),
        gate=None if gate is None else f32_to_bf16_bits(gate),
        residual=None if residual is None else f32_to_bf16_bits(residual),
        outlier_cols=np.sort(cols),
    )


def make_rows(M: int, K: int, seed: int, n_outliers: Optional[int] = None,
              factor: float = 30.0, sigma: float = 1.0) -> np.ndarray:
    """bf16 bit patterns of an [M,K] activation-like tensor (for quantizer-only cases)."""
    rng = np.random.default_rng([seed, 7919])
    n = _n_outliers(K) if n_outliers is None else n_outliers
    cols = rng.choice(K, n, replace=False) if n else np.zeros(0, np.int64)
    x = rng.standard_normal((M, K), dtype=np.float32) * np.float32(sigma)
    if cols.size:
        x[:, cols] *= np.float32(factor)
    return f32_to_bf16_bits(x)


def make_modulation(K: int, seed: int, sigma: float = 0.5):
    """bf16 bit patterns of a block's per-channel modulation (scale [K], shift [K]): the block
    applies y = n * (1 + scale) + shift. Both drawn as sigma * N(0,1) from PCG64 seeded with
    [seed, 104729]; with sigma = 0.5 some channels have 1 + scale near zero or negative."""
    rng = np.random.default_rng([seed, 104729])
    scale = rng.standard_normal(K, dtype=np.float32) * np.float32(sigma)
    shift = rng.standard_normal(K, dtype=np.float32) * np.float32(sigma)
    return f32_to_bf16_bits(scale), f32_to_bf16_bits(shift)


def make_qk_norm(seed: int) -> np.ndarray:
    """bf16 bit patterns of the query and key RMS-norm weights [2, 128]: 1 + 0.1 N(0,1), from
    PCG64 seeded with [seed, 130363]."""
    rng = np.random.default_rng([seed, 130363])
    return f32_to_bf16_bits(np.float32(1.0) + rng.standard_normal((2, 128), dtype=np.float32)
                            * np.float32(0.1))


def make_rope(M: int, n_text: int = 512, grid_w: int = 64, axes=(16, 56, 56),
              theta: float = 10000.0):
    """cos and sin [M, 64] float32 of FLUX-style rotary angles. Token m < n_text is a text
    token at position (0, 0, 0); token n_text + j is an image token at (0, j // grid_w,
    j % grid_w). The 64 channel pairs are split over the three position axes (8, 28, 28 pairs);
    pair p of an axis with d channels turns by position * theta^(-2p / d). These are inputs of
    the attention projection (the model computes them from token positions), not part of the
    quantized linear."""
    n_text = min(n_text, M)
    ids = np.zeros((M, 3), dtype=np.float64)
    j = np.arange(M - n_text)
    ids[n_text:, 1] = j // grid_w
    ids[n_text:, 2] = j % grid_w
    ang = []
    for a, d in enumerate(axes):
        omega = theta ** (-np.arange(0, d, 2, dtype=np.float64) / d)
        ang.append(ids[:, a:a + 1] * omega[None, :])
    ang = np.concatenate(ang, axis=1)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


# ---------------------------------------------------------------------------------------------
# Full denoising step: inputs drawn on the device (8.6 GB of weights are too slow to draw on the
# host). torch.Generator on the device, seeded 4_000_000 + 100 * block + 10 * stream + linear.
# ---------------------------------------------------------------------------------------------

def dit_step_plan(wl: Workload):
    """Execution order of the 228 linears of one step: for each of the 19 double-stream blocks,
    the image stream's then the text stream's QKV, proj, fc1, fc2; then for each of the 38
    single-stream blocks, linear1 and linear2. Each entry names its shape and seed."""
    by_name = {l.name: l for l in wl.linears}
    plan = []
    for b in range(19):
        for si, stream in enumerate(("img", "txt")):
            for li, part in enumerate(("qkv", "proj", "fc1", "fc2")):
                plan.append((by_name[f"double.{stream}.{part}"], 100 * b + 10 * si + li, stream))
    for b in range(38):
        for li, part in enumerate(("linear1", "linear2")):
            plan.append((by_name[f"single.{part}"], 100 * (19 + b) + 20 + li, "single"))
    return plan


def dit_step_calls(wl: Workload):
    """The step as launched: for each of the 19 double-stream blocks, its QKV, proj, fc1 and fc2
    each as ONE call over the joint sequence of 512 text rows then 4096 image rows, with the text
    and the image weight as two row segments; then for each of the 38 single-stream blocks,
    linear1 and linear2 over the 4608 rows. Each call lists its segments as (shape, seed offset,
    index in dit_step_plan)."""
    plan = dit_step_plan(wl)
    calls = []
    for b in range(19):
        for li, part in enumerate(("qkv", "proj", "fc1", "fc2")):
            segs = []
            for si, stream in ((1, "txt"), (0, "img")):
                idx = b * 8 + si * 4 + li
                shape, sub, _ = plan[idx]
                assert shape.name == f"double.{stream}.{part}"
                segs.append((shape, sub, idx))
            calls.append({"name": f"double.{part}", "block": b, "segments": segs,
                          "residual": "joint"})
    for b in range(38):
        for li, part in enumerate(("linear1", "linear2")):
            idx = 19 * 8 + 2 * b + li
            shape, sub, _ = plan[idx]
            calls.append({"name": f"single.{part}", "block": b, "segments": [(shape, sub, idx)],
                          "residual": "single"})
    for c in calls:
        first = c["segments"][0][0]
        c.update(M=sum(sh.M for sh, _, _ in c["segments"]), K=first.K, N=first.N,
                 epilogue=first.epilogue, act=f"{sum(sh.M for sh, _, _ in c['segments'])}x{first.K}",
                 flops=sum(sh.flops for sh, _, _ in c["segments"]))
    return calls


def dit_step_device_inputs(wl: Workload, device, quantize_weight, only=None,
                           keep_weights=False):
    """Draw the inputs of one step on `device` and hand each bf16 weight to `quantize_weight`
    (which returns its (codes, scales)); the bf16 weight is dropped afterwards unless
    keep_weights (then it is kept under "w").

    only: None for every call of dit_step_calls(wl), or a set of indices into that list (each
    weight has its own seed, so a subset gets exactly the values the whole step gets).

    Returns (calls, activations, residual_streams). Each call is a dit_step_calls entry whose
    "segments" are dicts with the segment's rows and its qw, sw, bias and gate. Activations are
    one [4608, K] buffer per K (the joint sequence; the single-stream blocks use the same 4608
    rows); the residual streams are the double blocks' joint [4608, 3072] and the single
    blocks' [4608, 3072], both updated in place by the gated linears."""
    import torch
    base = 4_000_000
    calls = dit_step_calls(wl)
    acts, residuals = {}, {}
    g = torch.Generator(device=device)
    for c in calls:
        key = c["act"]
        if key in acts:
            continue
        shape = c["segments"][0][0]
        M, K = c["M"], c["K"]
        g.manual_seed(base + 7 * M + K)
        x = torch.randn((M, K), generator=g, device=device, dtype=torch.float32)
        cols = torch.randperm(K, generator=g, device=device)[: shape.n_outliers]
        x[:, cols] *= shape.outlier_factor
        acts[key] = x.to(torch.bfloat16)
        del x
    for stream in ("joint", "single"):
        g.manual_seed(base + 99 + (1 if stream == "joint" else 2))
        residuals[stream] = torch.randn((4608, 3072), generator=g, device=device,
                                        dtype=torch.float32).to(torch.bfloat16)
    out = []
    for ci, c in enumerate(calls):
        if only is not None and ci not in only:
            continue
        segs = []
        for shape, sub, idx in c["segments"]:
            g.manual_seed(base + sub)
            w = (torch.randn((shape.N, shape.K), generator=g, device=device,
                             dtype=torch.float32) * 0.02).to(torch.bfloat16)
            qw, sw = quantize_weight(w)
            bias = (torch.randn(shape.N, generator=g, device=device) * 0.01).to(torch.bfloat16)
            gate = None
            if shape.epilogue == "gated_residual":
                gate = (1.0 + 0.1 * torch.randn(shape.N, generator=g, device=device)).to(
                    torch.bfloat16)
            seg = {"name": shape.name, "rows": shape.M, "qw": qw, "sw": sw, "bias": bias,
                   "gate": gate, "seed": base + sub, "plan_index": idx}
            if keep_weights:
                seg["w"] = w
            del w
            segs.append(seg)
        entry = dict(c)
        entry["segments"] = segs
        entry["call_index"] = ci
        entry["residual"] = c["residual"] if c["epilogue"] == "gated_residual" else None
        out.append(entry)
    return out, acts, residuals
