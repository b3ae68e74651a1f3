"""Helpers shared by the GPU parity tests: host <-> device copies and the output tolerance."""
import sys

import numpy as np
import torch

DEV = "cuda:0"


def announce(msg: str) -> None:
    """Print what the next GPU step is about to run, before it runs."""
    print(f"\n[gpu] {msg}", flush=True)
    sys.stdout.flush()


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("these tests need a GPU (run them with -m gpu on an MI355X)")


def bf16_to_dev(u16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).to(DEV)


def u8_to_dev(u8: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(u8, dtype=np.uint8)).to(DEV)


def f32_to_dev(f: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(f, dtype=np.float32)).to(DEV)


def dev_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def dev_to_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_within_tolerance(out: np.ndarray, ref: np.ndarray, rms: float = None, what: str = ""):
    """|out - ref| <= 4e-3 |ref| + 1e-3 rms(ref), elementwise.

    `ref` is the oracle's value before bf16 rounding; rms is over the whole output tensor (or
    over the sampled rows when only a sample is compared, which estimates it).
    """
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert out.shape == ref.shape
    assert np.all(np.isfinite(out)), f"{what}: non-finite outputs"
    if rms is None:
        rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(out - ref)
    bound = 4e-3 * np.abs(ref) + 1e-3 * rms
    bad = err > bound
    if bad.any():
        idx = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst at {idx}: "
            f"out={out[idx]!r} ref={ref[idx]!r} err={err[idx]:.3g} bound={bound[idx]:.3g} "
            f"rms={rms:.4g}")
    return float(np.max(err / np.maximum(bound, 1e-300)))
