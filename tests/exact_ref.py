"""Exact-arithmetic references used to pin the oracle. They share no arithmetic with it.

* `nearest_code_bruteforce`: nearest-value search over all 127 non-negative finite E4M3 values
  (built as exact rationals from the bit fields), ties to the even code, saturating at 448.
* `torch_encode` / `e4m3_values_torch`: the library routines (torch's float8_e4m3fn cast and
  decoder) as a second, independent reference.
* `fraction_to_f32`: correctly rounded (to nearest, ties to even) binary32 of an exact rational,
  by integer arithmetic, with subnormals.
* `bruteforce_linear`: the whole quantize -> contract -> epilogue chain on tiny shapes in exact
  rational arithmetic (the GELU's tanh in float64 math.tanh).
"""
import math
from fractions import Fraction

import numpy as np


def e4m3_values_exact():
    """Fractions for codes 0..126 built digit by digit: bits s.eeee.mmm read as a binary number."""
    vals = []
    for c in range(127):
        e = c >> 3
        m = c & 7
        if e == 0:
            # 0.mmm * 2^-6
            vals.append(Fraction(m, 8) * Fraction(1, 64))
        else:
            # 1.mmm * 2^(e-7)
            vals.append((1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7)))
    return vals


def e4m3_values_torch():
    """float64 values of codes 0..255 as torch's float8_e4m3fn decoder reads them."""
    import torch
    u = torch.arange(256, dtype=torch.uint8)
    return u.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def nearest_code_bruteforce(v):
    """Nearest E4M3 code of each finite float32 value by exhaustive search (ties -> even code).

    Distances are computed in float64. For |v| < 2^-10 the answer is +-0 and any rounding of
    the distances keeps that order. For 2^-10 <= |v| < 448 the difference |v| - t spans at most
    9 + 33 = 42 bits, so it is exact, and ties are detected exactly.
    """
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v.astype(np.float64))
    table = np.array([float(t) for t in e4m3_values_exact()], dtype=np.float64)   # 127 values
    out = np.empty(a.shape, dtype=np.int64)
    flat_a = a.reshape(-1)
    flat_o = out.reshape(-1)
    chunk = 1 << 16
    for s in range(0, flat_a.size, chunk):
        aa = flat_a[s:s + chunk]
        d = np.abs(aa[:, None] - table[None, :])           # [n, 127]
        dmin = d.min(axis=1, keepdims=True)
        ties = d == dmin
        codes = np.arange(127)[None, :]
        # among tied codes take the even one (two neighbours never share parity)
        even = ties & (codes % 2 == 0)
        has_even = even.any(axis=1)
        first = np.argmax(ties, axis=1)
        pick_even = np.argmax(even, axis=1)
        res = np.where(has_even, pick_even, first)
        res = np.where(aa >= 448.0, 0x7E, res)
        flat_o[s:s + chunk] = res
    out = np.where(np.signbit(v), out | 0x80, out)
    return out.astype(np.uint8)


def torch_encode(v):
    """Library routine: torch's RNE float -> float8_e4m3fn cast, after clamping to [-448, 448]
    (the cast alone does not saturate)."""
    import torch
    t = torch.from_numpy(np.asarray(v, dtype=np.float32).copy())
    t = torch.clamp(t, -448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def fraction_to_f32(fr: Fraction) -> float:
    """binary32 nearest to an exact rational (ties to even), returned as a Python float."""
    if fr == 0:
        return 0.0
    neg = fr < 0
    a = -fr if neg else fr
    # e = floor(log2 a)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    scaled = a / ulp
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * ulp
    if val >= Fraction(2) ** 128:
        out = math.inf
    else:
        out = float(val)      # exact: val has <= 24 significant bits
    return -out if neg else out


def nearest_code_fraction(a: Fraction, values):
    """Nearest code of a non-negative exact rational among `values` (codes 0..126), ties to the
    even code, saturating at 448."""
    if a >= 448:
        c = 0x7E
    else:
        best = None
        for c_, t in enumerate(values):
            d = abs(a - t)
            if best is None or d < best[0] or (d == best[0] and c_ % 2 == 0):
                best = (d, c_)
        c = best[1]
    return c


def bruteforce_quantize_row(xrow):
    """Exact-rational per-row quantization of a list of float32 (bf16) values.

    Returns (codes list, scale float). Signed zeros keep their sign bit."""
    values = e4m3_values_exact()
    fx = [Fraction(float(x)) for x in xrow]
    amax = max(abs(f) for f in fx)
    scale = fraction_to_f32(amax / 448)
    codes = []
    for x, f in zip(xrow, fx):
        sign = 0x80 if math.copysign(1.0, float(x)) < 0 else 0
        if scale == 0:
            codes.append(sign)
            continue
        qf = fraction_to_f32(f / Fraction(scale))
        c = nearest_code_fraction(Fraction(abs(qf)), values)
        codes.append(c | sign)
    return codes, scale


def bruteforce_linear(x, w, bias, epilogue, gate=None, residual=None):
    """Exact evaluation of the whole chain on tiny shapes.

    x [M,K], w [N,K], bias [N] (or None), gate [N], residual [M,N]: float32 arrays of bf16 values.
    Returns (q [M,K], sa [M], qw [N,K], sw [N], y float64 [M,N])."""
    values = e4m3_values_exact()
    M, K = x.shape
    N = w.shape[0]
    q, sa = zip(*[bruteforce_quantize_row(r) for r in x])
    qw, sw = zip(*[bruteforce_quantize_row(r) for r in w])

    def dec(c):
        v = values[c & 0x7F]
        return -v if c & 0x80 else v

    y = np.empty((M, N), dtype=np.float64)
    for m in range(M):
        for n in range(N):
            acc = sum((dec(q[m][k]) * dec(qw[n][k]) for k in range(K)), Fraction(0))
            v = acc * Fraction(sa[m]) * Fraction(sw[n])
            if bias is not None:
                v += Fraction(float(bias[n]))
            if epilogue == "bias":
                y[m, n] = float(v)
            elif epilogue == "gelu_tanh":
                vf = float(v)
                y[m, n] = 0.5 * vf * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (vf + 0.044715 * vf ** 3)))
            elif epilogue == "gated_residual":
                y[m, n] = float(Fraction(float(residual[m, n])) + Fraction(float(gate[n])) * v)
            else:
                raise ValueError(epilogue)
    return (np.array(q, dtype=np.uint8), np.array(sa, dtype=np.float32),
            np.array(qw, dtype=np.uint8), np.array(sw, dtype=np.float32), y)
