"""OCP FP8 E4M3 codes: value of each byte, and the round-to-nearest-even saturating encoder.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages ask for FP8 weights and activations (page "Solucion de WaveSpeed para Acelerar la
Generacion de Imagenes FLUX.1-dev", section "Cuantizacion Dinamica FP8") without naming the
flavour. The reading taken is OCP E4M3: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
bits, no infinities, NaN only as S.1111.111, subnormals below 2^-6 on a 2^-9 grid, largest
finite value 1.75 * 2^8 = 448.
"""
import numpy as np

E4M3_MAX = 448.0


def decode_table() -> np.ndarray:
    """float64[256]: the value of every E4M3 byte (NaN for 0x7F and 0xFF, -0.0 for 0x80).

    A byte c has sign s = c >> 7, exponent field e = (c >> 3) & 15, mantissa m = c & 7.
    e == 0 encodes the subnormal value m * 2^-9; otherwise the value is (1 + m/8) * 2^(e-7).
    """
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            t[c] = np.nan
        elif e == 0:
            t[c] = sign * m * 2.0 ** -9
        else:
            t[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


def encode_e4m3(v) -> np.ndarray:
    """Nearest E4M3 byte of each finite float32 value; ties go to the even code; |v| >= 448 -> 448.

    The work is done in float64, where every step below is exact: |v| is a float32, and scaling
    by a power of two neither overflows nor underflows in this range.

      * |v| >= 448: the code of 448 (values in [448, 464) round there anyway; anything larger
        would round past the largest finite value, and saturation keeps it at 448).
      * |v| < 2^-6: the grid is the subnormal one, spacing 2^-9; the rounded multiple
        r = rint(|v| * 2^9) in 0..8 is the code itself (r == 8 is the smallest normal, 0x08).
      * otherwise, with e = floor(log2 |v|) in -6..8, the grid spacing is 2^(e-3);
        r = rint(|v| * 2^(3-e)) lies in 8..16; r == 16 carries into the next binade.
        The code is ((e + 7) << 3) | (r - 8).
    rint rounds halves to even, and the code's last bit is r's last bit, so a tie goes to the
    even code. The sign bit is copied, so negative values that round to zero give 0x80.
    """
    v = np.asarray(v, dtype=np.float32)
    if not np.all(np.isfinite(v)):
        raise ValueError("encode_e4m3: inputs must be finite")
    neg = np.signbit(v)
    a = np.abs(v.astype(np.float64))

    code = np.zeros(a.shape, dtype=np.int64)

    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)

    nrm = (~sub) & (a < E4M3_MAX)
    an = a[nrm]
    _, ex = np.frexp(an)            # an = f * 2^ex with f in [0.5, 1)
    e = ex.astype(np.int64) - 1     # floor(log2 an)
    r = np.rint(np.ldexp(an, 3 - e)).astype(np.int64)
    carry = r == 16
    e = np.where(carry, e + 1, e)
    r = np.where(carry, 8, r)
    code[nrm] = ((e + 7) << 3) | (r - 8)

    code[a >= E4M3_MAX] = 0x7E
    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8)
