"""Number formats of the prologue, written from their public definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* bf16: the upper 16 bits of an IEEE binary32, rounded to nearest, ties to even.
* E4M3 (OCP OFP8 "E4M3FN", the FP8 type whose largest finite value is 448):
  1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
  holds subnormals m * 2^-9; S.1111.111 is NaN and there are no infinities.
  The prologue rounds to nearest even and saturates at +-448 (the pre_attn page's
  module docstring and ``norm_quant``: FP8 with scale amax / FP8_MAX).
* E8M0 (OCP MX scale): code c means 2^(c - 127); c = 255 is NaN.
* E2M1 (OCP MX FP4, the element type of NVFP4): 1 sign bit (0x8), 2 exponent
  bits with bias 1, 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6, no
  NaN or infinity. Rounded to nearest even and saturated at +-6 (the epilogue
  page's NVFP4 quantizer converts with satfinite).
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_SUBNORMAL_STEP = 2.0**-9
_MIN_NORMAL = 2.0**-6


def e4m3_decode_table() -> np.ndarray:
    """Value of each of the 256 E4M3 codes (float64; NaN for 0x7F / 0xFF)."""
    tab = np.empty(256, np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            tab[c] = np.nan
        elif e == 0:
            tab[c] = sign * m * _SUBNORMAL_STEP
        else:
            tab[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return tab


_TABLE = e4m3_decode_table()


def e4m3_decode(codes) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v) -> np.ndarray:
    """Round float64 values to E4M3 codes: saturate to 448, nearest, ties to even.

    The sign is kept, so -0.0 and tiny negatives give 0x80. Each binade
    [2^E, 2^(E+1)) (E >= -6) holds 8 codes spaced 2^(E-3); below 2^-6 the grid is
    the subnormal step 2^-9. Scaling by a power of two is exact, so np.rint (ties
    to even) on the scaled magnitude is the exact round-to-nearest-even, and the
    code is the grid index counted from zero.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("NaN has no saturating E4M3 encoding")
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)
    code = np.empty(a.shape, dtype=np.int64)
    sub = a < _MIN_NORMAL
    code[sub] = np.rint(a[sub] / _SUBNORMAL_STEP).astype(np.int64)
    an = a[~sub]
    _, ex = np.frexp(an)  # an = f * 2^ex with f in [0.5, 1)
    e = ex.astype(np.int64) - 1  # floor(log2(an)), in [-6, 8]
    m = np.rint(np.ldexp(an, (3 - e).astype(np.int32))).astype(np.int64)  # in [8, 16]
    code[~sub] = (e + 6) * 8 + m
    return (code | (neg.astype(np.int64) << 7)).astype(np.uint8)


def f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16) & 0xFFFF
    nan = np.isnan(x)
    r[nan] = ((b[nan] >> 16) | 0x40) & 0xFFFF
    return r.astype(np.uint16)


def bf16_bits_to_f32(u) -> np.ndarray:
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(u) -> np.ndarray:
    return bf16_bits_to_f32(u).astype(np.float64)


def e8m0_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    out = np.ldexp(1.0, (c - 127).astype(np.int32))
    return np.where(c == 255, np.nan, out)


E2M1_MAX = 6.0


def e2m1_decode(codes) -> np.ndarray:
    """Value of each 4-bit E2M1 code (float64)."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.ldexp(1.0, (e - 1).astype(np.int32)))
    return np.where(c & 0x8, -mag, mag)


def e2m1_encode(v) -> np.ndarray:
    """Round float64 values to E2M1 codes: saturate to 6, nearest, ties to even.

    Below 1 (exponent field 0) the grid is the subnormal step 0.5; the binade
    [2^E, 2^(E+1)) for E = 0, 1, 2 holds 2 codes spaced 2^(E-1). As for E4M3,
    np.rint on the magnitude scaled to its grid step is the exact
    nearest-even rounding. The sign is kept (-0 -> 0x8).
    """
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("NaN has no saturating E2M1 encoding")
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), E2M1_MAX)
    code = np.empty(a.shape, dtype=np.int64)
    sub = a < 1.0
    code[sub] = np.rint(a[sub] / 0.5).astype(np.int64)  # 0, 1 or 2 (2 = 1.0)
    an = a[~sub]
    _, ex = np.frexp(an)
    e = ex.astype(np.int64) - 1  # floor(log2(an)) in [0, 2]
    m = np.rint(np.ldexp(an, (1 - e).astype(np.int32))).astype(np.int64)  # in [2, 4]
    code[~sub] = e * 2 + m
    return (code | (neg.astype(np.int64) << 3)).astype(np.uint8)


def f32_mul_rz(a, b) -> np.ndarray:
    """float32 product a * b rounded toward zero (a, b float32).

    The product of two float32 values is exact in float64 (48 significant bits
    at most); its round-to-nearest float32 image is one of the two float32
    neighbours, and stepping it one ulp toward zero where it landed farther
    from zero than the exact value gives the truncated one."""
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    p = a.astype(np.float64) * b.astype(np.float64)
    r = p.astype(np.float32)
    over = np.abs(r.astype(np.float64)) > np.abs(p)
    r = np.where(over, np.nextafter(r, np.float32(0.0)), r)
    return r.astype(np.float32)
