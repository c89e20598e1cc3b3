"""Element formats of the compressed weights, decoded and encoded from their bit layouts.

ORACLE -- test infrastructure only.  Nothing in the library imports this module;
only the tests, the smoke check and the CPU-baseline leg of the benchmark do.

The pages describe the weights as NVFP4 ("block 4-bit floating point made for
NVIDIA tensor cores", ai-manual article, section "NVFP4 model conversion";
"NVFP4 was built for Blackwell", the author's post, opening) and as published FP8
regions that stay FP8 (author's post, section "v1.0 -> v1.1").  They do not give
the bit layouts.  The layouts below are the public OCP Microscaling (MX) v1.0
element encodings that NVFP4 and FP8 use:

  E2M1  (4 bits: s e1 e0 m, exponent bias 1, no inf/NaN)
        e == 0 : (-1)^s * m * 0.5                 (0 or the subnormal 0.5)
        e >  0 : (-1)^s * 2^(e-1) * (1 + m/2)
  E4M3FN (8 bits: s eeee mmm, exponent bias 7, no inf, NaN = s.1111.111)
        e == 0 : (-1)^s * m * 2^-9               (subnormals)
        e == 15 and m == 7 : NaN
        else   : (-1)^s * 2^(e-7) * (1 + m/8)

Encoders round to nearest with ties to the even code and saturate finite
overflow to the largest finite magnitude (6 for E2M1, 448 for E4M3FN).  They
keep the sign of zero.  All arithmetic here is float64.
"""

import numpy as np

E2M1_MAX = 6.0
E4M3_MAX = 448.0


def _e2m1_from_bits(c):
    """E2M1 value of each 4-bit code in the int64 array c, from the bit fields."""
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(s == 1, -mag, mag)


def _e4m3_from_bits(c):
    """E4M3FN value of each 8-bit code in the int64 array c, from the bit fields (NaN at s.1111.111)."""
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    normal = np.ldexp(1.0 + m / 8.0, e - 7)
    sub = m * 2.0 ** -9
    mag = np.where(e == 0, sub, normal)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


# Each format has only 16 / 256 codes: decode every code once from its bits
# and look large arrays up in that list (same values, far less work per weight).
_E2M1_VALUES = _e2m1_from_bits(np.arange(16, dtype=np.int64))
_E4M3_VALUES = _e4m3_from_bits(np.arange(256, dtype=np.int64))


def e2m1_decode(codes):
    """4-bit codes (values 0..15, any integer dtype) -> float64 values."""
    return np.take(_E2M1_VALUES, np.asarray(codes).astype(np.uint8, copy=False) & np.uint8(15))


def e4m3_decode(codes):
    """8-bit E4M3FN codes (values 0..255) -> float64 values (NaN for 0x7F/0xFF)."""
    return np.take(_E4M3_VALUES, np.asarray(codes).astype(np.uint8, copy=False))


def _round_half_even_to_grid(a, exp_floor, mant_bits, max_val):
    """Round |values| `a` (float64, >= 0) to a binary float grid.

    The grid has `mant_bits` fraction bits, exponents down to `exp_floor`
    (below it the spacing stays 2^(exp_floor - mant_bits): subnormals) and is
    clipped at `max_val`.  Returns the rounded magnitudes (float64).
    np.rint rounds halves to even, which on this grid means the even code.
    """
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        _, ex = np.frexp(a)          # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, exp_floor)  # unbiased exponent of the leading bit
    quantum = np.ldexp(1.0, e - mant_bits)
    r = np.rint(a / quantum) * quantum
    return np.minimum(r, max_val)


def e2m1_encode(values):
    """float64 values -> E2M1 codes (uint8 0..15), RNE, saturating, sign of zero kept."""
    v = np.asarray(values, dtype=np.float64)
    sign = np.signbit(v)
    mag = _round_half_even_to_grid(np.abs(v), exp_floor=0, mant_bits=1, max_val=E2M1_MAX)
    # magnitude -> code: subnormal/zero region uses 0.5 steps, else exponent/mantissa
    _, ex = np.frexp(mag)
    e_unb = ex - 1
    is_norm = mag >= 1.0
    e_field = np.where(is_norm, e_unb + 1, 0)
    m_field = np.where(is_norm, np.rint((mag / np.ldexp(1.0, e_unb) - 1.0) * 2.0), np.rint(mag * 2.0))
    code = (e_field.astype(np.int64) << 1) | m_field.astype(np.int64)
    return (code | (sign.astype(np.int64) << 3)).astype(np.uint8)


def e4m3_encode(values):
    """float64 values -> E4M3FN codes (uint8), RNE, saturating to +-448, sign of zero kept.

    NaN inputs are not accepted (the quantizers never produce them)."""
    v = np.asarray(values, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("e4m3_encode: NaN input")
    sign = np.signbit(v)
    mag = _round_half_even_to_grid(np.abs(v), exp_floor=-6, mant_bits=3, max_val=E4M3_MAX)
    _, ex = np.frexp(mag)
    e_unb = ex - 1
    is_norm = mag >= 2.0 ** -6
    e_field = np.where(is_norm, e_unb + 7, 0)
    m_field = np.where(is_norm, np.rint((mag / np.ldexp(1.0, e_unb) - 1.0) * 8.0), np.rint(mag * 2.0 ** 9))
    code = (e_field.astype(np.int64) << 3) | m_field.astype(np.int64)
    return (code | (sign.astype(np.int64) << 7)).astype(np.uint8)
