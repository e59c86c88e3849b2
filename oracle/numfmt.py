"""Number formats used by the path, from their bit-level definitions (fp64).

bf16: 1 sign, 8 exponent (bias 127), 7 stored mantissa bits; the scales of
the int8 card (model table, row "Weights": one bf16 scale per row and 128 of
K) and of the FP8 card (one bf16 scale per 128x128 block), and the rotated
activations.

f16 (IEEE binary16): 1 sign, 5 exponent (bias 15), 10 stored mantissa bits;
the scales of the DFlash drafter's int8 linears on the int8 card (model
table, row "Speculator": an f16 scale per row and 128 of K).

E4M3: the FP8 card's weight codes (model table, row "Weights": FP8 E4M3).
Read as the OCP "E4M3FN" flavour: 1 sign, 4 exponent (bias 7), 3 mantissa
bits, no infinities, S.1111.111 is NaN, largest finite 448.

Rounding is done once, from the fp64 value, to the nearest representable
value with ties to the even significand. Nothing here goes through float32
or a library cast; the tests compare against library casts separately.
"""

import numpy as np

BF16_MANT_BITS = 7          # stored bits; 8 significant bits with the hidden one
BF16_EMIN = -126            # exponent of the smallest normal
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127

F16_MANT_BITS = 10
F16_EMIN = -14
F16_MAX = 65504.0           # (2 - 2**-10) * 2**15

E4M3_MAX = 448.0            # 1.75 * 2**8
E4M3_EMIN = -6              # exponent of the smallest normal (bias 7)


def _round_to_quantum(x, emin, mbits):
    """Round fp64 x to a binary format with `mbits` stored mantissa bits and
    smallest normal exponent `emin` (ignoring overflow), ties to even.

    For |x| in [2**e, 2**(e+1)) the spacing is 2**(e - mbits); below the
    normal range it stays 2**(emin - mbits) (subnormals).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = x != 0
    # np.frexp gives x = m * 2**ex with 0.5 <= |m| < 1, so floor(log2|x|) = ex - 1
    _, ex = np.frexp(x[nz])
    e = np.maximum(ex - 1, emin)
    q = np.ldexp(1.0, e - mbits)
    # x / q and (...) * q are exact: q is a power of two in range
    out[nz] = np.rint(x[nz] / q) * q
    # keep the sign of x on results that round to zero
    out = np.where(out == 0, np.copysign(0.0, x), out)
    return out


def bf16_round(x):
    """Nearest bf16 value of fp64 x (ties to even), as fp64; overflow -> inf."""
    r = _round_to_quantum(x, BF16_EMIN, BF16_MANT_BITS)
    # a value rounds to infinity when it reaches max + half an ulp (2**119)
    big = np.abs(r) > BF16_MAX
    return np.where(big, np.copysign(np.inf, r), r)


def bf16_to_bits(v):
    """uint16 bit pattern of bf16-representable fp64 values."""
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (v32.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(b):
    """fp64 value of bf16 bit patterns (uint16)."""
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f16_round(x):
    """Nearest binary16 value of fp64 x (ties to even), as fp64; values that
    reach max + half an ulp (65520) become inf."""
    r = _round_to_quantum(x, F16_EMIN, F16_MANT_BITS)
    big = np.abs(r) > F16_MAX
    return np.where(big, np.copysign(np.inf, r), r)


def f16_to_bits(v):
    """uint16 bit pattern of binary16-representable fp64 values, from the
    fields: sign, biased exponent (0 for subnormals), 10 mantissa bits."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.int64) << 15
    a = np.abs(v)
    bits = np.zeros(a.shape, dtype=np.int64)
    inf = np.isinf(a)
    bits[inf] = 0x1F << 10
    nz = (a > 0) & ~inf
    m, ex = np.frexp(a[nz])             # a = m * 2**ex, 0.5 <= m < 1
    e = ex - 1
    normal = e >= F16_EMIN
    ef = np.where(normal, e + 15, 0)
    mf = np.where(normal, np.rint((2.0 * m - 1.0) * 1024.0), np.rint(a[nz] / 2.0 ** (F16_EMIN - 10)))
    bits[nz] = (ef << 10) | mf.astype(np.int64)
    return (bits | sign).astype(np.uint16)


def f16_from_bits(b):
    """fp64 value of binary16 bit patterns (finite or inf; no NaN handling)."""
    c = np.asarray(b, dtype=np.uint16).astype(np.int64)
    sign = np.where(c & 0x8000, -1.0, 1.0)
    ef = (c >> 10) & 0x1F
    mf = c & 0x3FF
    val = np.where(ef == 0, np.ldexp(mf / 1024.0, F16_EMIN), np.ldexp(1.0 + mf / 1024.0, ef - 15))
    return sign * np.where(ef == 0x1F, np.inf, val)


def e4m3_decode(codes):
    """fp64 value of each E4M3FN byte (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mf = c & 0x7
    normal = sign * np.ldexp(1.0 + mf / 8.0, ef - 7)
    sub = sign * np.ldexp(mf / 8.0, E4M3_EMIN)
    val = np.where(ef == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e4m3_round_sat(x):
    """Nearest E4M3FN value of fp64 x, ties to even, magnitudes beyond 448
    clamped to 448 (saturation); returned as fp64. x must be finite."""
    x = np.asarray(x, dtype=np.float64)
    r = _round_to_quantum(x, E4M3_EMIN, 3)
    return np.where(np.abs(r) > E4M3_MAX, np.copysign(E4M3_MAX, x), r)


def e4m3_encode_sat(x):
    """E4M3FN byte of fp64 x: round to nearest even with saturation at 448.

    The sign bit is the sign of x, also when the value rounds to zero.
    """
    r = e4m3_round_sat(x)
    sign = np.signbit(r).astype(np.int64) << 7
    a = np.abs(r)
    code = np.zeros(a.shape, dtype=np.int64)
    nz = a > 0
    m, ex = np.frexp(a[nz])            # a = m * 2**ex, 0.5 <= m < 1
    e = ex - 1                          # a = (2m) * 2**e, 1 <= 2m < 2
    is_normal = e >= E4M3_EMIN
    # normal: fields (e + 7, (2m - 1) * 8); subnormal: (0, a / 2**-9)
    ef = np.where(is_normal, e + 7, 0)
    mf = np.where(is_normal, np.rint((2.0 * m - 1.0) * 8.0),
                  np.rint(a[nz] / 2.0 ** (E4M3_EMIN - 3)))
    code[nz] = (ef << 3) | mf.astype(np.int64)
    return (code | sign).astype(np.uint8)
