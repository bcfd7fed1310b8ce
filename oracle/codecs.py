"""Number-format codecs of the oracle (test infrastructure only).

bf16: the upper 16 bits of an IEEE binary32 word (8 exponent bits, 7 stored
mantissa bits).  Decoding is exact; encoding rounds to nearest, ties to even.

e4m3: the OCP 8-bit float "E4M3FN" the DeepSeek V4-Flash architecture Q&A
names for forward activations and weights (Q7.2: 4 exponent bits, 3 mantissa
bits, range +-448).  Exponent bias 7, subnormals below 2^-6 in steps of 2^-9,
no infinities, S.1111.111 is NaN, so the largest finite magnitude is
1.75 * 2^8 = 448.  Encoding rounds to nearest, ties to even, and saturates
finite values beyond 448 to +-448.

Both are written from the format definitions; ``tests/test_oracle_codecs.py``
checks them against torch's CPU casts, an independent implementation.
"""

import numpy as np

E4M3_MAX = 448.0
_E4M3_MIN_NORMAL_EXP = -6      # 2^-6 is the smallest normal
_E4M3_SUBNORMAL_STEP = 2.0 ** -9


def bf16_bits_to_f64(bits):
    """uint16 bf16 bit patterns -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_to_bf16(a):
    """float64 values -> the nearest bf16 values (ties to even), as float64.

    One rounding straight from float64 (no float32 step): keep the top 8
    significant bits of the binary64 pattern.  Valid for finite values in
    bf16's normal range, which is all the layer produces."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    u = a.view(np.uint64)
    drop = np.uint64(45)                          # 52 - 7 stored mantissa bits
    lsb = (u >> drop) & np.uint64(1)
    r = (u + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    return r.view(np.float64)


def f32_to_bf16_bits(x):
    """float32 values -> uint16 bf16 bit patterns, round to nearest even.

    NaN maps to the quiet NaN 0x7FC0 (keeping the sign bit)."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    if np.any(nan):
        sign = ((u >> np.uint64(16)) & np.uint64(0x8000)).astype(np.uint16)
        rounded = np.where(nan, sign | np.uint16(0x7FC0), rounded)
    return rounded.astype(np.uint16)


def _e4m3_table():
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * m * _E4M3_SUBNORMAL_STEP
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3_VALUES = _e4m3_table()


def e4m3_bits_to_f64(bits):
    """uint8 e4m3 codes -> float64 values (exact)."""
    return _E4M3_VALUES[np.asarray(bits, dtype=np.uint8)]


def f32_to_e4m3_bits(x):
    """float32 values -> uint8 e4m3 codes: nearest, ties to even, saturating.

    NaN input maps to 0x7F (sign kept).  Works in float64, where every step
    below is exact for float32 input."""
    f = np.asarray(x, dtype=np.float32).astype(np.float64)
    sign = np.where(np.signbit(f), 0x80, 0x00).astype(np.int64)
    a = np.abs(f)
    a_safe = np.where(np.isfinite(a), a, 0.0)
    # subnormal range (a < 2^-6): value = m * 2^-9 with m in 0..8 (m = 8 is code 0x08,
    # the smallest normal, so the code is m itself); np.round rounds ties to even
    sub_code = np.round(a_safe / _E4M3_SUBNORMAL_STEP).astype(np.int64)
    # normal range: a = (1 + frac) * 2^e, frac quantised to eighths
    _, ex = np.frexp(np.where(a_safe > 0, a_safe, 1.0))
    e = ex.astype(np.int64) - 1
    mant = np.round((a_safe / np.ldexp(1.0, e) - 1.0) * 8.0).astype(np.int64)
    carry = mant == 8
    e = e + carry
    mant = np.where(carry, 0, mant)
    norm_code = ((e + 7) << 3) | mant
    code = np.where(a_safe < 2.0 ** _E4M3_MIN_NORMAL_EXP, sub_code, norm_code)
    code = np.where(a >= E4M3_MAX, 0x7E, np.minimum(code, 0x7E))   # 448 = S.1111.110
    code = np.where(np.isnan(f), 0x7F, code)
    return (sign | code).astype(np.uint8)
