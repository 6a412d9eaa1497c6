"""Exact element decoders and the fp8 encoder used by the oracle.

The pages name 8-bit KV storage ("PagedAttention deep dive" §3.2 and §4;
"KV-Cache evolution" §3C) without fixing a format. The reading taken here is
OCP E4M3FN: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
infinities, and S.1111.111 as the only NaN pattern. Its largest finite
magnitude is 1.75 * 2^8 = 448; its smallest subnormal is 2^-9.

Encoding rounds to nearest, ties to even, and saturates finite values whose
rounded magnitude would exceed 448 to +-448. NaN maps to 0x7F (0xFF when the
sign bit is set).
"""

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact).

    A bfloat16 is the upper half of a binary32, so shifting its 16 bits into
    the high half of a 32-bit word gives the same value as a float32.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _e4m3fn_value(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3FN codes -> float64 (exact), written from the format's fields."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1 == 1, -1.0, 1.0)
    exp_field = (c >> 3) & 0xF
    man_field = c & 0x7
    normal = sign * np.ldexp(1.0 + man_field / 8.0, exp_field - 7)
    subnormal = sign * np.ldexp(man_field / 8.0, -6)
    out = np.where(exp_field == 0, subnormal, normal)
    out = np.where((exp_field == 0xF) & (man_field == 0x7), np.nan, out)
    return out.astype(np.float64)


# the value of every one of the 256 codes, from the field formula above
_E4M3FN_VALUES = _e4m3fn_value(np.arange(256))


def e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3FN codes -> float64 (exact): each code's value by the format's
    field formula (``_e4m3fn_value``), looked up per code."""
    return _E4M3FN_VALUES[np.asarray(codes, dtype=np.uint8)]


E4M3FN_MAX = 448.0
_E4M3FN_MAX_CODE = 0x7E  # exponent field 15, mantissa 6


def e4m3fn_encode(x: np.ndarray) -> np.ndarray:
    """float32 values -> OCP E4M3FN codes: round to nearest even, saturate.

    The value is split into the binade it falls in; within a binade the
    representable values are evenly spaced (spacing 2^(e-3) for normal binades,
    2^-9 below the smallest normal 2^-6), so the rounded mantissa is the
    round-half-even of |x| / spacing. Every division by a power of two and the
    ``rint`` are exact in float64, so no double rounding occurs.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    out = np.zeros(x.shape, dtype=np.uint8)
    flat_x = x.reshape(-1)
    flat_o = out.reshape(-1)
    sign_bit = np.signbit(flat_x).astype(np.uint8) << np.uint8(7)
    a = np.abs(flat_x)
    nan = np.isnan(a)
    # Everything at or above 448 saturates to 448 (values in [448, 464] also
    # round to 448 under ties-to-even), so clamp first; this also keeps
    # infinities out of the arithmetic below.
    a = np.where(nan, 0.0, np.minimum(a, E4M3FN_MAX))

    # Subnormal binade: multiples of 2^-9 below 2^-6. A rounded count of 8
    # spills into the smallest normal, whose code (exponent 1, mantissa 0) is
    # also 8, so the count is the code itself.
    sub = a < 2.0 ** -6
    sub_code = np.rint(a / 2.0 ** -9).astype(np.int64)

    # Normal binades: a = f * 2^e with f in [0.5, 1) from frexp, so the
    # unbiased exponent of the leading one is e - 1.
    _, e = np.frexp(np.where(sub, 1.0, a))
    e_unb = e.astype(np.int64) - 1
    spacing = np.ldexp(1.0, e_unb - 3)
    q = np.rint(np.where(sub, 8.0, a) / spacing).astype(np.int64)  # in [8, 16]
    carry = q == 16
    e_unb = np.where(carry, e_unb + 1, e_unb)
    q = np.where(carry, 8, q)
    norm_code = ((e_unb + 7) << 3) | (q - 8)

    code = np.where(sub, sub_code, norm_code)
    assert code.size == 0 or code.max() <= _E4M3FN_MAX_CODE
    code = np.where(nan, 0x7F, code)
    flat_o[:] = code.astype(np.uint8) | sign_bit
    return out


INT8_MAX = 127


def int8_encode(x: np.ndarray) -> np.ndarray:
    """float32 values -> symmetric int8 codes: round to nearest, ties to even,
    saturating to [-127, 127]; NaN -> 0.

    The pages name INT8 KV storage beside FP8 ("PagedAttention deep dive" §4;
    "KV-Cache evolution" §3C) without a scheme. The reading taken: symmetric
    codes, the value of code c being c times the tensor's scale, -128 never
    produced (so negation is exact).
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    nan = np.isnan(x)
    q = np.clip(np.rint(np.where(nan, 0.0, x)), -INT8_MAX, INT8_MAX)
    return q.astype(np.int8)


def int8_decode(codes: np.ndarray) -> np.ndarray:
    """int8 codes -> float64 (exact): the code itself, to be scaled."""
    return np.asarray(codes, dtype=np.int8).astype(np.float64)


def to_f64(a: np.ndarray) -> np.ndarray:
    """Widen a stored array to float64 using the dtype convention of the package.

    float32 / float16 widen exactly through numpy; uint16 is bfloat16 bits;
    uint8 is E4M3FN codes; int8 is symmetric int8 codes.
    """
    a = np.asarray(a)
    if a.dtype == np.float64:
        return a
    if a.dtype in (np.float32, np.float16):
        return a.astype(np.float64)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    if a.dtype == np.uint8:
        return e4m3fn_decode(a)
    if a.dtype == np.int8:
        return int8_decode(a)
    raise TypeError(f"no stored-element convention for numpy dtype {a.dtype}")


def to_f32_exact(a: np.ndarray) -> np.ndarray:
    """Widen a 16-bit or 32-bit stored array to float32 (exact for all three)."""
    a = np.asarray(a)
    if a.dtype == np.float32:
        return a
    if a.dtype == np.float16:
        return a.astype(np.float32)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise TypeError(f"cannot widen numpy dtype {a.dtype} to float32 exactly")
