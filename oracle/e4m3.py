"""OCP E4M3FN codec, written out from the format's definition.

The pages fix the format as E4M3 for every FP8 tensor, forward and backward
(infra answer, FP8 paragraph; V3 notes §6).  The variant taken is OCP
E4M3FN: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
infinities, a single NaN pattern per sign (exponent 15, mantissa 7), largest
finite magnitude 448.  This is the variant whose 448 maximum the amax/448
scale rule is built around.

Encoding rounds to nearest with ties to the even code and saturates at
+-448; the sign of zero is kept (-0.0 encodes as 0x80).  All arithmetic
below is exact in float64 because the input is a float32 value.
"""

import math

import numpy as np

MAX_FINITE = 448.0
MIN_NORMAL = 2.0 ** -6
SUBNORMAL_STEP = 2.0 ** -9
NAN_CODES = (0x7F, 0xFF)


def decode_scalar(code: int) -> float:
    """Value of one E4M3FN byte (NaN for 0x7F / 0xFF)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * m * SUBNORMAL_STEP
    return sign * (2.0 ** (e - 7)) * (1.0 + m / 8.0)


def encode_scalar(v: float) -> int:
    """E4M3FN code of one finite float32 value (round half to even, saturate).

    Python's built-in round() on a float rounds half to even, exactly.
    """
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0x00
    a = abs(float(v))
    if a >= MAX_FINITE:
        return sign | 0x7E
    if a < MIN_NORMAL:
        # subnormal range: multiples of 2^-9; n == 8 lands on the smallest
        # normal (code 0x08), which is the correct rounding
        n = round(a / SUBNORMAL_STEP)
        return sign | n
    mant, ex = math.frexp(a)          # a = mant * 2^ex, mant in [0.5, 1)
    e = ex - 1                        # a = (2*mant) * 2^e, 2*mant in [1, 2)
    n = round((a / 2.0 ** e - 1.0) * 8.0)
    if n == 8:
        e += 1
        n = 0
    return sign | ((e + 7) << 3) | n


# Table of all 256 decoded values, used by the vectorised decoder.
_DECODE_TABLE = np.array([decode_scalar(c) for c in range(256)], dtype=np.float64)


def decode(codes: np.ndarray) -> np.ndarray:
    """Vectorised decode of uint8 codes to float64."""
    return _DECODE_TABLE[np.asarray(codes, dtype=np.uint8)]


_CHUNK = 1 << 16     # elements per pass (keeps the temporaries in cache)


def encode(values: np.ndarray) -> np.ndarray:
    """Vectorised encode of float32 values to uint8 codes.

    Same steps as encode_scalar, on whole arrays; np.rint rounds half to even.
    The elements are taken in slices of _CHUNK (each element independently,
    so the slicing changes no code; it only keeps the temporaries small).
    """
    v = np.asarray(values, dtype=np.float32)
    flat = v.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    for i in range(0, flat.size, _CHUNK):
        out[i:i + _CHUNK] = _encode_slice(flat[i:i + _CHUNK])
    return out.reshape(v.shape)


def _encode_slice(values: np.ndarray) -> np.ndarray:
    v = np.asarray(values, dtype=np.float32).astype(np.float64)
    sign = np.where(np.signbit(v), 0x80, 0x00).astype(np.int64)
    a = np.abs(v)
    out = np.zeros(a.shape, dtype=np.int64)

    sat = a >= MAX_FINITE
    sub = a < MIN_NORMAL
    nor = ~(sat | sub)

    out[sat] = 0x7E
    out[sub] = np.rint(a[sub] / SUBNORMAL_STEP).astype(np.int64)

    an = a[nor]
    _, ex = np.frexp(an)
    e = ex.astype(np.int64) - 1
    n = np.rint((an / np.ldexp(1.0, e) - 1.0) * 8.0).astype(np.int64)
    carry = n == 8
    e = e + carry
    n = np.where(carry, 0, n)
    out[nor] = ((e + 7) << 3) | n

    return (out | sign).astype(np.uint8)
