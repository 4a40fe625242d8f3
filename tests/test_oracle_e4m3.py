"""Pins of the oracle's E4M3FN codec against hand-worked codes and brute force.

The brute force knows nothing of exponents or mantissa fields: it decodes all
127 non-negative finite codes, picks the magnitude nearest to |v| (ties to the
even code), and restores the sign.  Rounding to nearest even with saturation
at 448 is exactly that rule on finite inputs.
"""

import numpy as np
import pytest

from oracle import e4m3


def _brute_force(values: np.ndarray) -> np.ndarray:
    mags = np.array([e4m3.decode_scalar(c) for c in range(127)], dtype=np.float64)
    v = values.astype(np.float64)
    # beyond the largest magnitude the distance order does not depend on |v|,
    # so clipping keeps the float64 distances exact without changing the answer
    a = np.minimum(np.abs(v), 1024.0)
    out = np.empty(v.shape, dtype=np.uint8)
    step = 1 << 15
    for i in range(0, v.size, step):
        ai = a[i:i + step]
        dist = np.abs(ai[:, None] - mags[None, :])
        dmin = dist.min(axis=1, keepdims=True)
        is_min = dist == dmin
        first = np.argmax(is_min, axis=1)
        n_min = is_min.sum(axis=1)
        # a tie is always between two neighbouring codes: take the even one
        code = np.where((n_min > 1) & (first % 2 == 1), first + 1, first)
        out[i:i + step] = code
    return out | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)


def _probe_values(seed=0):
    """Every (sign, exponent, top-7-mantissa) float32 pattern, each with
    several low-16-bit patterns (exact midpoints, just above/below, random)."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    r = np.random.default_rng(seed)
    lows = [0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF]
    parts = [hi | np.uint32(lo) for lo in lows]
    parts.append(hi | r.integers(0, 1 << 16, size=hi.size, dtype=np.uint32))
    bits = np.concatenate(parts)
    vals = bits.view(np.float32)
    return vals[np.isfinite(vals)]


def test_golden_codes(golden):
    g = golden("e4m3_codes.json")
    for case in g["cases"]:
        v = np.float32(float(case["value"]))
        want = int(case["code"], 16)
        assert e4m3.encode_scalar(float(v)) == want, case
        assert int(e4m3.encode(np.array([v]))[0]) == want, case


def test_decode_encode_identity_on_all_finite_codes():
    for c in range(256):
        if c in e4m3.NAN_CODES:
            assert np.isnan(e4m3.decode_scalar(c))
            continue
        v = e4m3.decode_scalar(c)
        assert e4m3.encode_scalar(v) == c
    codes = np.array([c for c in range(256) if c not in e4m3.NAN_CODES], dtype=np.uint8)
    vals = e4m3.decode(codes).astype(np.float32)
    assert np.array_equal(e4m3.encode(vals), codes)


def test_decode_known_values():
    assert e4m3.decode_scalar(0x7E) == 448.0
    assert e4m3.decode_scalar(0x08) == 2.0 ** -6
    assert e4m3.decode_scalar(0x01) == 2.0 ** -9
    assert e4m3.decode_scalar(0x38) == 1.0
    # 254 finite values, 127 distinct magnitudes strictly increasing with the code
    mags = [e4m3.decode_scalar(c) for c in range(127)]
    assert all(b > a for a, b in zip(mags, mags[1:]))


def test_vectorised_encode_matches_brute_force():
    vals = _probe_values()
    got = e4m3.encode(vals)
    want = _brute_force(vals)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(vals[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


def test_scalar_encode_matches_brute_force_sample():
    vals = _probe_values(seed=1)
    r = np.random.default_rng(2)
    sample = vals[r.choice(vals.size, size=20000, replace=False)]
    want = _brute_force(sample)
    got = np.array([e4m3.encode_scalar(float(v)) for v in sample], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_subnormal_float32_inputs_and_signed_zero():
    tiny = np.array([2.0 ** -149, -(2.0 ** -149), 2.0 ** -126, 0.0, -0.0], dtype=np.float32)
    assert list(e4m3.encode(tiny)) == [0x00, 0x80, 0x00, 0x00, 0x80]


@pytest.mark.parametrize("v,code", [(448.0, 0x7E), (449.0, 0x7E), (1e30, 0x7E), (-3e38, 0xFE),
                                    (463.99, 0x7E), (464.0, 0x7E)])
def test_saturation(v, code):
    assert int(e4m3.encode(np.array([v], np.float32))[0]) == code
    assert e4m3.encode_scalar(float(np.float32(v))) == code
