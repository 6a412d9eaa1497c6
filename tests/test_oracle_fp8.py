"""Pins for the oracle's element codecs.

* bfloat16 decode: against torch's bfloat16 -> float64 cast, exhaustive.
* E4M3FN decode: against hand-computed values of the format definition and
  torch's float8_e4m3fn cast, exhaustive over all 256 codes.
* E4M3FN encode: brute force (the nearest of all 254 finite codes, ties to
  the even mantissa) on random and boundary inputs; torch's cast where torch
  does not differ by design (|x| < 464: torch maps larger values to NaN
  instead of saturating); saturation and NaN rules.
"""

import numpy as np
import pytest
import torch

from oracle.numerics import bf16_bits_to_f64, e4m3fn_decode, e4m3fn_encode, to_f64

ALL8 = np.arange(256, dtype=np.uint8)


def test_bf16_decode_exhaustive():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_e4m3fn_decode_definition_values():
    d = e4m3fn_decode(ALL8)
    assert d[0x00] == 0.0 and np.signbit(d[0x80])
    assert d[0x01] == 2.0 ** -9                  # smallest subnormal
    assert d[0x07] == 7 * 2.0 ** -9              # largest subnormal
    assert d[0x08] == 2.0 ** -6                  # smallest normal
    assert d[0x38] == 1.0                        # exponent field 7 = bias
    assert d[0x3C] == 1.5
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert np.isnan(d).sum() == 2                # S.1111.111 is the only NaN
    assert np.isfinite(d[np.r_[0:0x7F, 0x80:0xFF]]).all()


def test_e4m3fn_decode_matches_torch():
    d = e4m3fn_decode(ALL8)
    t = torch.from_numpy(ALL8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(t)
    assert np.array_equal(np.isnan(d), nan)
    assert np.array_equal(d[~nan], t[~nan])
    assert np.array_equal(np.signbit(d[~nan]), np.signbit(t[~nan]))


def _brute_force_encode(x):
    """Nearest finite code; ties to the code with an even mantissa; beyond
    448 saturate."""
    finite = ALL8[np.isfinite(e4m3fn_decode(ALL8))]
    vals = e4m3fn_decode(finite)
    out = []
    for v in np.asarray(x, dtype=np.float32).astype(np.float64):
        if np.isnan(v):
            out.append(0xFF if np.signbit(v) else 0x7F)
            continue
        if abs(v) >= 448.0:
            out.append(0xFE if v < 0 else 0x7E)
            continue
        same_sign = finite[(finite >> 7) == (1 if np.signbit(v) else 0)]
        sv = e4m3fn_decode(same_sign)
        dist = np.abs(sv - v)
        best = np.nonzero(dist == dist.min())[0]
        if len(best) > 1:
            best = [i for i in best if (same_sign[i] & 1) == 0]
        out.append(int(same_sign[best[0]]))
    return np.asarray(out, dtype=np.uint8)


def test_e4m3fn_encode_brute_force_random():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(3000).astype(np.float32) * np.float32(30),
        rng.standard_normal(1000).astype(np.float32) * np.float32(0.01),
        (rng.standard_normal(500) * 600).astype(np.float32),
    ])
    assert np.array_equal(e4m3fn_encode(x), _brute_force_encode(x))


def test_e4m3fn_encode_midpoints_and_edges():
    finite = np.r_[0:0x7F].astype(np.uint8)
    vals = e4m3fn_decode(finite)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)  # all exact in float32
    assert np.array_equal(mids.astype(np.float64), (vals[:-1] + vals[1:]) / 2)
    probes = np.concatenate([vals.astype(np.float32), mids, -mids,
                             np.nextafter(mids, np.float32(np.inf)),
                             np.nextafter(mids, np.float32(-np.inf)),
                             np.float32([0.0, -0.0, 464.0, 465.0, 1e30, -1e30, 2.0 ** -10,
                                         2.0 ** -12, np.inf, -np.inf])])
    ours = e4m3fn_encode(probes)
    assert np.array_equal(ours, _brute_force_encode(probes))
    # every representable value encodes to itself
    assert np.array_equal(e4m3fn_encode(vals.astype(np.float32)), finite)
    # ties go to the even mantissa: midpoint of codes 0x38 (1.0) and 0x39 (1.125)
    assert e4m3fn_encode(np.float32([1.0625]))[0] == 0x38
    assert e4m3fn_encode(np.float32([1.1875]))[0] == 0x3A
    # saturation, infinities, NaN, signed zero
    assert e4m3fn_encode(np.float32([1e30, -1e30, np.inf, -np.inf])).tolist() == \
        [0x7E, 0xFE, 0x7E, 0xFE]
    assert e4m3fn_encode(np.float32([np.nan]))[0] == 0x7F
    assert e4m3fn_encode(np.float32([-0.0]))[0] == 0x80


def test_e4m3fn_encode_matches_torch_in_range():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal(200000) * 60).astype(np.float32)
    x = x[np.abs(x) < 464]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3fn_encode(x), ref)


def test_to_f64_dispatch():
    assert to_f64(np.float32([1.5]))[0] == 1.5
    assert to_f64(np.float16([0.25]))[0] == 0.25
    assert to_f64(np.uint16([0x3FC0]))[0] == 1.5
    assert to_f64(np.uint8([0x3C]))[0] == 1.5
    with pytest.raises(TypeError):
        to_f64(np.int32([1]))
