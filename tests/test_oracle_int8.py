"""Pins of the oracle's symmetric int8 codec (the reading of the pages' INT8
KV storage, "PagedAttention deep dive" §4, "KV-Cache evolution" §3C): every
code decodes to itself; encoding is the nearest code with ties to even,
saturating at +-127, checked against a brute-force search over all codes;
and the slot write quantises x / scale with a float32 division."""

import numpy as np

import oracle
from oracle.cache_ops import reshape_and_cache

CODES = np.arange(-127, 128, dtype=np.int64)


def _nearest_even(x):
    """Brute force: the code nearest to x (ties to the even code), with
    values beyond the range going to the end codes."""
    out = []
    for v in np.asarray(x, dtype=np.float64):
        if np.isnan(v):
            out.append(0)
            continue
        # beyond +-200 every distance would round to the same float64; the
        # nearest code of such a value is the end code either way
        v = min(max(v, -200.0), 200.0)
        d = np.abs(CODES - v)
        best = CODES[d == d.min()]
        out.append(int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0]))
    return np.asarray(out, dtype=np.int64)


def test_decode_every_code_is_itself():
    codes = np.arange(-128, 128).astype(np.int8)
    assert np.array_equal(oracle.int8_decode(codes), np.arange(-128, 128, dtype=np.float64))


def test_encode_matches_brute_force_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * 60,
        rng.uniform(-140, 140, 4000).astype(np.float32),
        (np.arange(-130, 131) + 0.5).astype(np.float32),     # every tie
        np.arange(-130, 131).astype(np.float32),
        np.array([np.inf, -np.inf, np.nan, 1e30, -1e30, 0.0, -0.0], dtype=np.float32),
    ])
    got = oracle.int8_encode(x).astype(np.int64)
    assert np.array_equal(got, _nearest_even(x))


def test_ties_and_saturation():
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, 127.49, 127.5, 300.0, -127.5, -1e9],
                 dtype=np.float32)
    assert oracle.int8_encode(x).tolist() == [0, 2, 2, 0, -2, -2, 126, 127, 127, 127, -127, -127]


def test_never_produces_minus_128_and_round_trip_error():
    rng = np.random.default_rng(1)
    x = rng.uniform(-127, 127, 100000).astype(np.float32)
    c = oracle.int8_encode(x)
    assert c.min() >= -127
    assert np.abs(oracle.int8_decode(c) - x.astype(np.float64)).max() <= 0.5


def test_slot_write_quantises_with_a_float32_division():
    """The int8 slot write is int8(float32(x) / float32(scale)), where the
    float32 quotient can differ from the float64 one near a tie."""
    rng = np.random.default_rng(2)
    key = rng.standard_normal((5, 2, 64)).astype(np.float32)
    value = rng.standard_normal((5, 2, 64)).astype(np.float32)
    kc = np.zeros((4, 16, 2, 64), np.int8)
    vc = np.zeros((4, 16, 2, 64), np.int8)
    ks = float(np.float32(np.abs(key).max() / 127))
    vs = float(np.float32(np.abs(value).max() / 127))
    slots = np.array([3, 17, -1, 40, 63])
    reshape_and_cache(key, value, kc, vc, slots, ks, vs)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        want_k = _nearest_even((key[t] / np.float32(ks)).astype(np.float32).reshape(-1))
        want_v = _nearest_even((value[t] / np.float32(vs)).astype(np.float32).reshape(-1))
        assert np.array_equal(kc[s // 16, s % 16].reshape(-1).astype(np.int64), want_k)
        assert np.array_equal(vc[s // 16, s % 16].reshape(-1).astype(np.int64), want_v)
    # with the scale taken over the written tokens, their amax lands on +-127
    live = slots >= 0
    kc2 = np.zeros_like(kc)
    ks2 = float(np.float32(np.abs(key[live]).max() / 127))
    reshape_and_cache(key, value, kc2, vc, slots, ks2, vs)
    assert np.abs(kc2).max() == 127
    # untouched rows stay zero
    assert not kc[0, :3].any() and not kc[2, :8].any()


def test_int8_cache_attention_uses_scaled_codes():
    """Decode over an int8 cache equals decode over the float cache holding
    code x scale (the definition of the dequantised values)."""
    rng = np.random.default_rng(3)
    kc = rng.integers(-127, 128, (6, 16, 2, 64)).astype(np.int8)
    vc = rng.integers(-127, 128, (6, 16, 2, 64)).astype(np.int8)
    q = rng.standard_normal((2, 4, 64)).astype(np.float32)
    bt = np.array([[4, 1, 0], [2, 5, 3]], dtype=np.int32)
    cl = np.array([40, 33], dtype=np.int32)
    ks, vs = 0.0125, 0.03
    a = oracle.paged_decode(q, kc, vc, bt, cl, 0.125, ks, vs)
    # the scales enter as float32 values, widened exactly
    b = oracle.paged_decode(q, kc.astype(np.float64) * float(np.float32(ks)),
                            vc.astype(np.float64) * float(np.float32(vs)), bt, cl, 0.125)
    assert np.allclose(a, b, rtol=0, atol=1e-12)
