"""Pins for the oracle of 8-bit caches with per-head / per-block scales
(``oracle.scaled`` and the block-scale arguments of ``oracle.attention``).

Each check can catch a plausible slip in the oracle:

* brute force in plain Python: each token's K/V value is its code's value
  times the scale looked up, per element, through the token's *physical*
  block and its *KV* head -- catches a scale taken by logical block, by query
  head, from the other cache, or a table transposed;
* the per-tensor case is a special case: a table holding one value
  everywhere gives bitwise the per-tensor result (already pinned elsewhere);
* relabelling physical blocks together with their scale rows changes nothing;
* the slot write per (token, head) reduces to the pinned per-tensor codec
  applied with that row's scale; the bulk form equals the loop form; the
  round trip error stays within the codec's rounding bound;
* copy-on-write moves scale rows with their blocks, from the pre-call state;
* planted mistakes (in a copy of the oracle's lookup) fail the pins.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import (copy_blocks_scaled, e4m3fn_decode, e4m3fn_encode, expand_scales,
                    int8_encode, paged_decode, reshape_and_cache, reshape_and_cache_scaled,
                    reshape_and_cache_scaled_bulk)
from oracle.scaled import PER_BLOCK, PER_BLOCK_HEAD, PER_HEAD

LAYOUTS = [PER_HEAD, PER_BLOCK, PER_BLOCK_HEAD]


def _table_shape(layout, nb, hkv):
    return {PER_HEAD: (hkv,), PER_BLOCK: (nb,), PER_BLOCK_HEAD: (nb, hkv)}[layout]


def _scales(rng, layout, nb, hkv):
    # distinct positive float32 values spread over two decades
    return (10.0 ** rng.uniform(-2, 0, _table_shape(layout, nb, hkv))).astype(np.float32)


def _code_value(code):
    """Value of one stored 8-bit code (int8: the integer; fp8: its E4M3FN value)."""
    if isinstance(code, np.int8):
        return float(int(code))
    return float(e4m3fn_decode(np.asarray([code], np.uint8))[0])


def _scale_of(table, layout, blk, g):
    """Plain lookup of the scale of (physical block blk, KV head g)."""
    if layout == PER_HEAD:
        return float(table[g])
    if layout == PER_BLOCK:
        return float(table[blk])
    return float(table[blk][g])


def _brute_force(q, kc, vc, table_row, n, ks, vs, layout, scale, group):
    """Plain-Python decode of one sequence over an 8-bit cache with scale
    tables: every element dequantised on its own."""
    bs = kc.shape[1]
    Hq, d = q.shape
    out = np.zeros((Hq, d))
    for h in range(Hq):
        g = h // group
        K, V = [], []
        for j in range(n):
            blk, off = int(table_row[j // bs]), j % bs
            K.append([_code_value(kc[blk, off, g, i]) * _scale_of(ks, layout, blk, g)
                      for i in range(d)])
            V.append([_code_value(vc[blk, off, g, i]) * _scale_of(vs, layout, blk, g)
                      for i in range(d)])
        s = [scale * sum(float(q[h, i]) * K[j][i] for i in range(d)) for j in range(n)]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        tot = sum(e)
        for i in range(d):
            out[h, i] = sum(e[j] * V[j][i] for j in range(n)) / tot
    return out


def _case(rng, kv, ctx, Hq, Hkv, d, bs, layout, spare=2):
    nblk = [-(-n // bs) for n in ctx]
    nb = sum(nblk) + spare
    perm = rng.permutation(nb)
    mbs = max(nblk)
    table = np.zeros((len(ctx), mbs), np.int32)
    pos = 0
    for b, k in enumerate(nblk):
        table[b, :k] = perm[pos:pos + k]
        pos += k
    if kv == "int8":
        kc = rng.integers(-127, 128, (nb, bs, Hkv, d)).astype(np.int8)
        vc = rng.integers(-127, 128, (nb, bs, Hkv, d)).astype(np.int8)
    else:
        kc = e4m3fn_encode(rng.standard_normal((nb, bs, Hkv, d)).astype(np.float32) * 30)
        vc = e4m3fn_encode(rng.standard_normal((nb, bs, Hkv, d)).astype(np.float32) * 30)
    q = rng.standard_normal((len(ctx), Hq, d)).astype(np.float32)
    ks = _scales(rng, layout, nb, Hkv)
    vs = _scales(rng, layout, nb, Hkv)
    return q, kc, vc, table, np.asarray(ctx, np.int32), ks, vs


def _oracle(q, kc, vc, table, cl, ks, vs, layout, scale):
    nb, _, hkv = kc.shape[:3]
    return paged_decode(q, kc, vc, table, cl, scale,
                        k_block_scales=expand_scales(ks, layout, nb, hkv),
                        v_block_scales=expand_scales(vs, layout, nb, hkv))


def test_expand_scales_by_definition():
    rng = np.random.default_rng(0)
    nb, hkv = 5, 3
    for layout in LAYOUTS:
        t = _scales(rng, layout, nb, hkv)
        e = expand_scales(t, layout, nb, hkv)
        assert e.shape == (nb, hkv) and e.dtype == np.float64
        for blk in range(nb):
            for g in range(hkv):
                assert e[blk, g] == _scale_of(t, layout, blk, g)
    # a table of the wrong shape is refused, not broadcast
    with pytest.raises(AssertionError):
        expand_scales(np.ones((hkv, nb), np.float32), PER_BLOCK_HEAD, nb, hkv)
    with pytest.raises(AssertionError):
        expand_scales(np.ones(nb, np.float32), PER_HEAD, nb, hkv)


@pytest.mark.parametrize("kv", ["int8", "fp8"])
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("ctx,Hq,Hkv,d,bs", [([1, 18, 33], 4, 2, 4, 8), ([21], 2, 2, 3, 4)])
def test_scaled_decode_brute_force(kv, layout, ctx, Hq, Hkv, d, bs):
    rng = np.random.default_rng(len(ctx) * 10 + layout + (kv == "fp8"))
    q, kc, vc, table, cl, ks, vs = _case(rng, kv, ctx, Hq, Hkv, d, bs, layout)
    scale = float(np.float32(0.3))
    out = _oracle(q, kc, vc, table, cl, ks, vs, layout, scale)
    for b, n in enumerate(ctx):
        ref = _brute_force(q[b], kc, vc, table[b], n, ks, vs, layout, scale, Hq // Hkv)
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


def test_uniform_table_is_the_per_tensor_cache_bitwise():
    rng = np.random.default_rng(3)
    q, kc, vc, table, cl, _, _ = _case(rng, "int8", [40, 17], 4, 2, 8, 16, PER_BLOCK_HEAD)
    nb = kc.shape[0]
    kv_s, v_s = np.float32(0.0123), np.float32(0.047)
    per_tensor = paged_decode(q, kc, vc, table, cl, 0.25, float(kv_s), float(v_s))
    for layout in LAYOUTS:
        shape = _table_shape(layout, nb, 2)
        out = _oracle(q, kc, vc, table, cl, np.full(shape, kv_s), np.full(shape, v_s), layout,
                      0.25)
        assert np.array_equal(out, per_tensor)


def test_relabelling_moves_scale_rows_with_blocks():
    rng = np.random.default_rng(4)
    q, kc, vc, table, cl, ks, vs = _case(rng, "fp8", [50, 3, 16], 8, 2, 8, 16, PER_BLOCK_HEAD)
    nb = kc.shape[0]
    base = _oracle(q, kc, vc, table, cl, ks, vs, PER_BLOCK_HEAD, 0.2)
    perm = rng.permutation(nb)           # old id -> new id
    inv = np.argsort(perm)               # new id -> old id
    out = _oracle(q, kc[inv], vc[inv], perm[table].astype(np.int32), cl, ks[inv], vs[inv],
                  PER_BLOCK_HEAD, 0.2)
    assert np.array_equal(out, base)


def test_planted_lookup_mistakes_are_caught(monkeypatch):
    """Copies of the oracle's scale lookup with one slip each: the scale of
    the logical block instead of the physical one, of the query head instead
    of the KV head (a [NB, Hq] reading), and V dequantised with K's table.
    The brute-force pin rejects every one."""
    rng = np.random.default_rng(6)
    q, kc, vc, table, cl, ks, vs = _case(rng, "int8", [45], 4, 2, 4, 16, PER_BLOCK_HEAD)
    ref = _brute_force(q[0], kc, vc, table[0], 45, ks, vs, PER_BLOCK_HEAD, 0.5, 2)
    good = _oracle(q, kc, vc, table, cl, ks, vs, PER_BLOCK_HEAD, 0.5)[0]
    assert np.abs(good - ref).max() < 1e-12

    import oracle.attention as att
    real = att.widen_blocks

    def logical_index(cache, ids, block_scales=None):
        x = oracle.to_f64(cache[ids])
        if block_scales is not None:
            x = x * np.asarray(block_scales)[np.arange(len(ids))][:, None, :, None]
        return x

    monkeypatch.setattr(att, "widen_blocks", logical_index)
    bad = _oracle(q, kc, vc, table, cl, ks, vs, PER_BLOCK_HEAD, 0.5)[0]
    assert np.abs(bad - ref).max() > 1e-3
    monkeypatch.setattr(att, "widen_blocks", real)

    # scales read per query head: heads 0, 1 of a [NB, Hq] table are both
    # KV head 0 of the cache; with head 1's column, KV head 0 takes a wrong scale
    wrong_k = ks.copy()
    wrong_k[:, 0] = ks[:, 1]
    bad = _oracle(q, kc, vc, table, cl, wrong_k, vs, PER_BLOCK_HEAD, 0.5)[0]
    assert np.abs(bad - ref).max() > 1e-3
    bad = _oracle(q, kc, vc, table, cl, ks, ks, PER_BLOCK_HEAD, 0.5)[0]
    assert np.abs(bad - ref).max() > 1e-3


@pytest.mark.parametrize("cache", [np.int8, np.uint8])
@pytest.mark.parametrize("src", [np.float32, np.float16, np.uint16])
@pytest.mark.parametrize("layout", LAYOUTS)
def test_slot_write_is_the_codec_with_each_rows_scale(cache, src, layout):
    """Per (token, head) the scaled slot write stores exactly what the pinned
    per-tensor slot write stores for that row with that row's scale."""
    rng = np.random.default_rng(layout * 7 + (cache == np.uint8))
    nb, bs, hkv, d = 5, 4, 3, 8
    x = rng.standard_normal((6, hkv, d)).astype(np.float32) * 3
    if src == np.uint16:
        key = (x.view(np.uint32) >> 16).astype(np.uint16)
        value = ((x * 0.5).view(np.uint32) >> 16).astype(np.uint16)
    else:
        key, value = x.astype(src), (x * 0.5).astype(src)
    ks = _scales(rng, layout, nb, hkv)
    vs = _scales(rng, layout, nb, hkv)
    slots = np.array([0, 7, -1, 13, 19, 8])
    kc = np.zeros((nb, bs, hkv, d), cache)
    vc = np.zeros((nb, bs, hkv, d), cache)
    reshape_and_cache_scaled(key, value, kc, vc, slots, ks, vs, layout)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = divmod(int(s), bs)
        for g in range(hkv):
            one_k = np.zeros((1, 1, 1, d), cache)
            one_v = np.zeros((1, 1, 1, d), cache)
            reshape_and_cache(key[t:t + 1, g:g + 1], value[t:t + 1, g:g + 1], one_k, one_v,
                              np.array([0]), _scale_of(ks, layout, blk, g),
                              _scale_of(vs, layout, blk, g))
            assert np.array_equal(kc[blk, off, g], one_k[0, 0, 0])
            assert np.array_equal(vc[blk, off, g], one_v[0, 0, 0])
    # bulk form, small chunks: identical bits; rows never written stay zero
    kb = np.zeros_like(kc)
    vb = np.zeros_like(vc)
    reshape_and_cache_scaled_bulk(key, value, kb, vb, slots, ks, vs, layout, chunk=2)
    assert np.array_equal(kb.view(np.uint8), kc.view(np.uint8))
    assert np.array_equal(vb.view(np.uint8), vc.view(np.uint8))
    assert not kc[0, 1:].any() and not kc[4, :3].any()


def test_int8_round_trip_within_half_a_step_of_each_block():
    """With each block's scale = its amax / 127, every written value comes
    back within half its own block's step (round to nearest), and the block's
    largest magnitude lands on +-127."""
    rng = np.random.default_rng(8)
    nb, bs, hkv, d = 4, 8, 2, 16
    x = (rng.standard_normal((nb * bs, hkv, d)) * rng.uniform(0.01, 10, (nb * bs, 1, 1)))
    x = x.astype(np.float32)
    slots = rng.permutation(nb * bs)
    amax = np.zeros((nb, hkv), np.float32)
    for t, s in enumerate(slots):
        amax[s // bs] = np.maximum(amax[s // bs], np.abs(x[t]).max(axis=1))
    ks = (amax / np.float32(127)).astype(np.float32)
    kc = np.zeros((nb, bs, hkv, d), np.int8)
    vc = np.zeros((nb, bs, hkv, d), np.int8)
    reshape_and_cache_scaled_bulk(x, x, kc, vc, slots, ks, ks, PER_BLOCK_HEAD)
    for t, s in enumerate(slots):
        blk, off = divmod(int(s), bs)
        back = kc[blk, off].astype(np.float64) * ks[blk][:, None].astype(np.float64)
        assert (np.abs(back - x[t]) <= 0.5 * ks[blk][:, None] * (1 + 1e-6)).all()
    assert (np.abs(kc.astype(np.int64)).reshape(nb, -1, hkv, d).max(axis=(1, 3)) == 127).all()


def test_fp8_encode_of_scaled_rows_matches_direct_codec():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((3, 2, 32)).astype(np.float32) * 100
    ks = np.array([[0.5, 0.25], [2.0, 0.125]], np.float32)
    kc = np.zeros((2, 2, 2, 32), np.uint8)
    vc = np.zeros((2, 2, 2, 32), np.uint8)
    slots = np.array([0, 3, 2])
    reshape_and_cache_scaled_bulk(x, x, kc, vc, slots, ks, ks, PER_BLOCK_HEAD)
    for t, s in enumerate(slots):
        blk, off = divmod(int(s), 2)
        for g in range(2):
            assert np.array_equal(kc[blk, off, g], e4m3fn_encode(x[t, g] / ks[blk, g]))
    # saturation past the largest code, sign kept
    y = np.full((1, 2, 32), 1e6, np.float32)
    y[0, 1] = -1e6
    reshape_and_cache_scaled_bulk(y, y, kc, vc, np.array([1]), ks, ks, PER_BLOCK_HEAD)
    assert (e4m3fn_decode(kc[0, 1, 0]) == 448.0).all()
    assert (e4m3fn_decode(kc[0, 1, 1]) == -448.0).all()
    assert (int8_encode(np.array([1e6], np.float32)) == 127).all()


@pytest.mark.parametrize("layout", LAYOUTS)
def test_copy_blocks_moves_scales_from_the_pre_call_state(layout):
    rng = np.random.default_rng(10 + layout)
    nb, bs, hkv, d = 6, 4, 2, 8
    kc = rng.integers(-127, 128, (nb, bs, hkv, d)).astype(np.int8)
    vc = rng.integers(-127, 128, (nb, bs, hkv, d)).astype(np.int8)
    ks = _scales(rng, layout, nb, hkv)
    vs = _scales(rng, layout, nb, hkv)
    k0, v0, ks0, vs0 = kc.copy(), vc.copy(), ks.copy(), vs.copy()
    pairs = np.array([[1, 4], [1, 5], [2, 0]])
    copy_blocks_scaled(kc, vc, ks, vs, layout, pairs)
    for src, dst in pairs:
        assert np.array_equal(kc[dst], k0[src]) and np.array_equal(vc[dst], v0[src])
    untouched = [1, 2, 3]
    assert np.array_equal(kc[untouched], k0[untouched])
    if layout == PER_HEAD:
        assert np.array_equal(ks, ks0) and np.array_equal(vs, vs0)
    else:
        for src, dst in pairs:
            assert np.array_equal(ks[dst], ks0[src]) and np.array_equal(vs[dst], vs0[src])
        assert np.array_equal(ks[untouched], ks0[untouched])
    # after the copy, decode through either block gives the same values
    table = np.array([[1], [4]], np.int32)
    q = rng.standard_normal((1, 2, d)).astype(np.float32)
    out = _oracle(q[[0, 0]], kc, vc, table, np.array([4, 4], np.int32), ks, vs, layout, 0.3)
    assert np.array_equal(out[0], out[1])
