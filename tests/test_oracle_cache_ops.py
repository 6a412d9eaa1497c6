"""Pins for the oracle's slot write and copy-on-write block copy.

Both are bit operations with one correct result, so the pins are their
definitions checked element by element on small pools, plus the CoW
properties the pages state: the shared source block stays unchanged, the
other sharers still read the old contents, and the writer sees its own token.
"""

import numpy as np
import pytest

import workloads as W
from oracle import copy_blocks, e4m3fn_decode, e4m3fn_encode, paged_decode, reshape_and_cache
from oracle.cache_ops import reshape_and_cache_bulk


def _pool(rng, nb=6, bs=4, hkv=2, d=8, dtype=np.float32):
    return (rng.standard_normal((nb, bs, hkv, d)).astype(dtype),
            rng.standard_normal((nb, bs, hkv, d)).astype(dtype))


def test_slot_write_bit_copy_and_skip():
    rng = np.random.default_rng(0)
    kc, vc = _pool(rng)
    k0, v0 = kc.copy(), vc.copy()
    key = rng.standard_normal((3, 2, 8)).astype(np.float32)
    val = rng.standard_normal((3, 2, 8)).astype(np.float32)
    slots = np.asarray([5, -1, 22])          # block 1 off 1; skipped; block 5 off 2
    reshape_and_cache(key, val, kc, vc, slots)
    assert np.array_equal(kc[1, 1], key[0]) and np.array_equal(vc[5, 2], val[2])
    touched = np.zeros(kc.shape[:2], bool)
    touched[1, 1] = touched[5, 2] = True
    assert np.array_equal(kc[~touched], k0[~touched])
    assert np.array_equal(vc[~touched], v0[~touched])


def test_slot_write_bf16_is_bitwise():
    rng = np.random.default_rng(1)
    kc = rng.integers(0, 1 << 16, size=(4, 4, 1, 8), dtype=np.uint16)
    vc = kc.copy()
    key = rng.integers(0, 1 << 16, size=(2, 1, 8), dtype=np.uint16)   # includes NaN patterns
    reshape_and_cache(key, key, kc, vc, np.asarray([0, 15]))
    assert np.array_equal(kc[0, 0], key[0]) and np.array_equal(kc[3, 3], key[1])


def test_slot_write_fp8_quantises():
    rng = np.random.default_rng(2)
    kc = np.zeros((4, 4, 2, 8), np.uint8)
    vc = np.zeros((4, 4, 2, 8), np.uint8)
    key = (rng.standard_normal((2, 2, 8)) * 3).astype(np.float32)
    val = (rng.standard_normal((2, 2, 8)) * 3).astype(np.float32)
    import torch
    kb = torch.from_numpy(key).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    vb = torch.from_numpy(val).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    kf = (kb.astype(np.uint32) << 16).view(np.float32)
    ks = float(np.float32(np.abs(kf).max() / np.float32(448)))
    vs = 0.002                                             # small: some values saturate
    reshape_and_cache(kb, vb, kc, vc, np.asarray([3, 9]), k_scale=ks, v_scale=vs)
    # stored code = nearest E4M3FN value of float32(x) / float32(scale)
    expect = e4m3fn_encode(kf[0] / np.float32(ks))
    assert np.array_equal(kc[0, 3], expect)
    dec = e4m3fn_decode(kc[0, 3])
    assert np.all(np.abs(dec - (kf[0] / np.float32(ks))) <= np.abs(dec) / 16 + 2.0 ** -10)
    assert np.array_equal(vc[2, 1], e4m3fn_encode(
        (vb[1].astype(np.uint32) << 16).view(np.float32) / np.float32(vs)))
    assert (np.abs(e4m3fn_decode(vc[2, 1])) == 448).any()


def test_slot_write_bulk_equals_loop():
    rng = np.random.default_rng(3)
    kc, vc = _pool(rng, nb=10)
    key = rng.standard_normal((17, 2, 8)).astype(np.float32)
    val = rng.standard_normal((17, 2, 8)).astype(np.float32)
    slots = rng.permutation(40)[:17]
    slots[[2, 9]] = -1
    a = reshape_and_cache(key, val, kc.copy(), vc.copy(), slots)
    b = reshape_and_cache_bulk(key, val, kc.copy(), vc.copy(), slots)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_slot_write_rejects_duplicates():
    rng = np.random.default_rng(4)
    kc, vc = _pool(rng)
    key = rng.standard_normal((2, 2, 8)).astype(np.float32)
    with pytest.raises(AssertionError):
        reshape_and_cache(key, key, kc, vc, np.asarray([3, 3]))


def test_copy_blocks_snapshot_semantics():
    rng = np.random.default_rng(5)
    kc, vc = _pool(rng, nb=8)
    k0, v0 = kc.copy(), vc.copy()
    pairs = np.asarray([[1, 4], [1, 5], [2, 6]])
    copy_blocks(kc, vc, pairs)
    for s, d in pairs:
        assert np.array_equal(kc[d], k0[s]) and np.array_equal(vc[d], v0[s])
    for blk in (0, 1, 2, 3, 7):
        assert np.array_equal(kc[blk], k0[blk]) and np.array_equal(vc[blk], v0[blk])
    copy_blocks(kc, vc, np.zeros((0, 2), np.int64))     # no pairs: no change
    with pytest.raises(AssertionError):
        copy_blocks(kc, vc, np.asarray([[1, 4], [2, 4]]))  # destinations must be distinct
    with pytest.raises(AssertionError):
        copy_blocks(kc, vc, np.asarray([[1, 4], [4, 5]]))  # a destination may not be a source


def test_copy_on_write_end_to_end():
    """Two samples share a partly filled block; the first one to write a
    different token copies it. Afterwards the source is unchanged, the other
    sample reads exactly what it read before, and the writer reads its own
    token."""
    bs, hkv, d = 4, 1, 8
    pool = W.BlockPool(8, bs, order=[3, 0, 6, 1, 7, 2, 5, 4])
    a = pool.new_sequence()
    for _ in range(6):                       # blocks [3, 0], block 0 half full
        pool.append_slot(a)
    b = pool.fork(a)
    rng = np.random.default_rng(6)
    kc = rng.standard_normal((8, bs, hkv, d))
    vc = rng.standard_normal((8, bs, hkv, d))
    q = rng.standard_normal((2, 1, d))

    def decode(seqs, k, v):
        t = np.zeros((2, 2), np.int32)
        for i, s in enumerate(seqs):
            t[i, : len(s.block_table)] = s.block_table
        cl = np.asarray([s.length for s in seqs], np.int32)
        return paged_decode(q, k, v, t, cl, 0.3)

    before = decode([a, b], kc, vc)
    slot_a, cow = pool.append_slot(a)        # a writes first: block 0 is shared -> copy
    assert cow == (0, 6) and a.block_table == [3, 6] and b.block_table == [3, 0]
    k_src, v_src = kc[0].copy(), vc[0].copy()
    copy_blocks(kc, vc, np.asarray([cow]))
    new_k = rng.standard_normal((1, hkv, d))
    new_v = rng.standard_normal((1, hkv, d))
    reshape_and_cache(new_k, new_v, kc, vc, np.asarray([slot_a]))
    assert slot_a == 6 * bs + 2
    assert np.array_equal(kc[0], k_src) and np.array_equal(vc[0], v_src)
    after = decode([a, b], kc, vc)
    assert np.array_equal(after[1], before[1])                  # b unaffected, bitwise
    assert np.array_equal(kc[6, :2], kc[0, :2])                 # copied prefix
    assert np.array_equal(kc[6, 2], new_k[0])                   # a's own token
    slot_b, cow_b = pool.append_slot(b)      # b is now the only holder: in place
    assert cow_b is None and slot_b == 0 * bs + 2


@pytest.mark.parametrize("src", ["bf16", "f16"])
@pytest.mark.parametrize("cache,scale", [("fp8", 0.013), ("fp8", 1.0), ("int8", 0.021),
                                         ("int8", 3.5e-5)])
def test_slot_write_16bit_patterns_match_direct_encoding(src, cache, scale):
    """The 8-bit slot write of a 16-bit source looks each bit pattern's code
    up in a table of all 65536 patterns: over every pattern (NaN, infinities,
    subnormals, both zeros included) it equals the encoding applied to
    float32(x) / float32(scale) element by element, and the chunked bulk
    write equals the per-token loop."""
    from oracle import int8_encode
    from oracle.cache_ops import _encode_rows

    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    if src == "bf16":
        rows, x32 = pats, (pats.astype(np.uint32) << 16).view(np.float32)
    else:
        rows = pats.view(np.float16)
        x32 = rows.astype(np.float32)
    cdt = np.uint8 if cache == "fp8" else np.int8
    enc = e4m3fn_encode if cache == "fp8" else int8_encode
    with np.errstate(invalid="ignore", over="ignore"):
        want = enc(x32 / np.float32(scale))
    assert np.array_equal(_encode_rows(rows.reshape(256, 1, 256), cdt, scale).reshape(-1), want)
    # bulk (chunked) against the loop on a 16-bit source
    rng = np.random.default_rng(7)
    key = rows[rng.integers(0, 1 << 16, size=(37, 2, 8))]
    kc = np.zeros((12, 4, 2, 8), cdt)
    slots = rng.permutation(48)[:37]
    a = reshape_and_cache(key, key, kc.copy(), kc.copy(), slots, scale, scale)
    b = reshape_and_cache_bulk(key, key, kc.copy(), kc.copy(), slots, scale, scale, chunk=5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
