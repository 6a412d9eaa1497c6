"""Oracle for an 8-bit KV cache whose scales are finer than one per tensor:
one float32 scale per KV head, per physical block, or per (physical block,
KV head).

TEST INFRASTRUCTURE ONLY (see the package header).

What the pages fix: the K/V cache may be stored as INT8 or FP8 instead of
FP16, halving its memory, with quality kept within acceptable bounds
("KV-Cache evolution", §3C), and such quantisation is combined with paging
to shrink each cache unit further ("PagedAttention deep dive", §4 item 1;
"KV-cache sharing article", §6, INT8 storage together with block sharing).
The codecs themselves are those of ``oracle.numerics`` (E4M3FN, symmetric
int8), exactly as in the per-tensor case.

Readings taken where the pages are silent (they name the codecs, not the
granularity of their scales):

* A stored code c in physical block ``blk``, KV head ``g`` stands for the
  value value(c) * S[blk, g], where S is the cache's scale table expanded to
  [num_blocks, Hkv] (``expand_scales``): a per-head table repeats one row
  for every block, a per-block table one column for every head.
* The slot write quantises a new token's row of KV head g that lands in
  slot s with the scale of block s // block_size and head g:
  code = enc(float32(x) / float32(S[s // bs, g])), the same rounding as the
  per-tensor slot write.
* Copy-on-write copies a block's scales together with its codes: the scale
  belongs to the block's contents.
* The scales are inputs: how they are chosen (a calibration, e.g. the block's
  largest magnitude over the codec's largest code) is the caller's concern.
"""

import numpy as np

from .cache_ops import _encode_rows
from .numerics import e4m3fn_encode, int8_encode, to_f32_exact

# Layouts of a scale table (the numbering of the library's C interface).
PER_HEAD = 1        # [Hkv]
PER_BLOCK = 2       # [num_blocks]
PER_BLOCK_HEAD = 3  # [num_blocks, Hkv]


def expand_scales(scales, layout, num_blocks, num_kv_heads) -> np.ndarray:
    """The scale of every (physical block, KV head): float64 [num_blocks, Hkv]
    (float32 values widened exactly)."""
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    if layout == PER_HEAD:
        assert s.shape == (num_kv_heads,)
        return np.broadcast_to(s[None, :], (num_blocks, num_kv_heads)).copy()
    if layout == PER_BLOCK:
        assert s.shape == (num_blocks,)
        return np.broadcast_to(s[:, None], (num_blocks, num_kv_heads)).copy()
    if layout == PER_BLOCK_HEAD:
        assert s.shape == (num_blocks, num_kv_heads)
        return s.copy()
    raise ValueError(f"unknown scale layout {layout}")


def reshape_and_cache_scaled(key, value, k_cache, v_cache, slot_mapping, k_scales, v_scales,
                             layout):
    """Slot write into an 8-bit cache with a scale table: for each token t
    with slot s = slot_mapping[t] >= 0 and each KV head g,
    cache[s // bs, s % bs, g] = enc(float32(row) / float32(S[s // bs, g])).
    In place; returns the caches. Slots must be distinct (checked)."""
    nb, bs, hkv = k_cache.shape[:3]
    ks = expand_scales(k_scales, layout, nb, hkv)
    vs = expand_scales(v_scales, layout, nb, hkv)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    live = np.nonzero(slots >= 0)[0]
    assert len(np.unique(slots[live])) == len(live), "duplicate slots in one call"
    for t in live:
        blk, off = divmod(int(slots[t]), bs)
        for g in range(hkv):
            k_cache[blk, off, g] = _encode_rows(key[t, g], k_cache.dtype, np.float32(ks[blk, g]))
            v_cache[blk, off, g] = _encode_rows(value[t, g], v_cache.dtype,
                                                np.float32(vs[blk, g]))
    return k_cache, v_cache


def reshape_and_cache_scaled_bulk(key, value, k_cache, v_cache, slot_mapping, k_scales,
                                  v_scales, layout, chunk=4096):
    """Same result as ``reshape_and_cache_scaled`` for many tokens at once: the
    same elementwise float32 division and encoding, with each row's scale
    broadcast over its head's elements, tokens taken in chunks."""
    nb, bs, hkv = k_cache.shape[:3]
    slots = np.asarray(slot_mapping, dtype=np.int64)
    live = np.nonzero(slots >= 0)[0]
    assert len(np.unique(slots[live])) == len(live), "duplicate slots in one call"
    key, value = np.asarray(key), np.asarray(value)
    for cache, src, table in ((k_cache, key, k_scales), (v_cache, value, v_scales)):
        s32 = expand_scales(table, layout, nb, hkv).astype(np.float32)
        enc = e4m3fn_encode if cache.dtype == np.uint8 else int8_encode
        assert cache.dtype in (np.uint8, np.int8)
        flat = cache.reshape(nb * bs, *cache.shape[2:])
        for c in range(0, len(live), chunk):
            t = live[c:c + chunk]
            blk = slots[t] // bs
            with np.errstate(over="ignore", invalid="ignore"):
                q = to_f32_exact(src[t]) / s32[blk][:, :, None]
            assert q.dtype == np.float32
            flat[slots[t]] = enc(q)
    return k_cache, v_cache


def copy_blocks_scaled(k_cache, v_cache, k_scales, v_scales, layout, block_mapping):
    """Copy-on-write of blocks and their scales: for each (src, dst) pair,
    cache[dst] = cache[src] for both caches and, for a per-block or
    per-(block, head) table, scales[dst] = scales[src]; every pair reads the
    state before the call (destinations distinct and never a source). A
    per-head table has no per-block entries and is left as it is. In place;
    returns (k_cache, v_cache, k_scales, v_scales)."""
    pairs = np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2)
    if len(pairs) == 0:
        return k_cache, v_cache, k_scales, v_scales
    dst = pairs[:, 1]
    assert len(np.unique(dst)) == len(dst), "destination blocks must be distinct"
    assert not np.isin(dst, pairs[:, 0]).any(), "a destination may not be a source"
    arrays = [k_cache, v_cache]
    if layout in (PER_BLOCK, PER_BLOCK_HEAD):
        arrays += [k_scales, v_scales]
    snaps = [a.copy() for a in arrays]
    for src, d in pairs:
        for a, snap in zip(arrays, snaps):
            a[d] = snap[src]
    return k_cache, v_cache, k_scales, v_scales
