"""Oracle for the two cache-writing operations: the slot write of new tokens'
K/V and the copy-on-write block copy.

* Slot write: during generation, a sequence's newest K/V are appended to its
  cache; tokens fill the current block and a fresh physical block is taken
  only when that one is full ("PagedAttention deep dive", §2.2; "vLLM
  inference principles", two phases of generation: decode extends the cache).
  The host decides the physical slot of each new token (slot = block_id *
  block_size + offset); the device operation stores the token's rows there.
  Reading taken: a negative slot means "no write" (padding tokens).
* Copy-on-write: sequences that share a prompt point at the same physical
  blocks; when one of them must write a different token into a shared block,
  that block is first copied to a new physical block and the writer's mapping
  is updated ("PagedAttention deep dive", §2.3; "KV-cache sharing article",
  §3.1). The device operation is the copy; the decision is host bookkeeping.
  Reading taken: every (src, dst) pair copies from the state before the call
  (destinations distinct and never a source), so pair order does not matter.

Stored element conventions are those of ``oracle.numerics``.
"""

import numpy as np

from .numerics import e4m3fn_encode, int8_encode, to_f32_exact


def _encode_rows(rows: np.ndarray, cache_dtype, scale) -> np.ndarray:
    """Bit copy when the source and cache element types match; otherwise the
    8-bit quantisation e4m3fn(float32(x) / float32(scale)) (fp8 cache) or
    int8(float32(x) / float32(scale)) (int8 cache) with a correctly rounded
    float32 division (numpy's float32 divide is IEEE)."""
    if rows.dtype == cache_dtype:
        return rows.copy()
    if cache_dtype in (np.uint8, np.int8) and rows.dtype in (np.uint16, np.float16):
        # a 16-bit source has 65536 bit patterns: the same encoding evaluated
        # once per pattern, then looked up per element
        patterns = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(rows.dtype)
        with np.errstate(over="ignore", invalid="ignore"):  # inf and NaN patterns
            codes = _encode_rows(patterns.astype(np.float32) if rows.dtype == np.float16
                                 else to_f32_exact(patterns), cache_dtype, scale)
        return codes[np.asarray(rows).view(np.uint16)]
    if cache_dtype in (np.uint8, np.int8):
        x32 = to_f32_exact(rows)
        q = x32 / np.float32(scale)
        assert q.dtype == np.float32
        return e4m3fn_encode(q) if cache_dtype == np.uint8 else int8_encode(q)
    raise TypeError(f"unsupported slot write {rows.dtype} -> {cache_dtype}")


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping,
                      k_scale=1.0, v_scale=1.0):
    """Write token t's rows key[t], value[t] ([Hkv, d]) into
    cache[slot // bs, slot % bs] for every t with slot_mapping[t] >= 0.

    Updates ``k_cache`` / ``v_cache`` in place and returns them. Slots must be
    distinct among the non-negative entries (checked).
    """
    bs = k_cache.shape[1]
    slots = np.asarray(slot_mapping, dtype=np.int64)
    live = np.nonzero(slots >= 0)[0]
    assert len(np.unique(slots[live])) == len(live), "duplicate slots in one call"
    for t in live:
        blk, off = divmod(int(slots[t]), bs)
        k_cache[blk, off] = _encode_rows(key[t], k_cache.dtype, k_scale)
        v_cache[blk, off] = _encode_rows(value[t], v_cache.dtype, v_scale)
    return k_cache, v_cache


def reshape_and_cache_bulk(key, value, k_cache, v_cache, slot_mapping,
                           k_scale=1.0, v_scale=1.0, chunk=8192):
    """Same result as ``reshape_and_cache`` for many tokens at once.

    The per-token loop is replaced by one indexed assignment over the flat
    [num_blocks * bs, Hkv, d] view of each cache; the encoding of each row is
    the same function applied elementwise, so the stored bits are identical.
    """
    bs = k_cache.shape[1]
    slots = np.asarray(slot_mapping, dtype=np.int64)
    live = np.nonzero(slots >= 0)[0]
    assert len(np.unique(slots[live])) == len(live), "duplicate slots in one call"
    kf = k_cache.reshape(k_cache.shape[0] * bs, *k_cache.shape[2:])
    vf = v_cache.reshape(v_cache.shape[0] * bs, *v_cache.shape[2:])
    key, value = np.asarray(key), np.asarray(value)
    # tokens in chunks, so that the float64 temporaries of an 8-bit encoding
    # stay small for long histories (the encoding is elementwise)
    for c in range(0, len(live), chunk):
        t = live[c:c + chunk]
        kf[slots[t]] = _encode_rows(key[t], k_cache.dtype, k_scale)
        vf[slots[t]] = _encode_rows(value[t], v_cache.dtype, v_scale)
    return k_cache, v_cache


def copy_blocks(k_cache, v_cache, block_mapping):
    """For each (src, dst) pair: cache[dst] = cache[src] (bit copy) for both
    caches, all pairs reading the state before the call. In place; returns the
    caches."""
    pairs = np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2)
    if len(pairs) == 0:
        return k_cache, v_cache
    dst = pairs[:, 1]
    assert len(np.unique(dst)) == len(dst), "destination blocks must be distinct"
    assert not np.isin(dst, pairs[:, 0]).any(), "a destination may not be a source"
    k_snap = k_cache.copy()
    v_snap = v_cache.copy()
    for src, d in pairs:
        k_cache[d] = k_snap[src]
        v_cache[d] = v_snap[src]
    return k_cache, v_cache
