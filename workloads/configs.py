"""Seeded synthetic decode workloads.

Each builder returns a ``Workload``: one decode step of one attention layer,
with the cache state before the step and the writes the step performs, in
order:

1. ``copy_blocks(cow_pairs)`` -- copy-on-write copies decided by the host,
2. ``reshape_and_cache(hist_*)`` -- earlier tokens still to be written (the
   fp8 pool fill, or the private tokens of forked samples),
3. ``reshape_and_cache(new_*)`` -- this step's token of every sequence, at
   logical position context_len - 1,
4. ``decode`` over ``context_lens`` tokens.

This module only draws random numbers, rounds them to the storage type, and
runs the host block manager; it holds none of the attention or cache-write
arithmetic, and it is the only code the device path and the oracle share.

Array conventions: float32 / float16 arrays hold those types; uint16 arrays
hold bfloat16 bit patterns; uint8 arrays hold OCP E4M3FN codes.
"""

from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import math

import numpy as np

from .blockpool import BlockPool

STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8_e4m3fn": np.uint8,
           "int8": np.int8}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3fn": 1, "int8": 1}
# 8-bit cache types: filled through the slot write with scale amax|x| / CODE_MAX
CODE_MAX = {"fp8_e4m3fn": 448.0, "int8": 127.0}


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 random draws -> the storage type, round to nearest even."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    import torch

    if dtype == "f16":
        return torch.from_numpy(x).to(torch.float16).numpy()
    if dtype == "bf16":
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(f"random values are not drawn directly in {dtype}")


def normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    return round_to_storage(rng.standard_normal(shape, dtype=np.float32), dtype)


@dataclass
class Workload:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    q_dtype: str
    kv_dtype: str
    q: np.ndarray              # [B, Hq, d]
    k_cache: np.ndarray        # [NB, bs, Hkv, d], state before the step's writes
    v_cache: np.ndarray
    block_tables: np.ndarray   # [B, MBS] int32
    context_lens: np.ndarray   # [B] int32
    scale: float               # softmax scale, a float32 value
    k_scale: float = 1.0
    v_scale: float = 1.0
    cow_pairs: np.ndarray = field(default_factory=lambda: np.zeros((0, 2), np.int64))
    hist_key: Optional[np.ndarray] = None     # [Nh, Hkv, d] (q dtype)
    hist_value: Optional[np.ndarray] = None
    hist_slots: Optional[np.ndarray] = None   # [Nh] int64
    hist_seq: Optional[np.ndarray] = None     # [Nh] int32: the sequence each history token belongs to
    new_key: Optional[np.ndarray] = None      # [B, Hkv, d] (q dtype)
    new_value: Optional[np.ndarray] = None
    new_slots: Optional[np.ndarray] = None    # [B] int64
    partition_size: int = 0                   # launch configuration: 0 single pass, >0 tokens
                                              # per partition, <0 balanced split (-1: automatic)
    # groups of sequences sharing a prompt prefix: member ids [G, M] (-1 for
    # an empty slot) and the shared prefix in tokens [G]; None when no
    # sequences share blocks
    prefix_members: Optional[np.ndarray] = None
    prefix_lens: Optional[np.ndarray] = None
    # 8-bit caches with scale tables instead of per-tensor scales: the layout
    # (1 per KV head [Hkv], 2 per block [NB], 3 per (block, KV head)
    # [NB, Hkv]; 0: per-tensor k_scale / v_scale) and float32 tables
    scale_layout: int = 0
    k_scales: Optional[np.ndarray] = None
    v_scales: Optional[np.ndarray] = None
    info: Dict = field(default_factory=dict)

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def tokens_attended(self) -> int:
        return int(self.context_lens.astype(np.int64).sum())

    def kv_bytes_attended(self) -> int:
        """K and V bytes one decode launch must read: every attended token's
        row of every KV head, once."""
        return self.tokens_attended * 2 * self.num_kv_heads * self.head_dim * ELEM_BYTES[self.kv_dtype]


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def _tables(seqs, mbs: int) -> np.ndarray:
    """Block tables padded with block 0 (any valid id: entries past a
    sequence's last block are never read)."""
    t = np.zeros((len(seqs), mbs), dtype=np.int32)
    for i, s in enumerate(seqs):
        t[i, : len(s.block_table)] = s.block_table
    return t


def _fill_then_append(pool: BlockPool, ctx_lens) -> (List, np.ndarray):
    """Give each sequence ctx-1 cached tokens, then reserve the slot of its
    new token (position ctx-1) through the block manager."""
    seqs, new_slots = [], []
    bs = pool.block_size
    for n in ctx_lens:
        s = pool.new_sequence()
        cached = int(n) - 1
        s.block_table = [pool.allocate() for _ in range(-(-cached // bs))]
        s.length = cached
        slot, cow = pool.append_slot(s)
        assert cow is None
        seqs.append(s)
        new_slots.append(slot)
    return seqs, np.asarray(new_slots, dtype=np.int64)


def shared_prefix_lens(block_tables, context_lens, block_size, members) -> np.ndarray:
    """Shared prefix of each group, in tokens: the leading whole blocks that
    every member's block table holds alike (the blocks a fork shares by
    reference), no further than any member's context reaches with whole
    blocks. members [G, M], -1 for an empty slot."""
    out = np.zeros(len(members), dtype=np.int32)
    for g, row in enumerate(members):
        ids = [int(b) for b in row if b >= 0]
        if not ids:
            continue
        k = min(int(context_lens[b]) // block_size for b in ids)
        first = block_tables[ids[0]]
        j = 0
        while j < k and all(block_tables[b][j] == first[j] for b in ids[1:]):
            j += 1
        out[g] = j * block_size
    return out


def _slots_of_positions(block_table, positions, bs) -> np.ndarray:
    positions = np.asarray(positions, dtype=np.int64)
    return np.asarray(block_table, dtype=np.int64)[positions // bs] * bs + positions % bs


def _dense_workload(name, rng, ctx_lens, num_blocks, Hq, Hkv, d, bs, q_dtype, kv_dtype,
                    partition_size, mbs=None, contiguous=False) -> Workload:
    """Pool filled with random values; one new token per sequence. Physical
    blocks are handed out in a seeded random order, or in id order (each
    sequence's blocks then sit next to each other) with ``contiguous``."""
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    order = np.arange(num_blocks) if contiguous else rng.permutation(num_blocks)
    pool = BlockPool(num_blocks, bs, order=order)
    seqs, new_slots = _fill_then_append(pool, ctx_lens)
    mbs = mbs or max(-(-int(n) // bs) for n in ctx_lens)
    B = len(ctx_lens)
    q = normal(rng, (B, Hq, d), q_dtype)
    k_cache = normal(rng, (num_blocks, bs, Hkv, d), kv_dtype)
    v_cache = normal(rng, (num_blocks, bs, Hkv, d), kv_dtype)
    new_key = normal(rng, (B, Hkv, d), q_dtype)
    new_value = normal(rng, (B, Hkv, d), q_dtype)
    return Workload(
        name=name, num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
        block_size=bs, num_blocks=num_blocks, q_dtype=q_dtype, kv_dtype=kv_dtype,
        q=q, k_cache=k_cache, v_cache=v_cache, block_tables=_tables(seqs, mbs),
        context_lens=ctx_lens, scale=float(np.float32(1.0 / math.sqrt(d))),
        new_key=new_key, new_value=new_value, new_slots=new_slots,
        partition_size=partition_size,
        info={"blocks_used": pool.blocks_in_use(), "shared_ratio": pool.shared_ratio()},
    )


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def tiny_fp32_gqa2(seed: int = 1, partition_size: int = 0) -> Workload:
    """Batch 2, context lengths 37 and 50, 4 query / 2 KV heads (group 2),
    head_dim 64, fp32, block_size 16, pool of 16 physical blocks handed out
    in a seeded random order; scale 1/8."""
    rng = np.random.default_rng(seed)
    return _dense_workload("tiny_fp32_gqa2", rng, [37, 50], 16, 4, 2, 64, 16,
                           "f32", "f32", partition_size)


def llama3_8b_b32(seed: int = 2, partition_size: int = -1, block_size: int = 16,
                  placement: str = "permuted") -> Workload:
    """Llama-3-8B-shaped layer: batch 32, context lengths uniform on
    [512, 4096], 32 query / 8 KV heads, head_dim 128, bf16, block_size 16,
    pool 10 % larger than the blocks in use, handed out in random order.
    ``block_size`` and ``placement`` ("permuted" or "contiguous") vary the
    paging for the block-size study; the context lengths stay the same."""
    if placement not in ("permuted", "contiguous"):
        raise ValueError(f"placement {placement!r}")
    rng = np.random.default_rng(seed)
    ctx = rng.integers(512, 4096, size=32, endpoint=True)
    bs = int(block_size)
    needed = sum(-(-int(n) // bs) for n in ctx)
    nb = math.ceil(1.1 * needed)
    name = "llama3_8b_b32" if (bs, placement) == (16, "permuted") else \
        f"llama3_8b_b32_bs{bs}_{placement}"
    return _dense_workload(name, rng, ctx, nb, 32, 8, 128, bs,
                           "bf16", "bf16", partition_size, mbs=-(-4096 // bs),
                           contiguous=placement == "contiguous")


def mha_b32_ctx4096(seed: int = 3, partition_size: int = -1) -> Workload:
    """MHA-shaped layer: batch 32, every context 4096 tokens, 32 query = 32 KV
    heads, head_dim 128, fp16 (2 GiB of K+V), block_size 16, pool exactly the
    8192 blocks in use, handed out in random order."""
    rng = np.random.default_rng(seed)
    ctx = np.full(32, 4096)
    return _dense_workload("mha_b32_ctx4096", rng, ctx, 32 * 256, 32, 32, 128, 16,
                           "f16", "f16", partition_size)


def shared_prefix_cow_b64(seed: int = 4, partition_size: int = -1, groups: int = 16,
                          samples: int = 4, prompt: int = 2048, parent_decoded: int = 8,
                          private: int = 128, Hq: int = 32, Hkv: int = 8, d: int = 128,
                          bs: int = 16) -> Workload:
    """Parallel sampling over shared prompts: ``groups`` prompts of ``prompt``
    tokens, each decoded ``parent_decoded`` tokens by its parent and then
    forked into ``samples`` samples that share every prompt block by
    reference count. Each sample then appends ``private`` divergent tokens;
    the first private write hits the shared, partly filled last block, so all
    but the last holder copy it first (copy-on-write). The last private token
    is this step's new token. bf16, 32 query / 8 KV heads, head_dim 128.

    The shared prefix is prompt + parent_decoded tokens so that its last block
    is partly filled (a 2048-token prompt alone fills whole 16-token blocks).
    """
    rng = np.random.default_rng(seed)

    def simulate(num_blocks, order):
        pool = BlockPool(num_blocks, bs, order=order)
        parents = []
        for _ in range(groups):
            s = pool.new_sequence()
            for _ in range(prompt + parent_decoded):
                pool.append_slot(s)
            parents.append(s)
        seqs = []
        for p in parents:
            seqs += [p] + [pool.fork(p) for _ in range(samples - 1)]
        shared_ratio_after_fork = pool.shared_ratio()
        cow, hist, new, owner = [], [], [], []
        for step in range(private):
            for i, s in enumerate(seqs):
                slot, pair = pool.append_slot(s)
                if pair is not None:
                    cow.append(pair)
                if step < private - 1:
                    hist.append(slot)
                    owner.append(i)
                else:
                    new.append(slot)
        return pool, seqs, cow, hist, new, owner, shared_ratio_after_fork

    used = simulate(1 << 20, None)[0].blocks_in_use()
    nb = math.ceil(1.1 * used)
    pool, seqs, cow, hist, new, owner, ratio_fork = simulate(nb, rng.permutation(nb))
    B = len(seqs)
    ctx = np.asarray([s.length for s in seqs], dtype=np.int32)
    mbs = max(len(s.block_table) for s in seqs)
    q = normal(rng, (B, Hq, d), "bf16")
    k_cache = normal(rng, (nb, bs, Hkv, d), "bf16")
    v_cache = normal(rng, (nb, bs, Hkv, d), "bf16")
    hist_key = normal(rng, (len(hist), Hkv, d), "bf16")
    hist_value = normal(rng, (len(hist), Hkv, d), "bf16")
    new_key = normal(rng, (B, Hkv, d), "bf16")
    new_value = normal(rng, (B, Hkv, d), "bf16")
    distinct_blocks = len({blk for s in seqs for blk in s.block_table})
    members = np.arange(B, dtype=np.int32).reshape(groups, samples)
    tables = _tables(seqs, mbs)
    return Workload(
        name="shared_prefix_cow_b64", num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv,
        head_dim=d, block_size=bs, num_blocks=nb, q_dtype="bf16", kv_dtype="bf16",
        q=q, k_cache=k_cache, v_cache=v_cache, block_tables=tables,
        context_lens=ctx, scale=float(np.float32(1.0 / math.sqrt(d))),
        cow_pairs=np.asarray(cow, dtype=np.int64).reshape(-1, 2),
        hist_key=hist_key, hist_value=hist_value,
        hist_slots=np.asarray(hist, dtype=np.int64), hist_seq=np.asarray(owner, dtype=np.int32),
        new_key=new_key, new_value=new_value, new_slots=np.asarray(new, dtype=np.int64),
        partition_size=partition_size, prefix_members=members,
        prefix_lens=shared_prefix_lens(tables, ctx, bs, members),
        info={"blocks_used": pool.blocks_in_use(), "shared_ratio": pool.shared_ratio(),
              "shared_ratio_after_fork": ratio_fork, "distinct_blocks": distinct_blocks,
              "groups": groups, "samples": samples},
    )


def long_ctx_fp8_b8(seed: int = 5, partition_size: int = 512, batch: int = 8,
                    ctx_lo: int = 16384, ctx_hi: int = 32768,
                    kv_dtype: str = "fp8_e4m3fn") -> Workload:
    """Long contexts with an fp8 cache: batch 8, context lengths uniform on
    [16384, 32768], 32 query / 8 KV heads, head_dim 128, bf16 queries, K/V
    stored as OCP E4M3FN with one float32 scale per tensor, block_size 16,
    split into 512-token partitions.

    The history (positions 0 .. ctx-2) is drawn N(0,1), rounded to bf16 and
    written through the slot write, which quantises it; the pool starts as
    zeros. Each scale is amax|x| / 448 over that tensor's bf16 values
    (448 being the largest E4M3FN magnitude), rounded to float32.
    With kv_dtype "int8" the cache holds symmetric int8 codes instead, with
    scale amax|x| / 127 (the same workload otherwise).
    """
    rng = np.random.default_rng(seed)
    Hq, Hkv, d, bs = 32, 8, 128, 16
    ctx = rng.integers(ctx_lo, ctx_hi, size=batch, endpoint=True).astype(np.int32)
    needed = sum(-(-int(n) // bs) for n in ctx)
    pool = BlockPool(needed, bs, order=rng.permutation(needed))
    seqs, new_slots = _fill_then_append(pool, ctx)
    hist_slots = np.concatenate([
        _slots_of_positions(s.block_table, np.arange(int(n) - 1), bs)
        for s, n in zip(seqs, ctx)])
    hist_seq = np.repeat(np.arange(batch, dtype=np.int32), ctx - 1)
    q = normal(rng, (batch, Hq, d), "bf16")
    hist_key = normal(rng, (len(hist_slots), Hkv, d), "bf16")
    hist_value = normal(rng, (len(hist_slots), Hkv, d), "bf16")
    new_key = normal(rng, (batch, Hkv, d), "bf16")
    new_value = normal(rng, (batch, Hkv, d), "bf16")

    def amax_scale(*parts):
        m = max(float(np.abs(_bf16_as_f32(p)).max()) for p in parts)
        return float(np.float32(np.float32(m) / np.float32(CODE_MAX[kv_dtype])))

    zeros = np.zeros((needed, bs, Hkv, d), dtype=STORAGE[kv_dtype])
    return Workload(
        name="long_ctx_fp8_b8" if kv_dtype == "fp8_e4m3fn" else f"long_ctx_{kv_dtype}_b8",
        num_seqs=batch, num_q_heads=Hq, num_kv_heads=Hkv,
        head_dim=d, block_size=bs, num_blocks=needed, q_dtype="bf16", kv_dtype=kv_dtype,
        q=q, k_cache=zeros, v_cache=zeros.copy(),
        block_tables=_tables(seqs, 32768 // bs), context_lens=ctx,
        scale=float(np.float32(1.0 / math.sqrt(d))),
        k_scale=amax_scale(hist_key, new_key), v_scale=amax_scale(hist_value, new_value),
        hist_key=hist_key, hist_value=hist_value, hist_slots=hist_slots, hist_seq=hist_seq,
        new_key=new_key, new_value=new_value, new_slots=new_slots,
        partition_size=partition_size,
        info={"blocks_used": pool.blocks_in_use(), "shared_ratio": pool.shared_ratio()},
    )


def _bf16_as_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


BUILDERS = {
    "tiny_fp32_gqa2": tiny_fp32_gqa2,
    "llama3_8b_b32": llama3_8b_b32,
    "mha_b32_ctx4096": mha_b32_ctx4096,
    "shared_prefix_cow_b64": shared_prefix_cow_b64,
    "long_ctx_fp8_b8": long_ctx_fp8_b8,
    "long_ctx_int8_b8": lambda **kw: long_ctx_fp8_b8(**{"kv_dtype": "int8", **kw}),
}


def build(name: str, **kw) -> Workload:
    return BUILDERS[name](**kw)


# ---------------------------------------------------------------------------
# generic generator for edge cases
# ---------------------------------------------------------------------------

def custom(ctx_lens, Hq, Hkv, d, q_dtype="bf16", kv_dtype="bf16", bs=16, seed=0,
           extra_blocks=3, partition_size=0, mbs=None, name="custom") -> Workload:
    """Random workload with given context lengths (a context length of 0 is
    allowed: such a sequence owns no block and gets no new token)."""
    rng = np.random.default_rng(seed)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    needed = sum(-(-int(n) // bs) for n in ctx_lens)
    nb = needed + extra_blocks
    pool = BlockPool(nb, bs, order=rng.permutation(nb))
    seqs, slots = [], []
    for n in ctx_lens:
        s = pool.new_sequence()
        if n > 0:
            cached = int(n) - 1
            s.block_table = [pool.allocate() for _ in range(-(-cached // bs))]
            s.length = cached
            slot, _ = pool.append_slot(s)
        else:
            slot = -1
        seqs.append(s)
        slots.append(slot)
    B = len(ctx_lens)
    mbs = mbs or max(1, max(-(-int(n) // bs) for n in ctx_lens))
    store_kv = kv_dtype if kv_dtype not in CODE_MAX else None
    if store_kv is None:
        k_cache = np.zeros((nb, bs, Hkv, d), STORAGE[kv_dtype])
        v_cache = np.zeros((nb, bs, Hkv, d), STORAGE[kv_dtype])
        hist_slots = np.concatenate([
            _slots_of_positions(s.block_table, np.arange(int(n) - 1), bs)
            for s, n in zip(seqs, ctx_lens) if n > 1] or [np.zeros(0, np.int64)])
        hist_seq = np.repeat(np.arange(len(ctx_lens), dtype=np.int32),
                             np.maximum(ctx_lens.astype(np.int64) - 1, 0))
        hist_key = normal(rng, (len(hist_slots), Hkv, d), q_dtype)
        hist_value = normal(rng, (len(hist_slots), Hkv, d), q_dtype)
    else:
        k_cache = normal(rng, (nb, bs, Hkv, d), kv_dtype)
        v_cache = normal(rng, (nb, bs, Hkv, d), kv_dtype)
        hist_slots = hist_key = hist_value = hist_seq = None
    q = normal(rng, (B, Hq, d), q_dtype)
    new_key = normal(rng, (B, Hkv, d), q_dtype)
    new_value = normal(rng, (B, Hkv, d), q_dtype)
    wl = Workload(
        name=name, num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, block_size=bs,
        num_blocks=nb, q_dtype=q_dtype, kv_dtype=kv_dtype, q=q, k_cache=k_cache,
        v_cache=v_cache, block_tables=_tables(seqs, mbs), context_lens=ctx_lens,
        scale=float(np.float32(1.0 / math.sqrt(d))), hist_key=hist_key,
        hist_value=hist_value, hist_slots=hist_slots, hist_seq=hist_seq, new_key=new_key,
        new_value=new_value,
        new_slots=np.asarray(slots, dtype=np.int64), partition_size=partition_size,
        info={"blocks_used": pool.blocks_in_use()},
    )
    if store_kv is None:
        parts_k = [_bf16_as_f32(a) if a.dtype == np.uint16 else a.astype(np.float32)
                   for a in (hist_key, new_key)]
        parts_v = [_bf16_as_f32(a) if a.dtype == np.uint16 else a.astype(np.float32)
                   for a in (hist_value, new_value)]
        cmax = np.float32(CODE_MAX[kv_dtype])
        wl.k_scale = float(np.float32(np.float32(max(np.abs(p).max() for p in parts_k if p.size))
                                      / cmax))
        wl.v_scale = float(np.float32(np.float32(max(np.abs(p).max() for p in parts_v if p.size))
                                      / cmax))
    return wl


# ---------------------------------------------------------------------------
# scale tables for 8-bit caches
# ---------------------------------------------------------------------------

def with_scale_tables(wl: Workload, layout: int) -> Workload:
    """The same workload with its 8-bit cache quantised through scale tables
    of the given layout (1 per KV head, 2 per physical block, 3 per (block,
    KV head)) instead of one scale per tensor.

    The tables are a caller's calibration, fixed before any write: each
    entry is amax|x| / code_max over the K (resp. V) values of every token
    the step writes into that block and head (history and new tokens),
    rounded to float32 (code_max 448 for E4M3FN, 127 for int8); an entry no
    token reaches is 1.0. The pool holds no other values (it starts empty and
    is filled by the step's writes)."""
    assert wl.kv_dtype in CODE_MAX and wl.hist_slots is not None
    nb, hkv = wl.num_blocks, wl.num_kv_heads
    slots = np.concatenate([wl.hist_slots, wl.new_slots[wl.new_slots >= 0]])
    blk = slots // wl.block_size
    cmax = np.float32(CODE_MAX[wl.kv_dtype])

    def table(hist, new):
        rows = np.concatenate([hist, new[wl.new_slots >= 0]])
        x = _bf16_as_f32(rows) if rows.dtype == np.uint16 else rows.astype(np.float32)
        per_row = np.abs(x).max(axis=2)                 # [N, Hkv]
        amax = np.zeros((nb, hkv), np.float32)
        np.maximum.at(amax, blk, per_row)
        if layout == 1:
            keep = amax.max(axis=0)
        elif layout == 2:
            keep = amax.max(axis=1)
        else:
            keep = amax
        keep = np.asarray(keep, np.float32)
        return np.where(keep > 0, keep / cmax, np.float32(1.0)).astype(np.float32)

    zeros = np.zeros_like(wl.k_cache)
    return replace(wl, name=f"{wl.name}_scales{layout}", scale_layout=int(layout),
                   k_scales=table(wl.hist_key, wl.new_key),
                   v_scales=table(wl.hist_value, wl.new_value),
                   k_cache=zeros, v_cache=zeros.copy(), k_scale=1.0, v_scale=1.0)


# ---------------------------------------------------------------------------
# relabelings used by the invariance tests
# ---------------------------------------------------------------------------

def permute_physical(wl: Workload, seed: int) -> Workload:
    """The same logical caches with every physical block id relabelled by a
    random permutation (pool contents moved accordingly)."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(wl.num_blocks)          # old id -> new id
    inv = np.argsort(perm)                          # new id -> old id
    bs = wl.block_size

    def slots(s):
        if s is None:
            return None
        s = np.asarray(s, dtype=np.int64)
        return np.where(s >= 0, perm[np.maximum(s, 0) // bs] * bs + np.maximum(s, 0) % bs, s)

    return replace(
        wl,
        k_cache=wl.k_cache[inv].copy(), v_cache=wl.v_cache[inv].copy(),
        block_tables=perm[wl.block_tables].astype(np.int32),
        cow_pairs=perm[wl.cow_pairs].astype(np.int64).reshape(-1, 2),
        hist_slots=slots(wl.hist_slots), new_slots=slots(wl.new_slots),
        # per-block scale tables move with their blocks
        k_scales=wl.k_scales[inv].copy() if wl.scale_layout in (2, 3) else wl.k_scales,
        v_scales=wl.v_scales[inv].copy() if wl.scale_layout in (2, 3) else wl.v_scales,
    )


def unshare(wl: Workload) -> Workload:
    """The same logical caches with no block referenced by two sequences:
    every extra reference gets a private copy of the block, appended to the
    pool. Only meaningful once all writes of the step are applied (the
    copy-on-write pairs and slots are dropped), so it takes a workload whose
    caches already hold the step's writes."""
    seen = set()
    tables = wl.block_tables.copy()
    extra_k, extra_v = [], []
    nb = wl.num_blocks
    for b in range(wl.num_seqs):
        nblk = -(-int(wl.context_lens[b]) // wl.block_size)
        for j in range(nblk):
            blk = int(tables[b, j])
            if blk in seen:
                extra_k.append(wl.k_cache[blk])
                extra_v.append(wl.v_cache[blk])
                tables[b, j] = nb
                nb += 1
            else:
                seen.add(blk)
    k = np.concatenate([wl.k_cache, np.stack(extra_k)]) if extra_k else wl.k_cache.copy()
    v = np.concatenate([wl.v_cache, np.stack(extra_v)]) if extra_v else wl.v_cache.copy()
    return replace(wl, k_cache=k, v_cache=v, block_tables=tables, num_blocks=nb,
                   cow_pairs=np.zeros((0, 2), np.int64), hist_key=None, hist_value=None,
                   hist_slots=None, hist_seq=None, new_key=None, new_value=None, new_slots=None)


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

@dataclass
class PrefillWorkload:
    """A cache state (``cache``: a decode Workload whose step writes fill every
    sequence's context, chunk included) plus the chunks' query rows."""
    name: str
    cache: Workload
    q: np.ndarray             # [T, Hq, d] (q dtype)
    query_start: np.ndarray   # [B + 1] int32
    chunk_lens: np.ndarray    # [B] int32

    @property
    def max_query_len(self) -> int:
        return int(self.chunk_lens.max()) if len(self.chunk_lens) else 0

    @property
    def num_query_tokens(self) -> int:
        return int(self.query_start[-1])


def prefill_custom(ctx_lens, chunk_lens, Hq, Hkv, d, q_dtype="bf16", kv_dtype="bf16", bs=16,
                   seed=0, extra_blocks=3, name="prefill_custom") -> PrefillWorkload:
    """Sequences of ctx_lens cached tokens whose last chunk_lens tokens are
    the chunk being prefilled. Values: fp32 N(0,1) rounded to the storage
    types (8-bit caches through the slot write, as ``custom``)."""
    ctx_lens = np.asarray(ctx_lens, dtype=np.int64)
    chunk_lens = np.asarray(chunk_lens, dtype=np.int64)
    assert (chunk_lens <= ctx_lens).all() and (chunk_lens >= 0).all()
    wl = custom(ctx_lens, Hq, Hkv, d, q_dtype=q_dtype, kv_dtype=kv_dtype, bs=bs, seed=seed,
                extra_blocks=extra_blocks, name=name)
    rng = np.random.default_rng([426, 7, int(seed)])
    qs = np.concatenate([[0], np.cumsum(chunk_lens)]).astype(np.int32)
    q = normal(rng, (int(qs[-1]), Hq, d), q_dtype)
    return PrefillWorkload(name=name, cache=wl, q=q, query_start=qs,
                           chunk_lens=chunk_lens.astype(np.int32))


def prefill_llama3_8b_b8(seed: int = 8, prefix: int = 2048, chunk: int = 2048,
                         batch: int = 8) -> PrefillWorkload:
    """Chunked prefill with Llama-3-8B attention shapes: 8 sequences, each a
    2048-token chunk after a 2048-token cached prefix (contexts of 4096), 32
    query / 8 KV heads, head_dim 128, bf16, 16-token blocks in a permuted
    pool."""
    return prefill_custom([prefix + chunk] * batch, [chunk] * batch, 32, 8, 128, "bf16", "bf16",
                          seed=seed, name="prefill_llama3_8b_b8")


PREFILL_BUILDERS = {"prefill_llama3_8b_b8": prefill_llama3_8b_b8}
