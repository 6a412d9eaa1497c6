"""Host-side checks of the preconditions that live in device data.

The C ABI validates every size, type and pointer before it enqueues work,
but the contents of the index tensors are device data the kernels read
without checking (a check there would cost a memory round trip per access):
block ids, context lengths, slots, copy pairs, prefix groups. These
functions check them on the host, from copies of the small index tensors
(never the caches), and raise ``ContractError`` naming the first breach.

They run before every call of the binding when debug checks are on
(``set_debug_checks(True)`` or the environment variable ``PA_DEBUG_CHECKS=1``);
each then synchronises with the device to read the indices, so they are
meant for tests and debugging, not for serving.

The contracts (include/pa.h states each beside its entry point):

* decode: 0 <= context_lens[b] <= max_blocks_per_seq * block_size, and the
  first ceil(context_lens[b] / block_size) entries of block_tables[b] are in
  [0, num_blocks) (a sequence's tokens live in the blocks its table names:
  "PagedAttention deep dive" section 2.1);
* slot write: every non-negative slot is below num_blocks * block_size, and
  the non-negative slots of one call are distinct;
* block copy: every id in [0, num_blocks); destinations distinct and never a
  source of the same call (copy-on-write copies a shared block to a fresh
  one: "PagedAttention deep dive" section 2.3);
* decode with append: the slot of each non-empty sequence's last position
  (n - 1) is distinct, and the block holding it is private to that sequence
  (no other sequence's used block-table entries name it), since the launch
  writes that row while other workgroups read their own blocks;
* prefill: query_start[0] = 0, non-decreasing, query_start[B] = the query
  rows, and each chunk no longer than its sequence's context;
* shared-prefix decode: members in [-1, num_seqs), each sequence in at most
  one slot; each group's whole-block prefix lies within every member's
  context and its table entries are the same physical blocks for every
  member.
"""

import os
from typing import Optional

import numpy as np

__all__ = ["ContractError", "set_debug_checks", "debug_checks_enabled", "check_decode",
           "check_slot_mapping", "check_block_mapping", "check_shared_prefix", "check_append",
           "check_query_start"]


class ContractError(ValueError):
    """Device-data inputs that break an entry point's preconditions."""


_ENABLED: Optional[bool] = None


def set_debug_checks(on: bool) -> None:
    """Turn the checks before every binding call on or off (overrides the
    PA_DEBUG_CHECKS environment variable)."""
    global _ENABLED
    _ENABLED = bool(on)


def debug_checks_enabled() -> bool:
    if _ENABLED is not None:
        return _ENABLED
    return os.environ.get("PA_DEBUG_CHECKS", "0") not in ("", "0")


def _host(a) -> np.ndarray:
    """A host numpy copy of an index tensor (torch, on any device) or array."""
    if hasattr(a, "detach"):
        return a.detach().to("cpu").numpy()
    return np.asarray(a)


def check_decode(block_tables, context_lens, num_blocks: int, block_size: int) -> None:
    bt = _host(block_tables).astype(np.int64)
    cl = _host(context_lens).astype(np.int64)
    B, mbs = bt.shape
    if cl.shape != (B,):
        raise ContractError(f"context_lens has shape {cl.shape}, expected ({B},)")
    cap = mbs * block_size
    bad = np.nonzero((cl < 0) | (cl > cap))[0]
    if len(bad):
        b = int(bad[0])
        raise ContractError(f"context_lens[{b}] = {int(cl[b])} outside [0, {cap}] "
                            f"(max_blocks_per_seq {mbs} x block_size {block_size})")
    used = -(-cl // block_size)
    for b in range(B):
        ids = bt[b, : used[b]]
        out = np.nonzero((ids < 0) | (ids >= num_blocks))[0]
        if len(out):
            j = int(out[0])
            raise ContractError(f"block_tables[{b}][{j}] = {int(ids[j])} outside "
                                f"[0, {num_blocks}) (sequence {b} reads {int(used[b])} blocks)")


def check_slot_mapping(slot_mapping, num_blocks: int, block_size: int) -> None:
    s = _host(slot_mapping).astype(np.int64).reshape(-1)
    live = s[s >= 0]
    over = np.nonzero(live >= num_blocks * block_size)[0]
    if len(over):
        raise ContractError(f"slot {int(live[over[0]])} beyond the pool "
                            f"({num_blocks} blocks x {block_size} tokens)")
    u, counts = np.unique(live, return_counts=True)
    if (counts > 1).any():
        raise ContractError(f"slot {int(u[counts > 1][0])} written twice in one call")


def check_block_mapping(block_mapping, num_blocks: int) -> None:
    m = _host(block_mapping).astype(np.int64).reshape(-1, 2)
    if m.size == 0:
        return
    out = np.nonzero((m < 0) | (m >= num_blocks))
    if len(out[0]):
        i, k = int(out[0][0]), int(out[1][0])
        raise ContractError(f"block_mapping[{i}][{k}] = {int(m[i, k])} outside [0, {num_blocks})")
    src, dst = m[:, 0], m[:, 1]
    u, counts = np.unique(dst, return_counts=True)
    if (counts > 1).any():
        raise ContractError(f"block {int(u[counts > 1][0])} is the destination of two copies")
    both = np.intersect1d(src, dst)
    if len(both):
        raise ContractError(f"block {int(both[0])} is both a source and a destination")


def check_shared_prefix(block_tables, context_lens, group_members, prefix_lens,
                        block_size: int) -> None:
    bt = _host(block_tables).astype(np.int64)
    cl = _host(context_lens).astype(np.int64)
    gm = _host(group_members).astype(np.int64)
    pl = _host(prefix_lens).astype(np.int64)
    B, mbs = bt.shape
    if gm.ndim != 2 or pl.shape != (gm.shape[0],):
        raise ContractError("group_members must be [G, M] and prefix_lens [G]")
    bad = np.nonzero((gm < -1) | (gm >= B))
    if len(bad[0]):
        g, m = int(bad[0][0]), int(bad[1][0])
        raise ContractError(f"group_members[{g}][{m}] = {int(gm[g, m])} outside [-1, {B})")
    listed = gm[gm >= 0]
    u, counts = np.unique(listed, return_counts=True)
    if (counts > 1).any():
        raise ContractError(f"sequence {int(u[counts > 1][0])} is in more than one slot")
    for g in range(gm.shape[0]):
        ids = [int(b) for b in gm[g] if b >= 0]
        if not ids or pl[g] <= 0:
            continue
        pb = min(int(pl[g]) // block_size, mbs)
        for b in ids:
            if cl[b] < pb * block_size:
                raise ContractError(f"group {g}: sequence {b} has {int(cl[b])} tokens, fewer "
                                    f"than the group's whole-block prefix {pb * block_size}")
            if not np.array_equal(bt[b, :pb], bt[ids[0], :pb]):
                j = int(np.nonzero(bt[b, :pb] != bt[ids[0], :pb])[0][0])
                raise ContractError(f"group {g}: sequences {ids[0]} and {b} hold different "
                                    f"blocks at prefix block {j}")


def check_append(block_tables, context_lens, block_size: int) -> None:
    """Decode with append writes each non-empty sequence's position n - 1 in
    the same launch that reads the caches: the block holding it must be named
    by no other sequence's used table entries (a shared block is copied first,
    "PagedAttention deep dive" section 2.3), which also makes the written
    slots distinct."""
    bt = _host(block_tables).astype(np.int64)
    cl = _host(context_lens).astype(np.int64)
    B = bt.shape[0]
    used = -(-cl // block_size)
    owners = {}
    for b in range(B):
        for blk in np.unique(bt[b, : used[b]]).tolist():
            owners.setdefault(int(blk), set()).add(b)
    for b in range(B):
        if cl[b] <= 0:
            continue
        last = int(bt[b, (cl[b] - 1) // block_size])
        others = sorted(owners.get(last, set()) - {b})
        if others:
            raise ContractError(f"sequence {b} appends into block {last}, which sequence "
                                f"{others[0]} also reads (copy the shared block first)")


def check_query_start(query_start, context_lens, num_query_tokens: int) -> None:
    """Prefill: the chunks tile the query rows in sequence order, and each
    chunk (the last tokens of its sequence) fits in the sequence's context."""
    qs = _host(query_start).astype(np.int64)
    cl = _host(context_lens).astype(np.int64)
    if qs.shape != (len(cl) + 1,):
        raise ContractError(f"query_start has shape {qs.shape}, expected ({len(cl) + 1},)")
    if qs[0] != 0 or qs[-1] != num_query_tokens:
        raise ContractError(f"query_start must run from 0 to {num_query_tokens} "
                            f"(got {int(qs[0])} .. {int(qs[-1])})")
    c = np.diff(qs)
    bad = np.nonzero(c < 0)[0]
    if len(bad):
        raise ContractError(f"query_start decreases at sequence {int(bad[0])}")
    over = np.nonzero(c > cl)[0]
    if len(over):
        b = int(over[0])
        raise ContractError(f"sequence {b}: chunk of {int(c[b])} tokens exceeds its context "
                            f"of {int(cl[b])}")
