"""Host-side block manager: a reference-counted pool of physical KV blocks.

This is the bookkeeping half of paging; the device only ever sees its output
(block tables, slot numbers and copy pairs).

* The cache is cut into fixed-size blocks; each sequence's logical blocks map
  to physical blocks through its block table ("PagedAttention deep dive",
  §2.1).
* A new physical block is taken from the global free pool only when the
  sequence's current block is full ("PagedAttention deep dive", §2.2;
  "KV-cache sharing article", §2.2).
* Blocks carry a reference count; forked sequences (parallel sampling, beam
  search) point at the same blocks without copying ("KV-cache sharing
  article", §2.1 and §2.2).
* Copy-on-write: when a sequence must write into a block that others still
  reference, the block is copied to a fresh one and the writer's table entry
  is redirected; the last remaining holder writes in place ("PagedAttention
  deep dive", §2.3; "KV-cache sharing article", §3.1).
* A sequence's blocks are released at once when it finishes or is pruned;
  a block returns to the pool when its count reaches zero ("KV-cache sharing
  article", §4.1).
"""

from collections import deque
from dataclasses import dataclass, field
from typing import Iterable, List, Optional, Tuple


class PoolExhausted(RuntimeError):
    """Raised when a block is requested from an empty free pool."""


@dataclass
class Sequence:
    seq_id: int
    block_table: List[int] = field(default_factory=list)
    length: int = 0


class BlockPool:
    def __init__(self, num_blocks: int, block_size: int, order: Optional[Iterable[int]] = None):
        """``order`` is the order in which free blocks are handed out (a seeded
        permutation scatters a sequence's blocks through the pool)."""
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        ids = list(range(self.num_blocks)) if order is None else [int(i) for i in order]
        assert sorted(ids) == list(range(self.num_blocks)), "order must be a permutation"
        self._free = deque(ids)
        self.ref = [0] * self.num_blocks
        self._next_seq = 0

    # -- pool -------------------------------------------------------------
    @property
    def num_free(self) -> int:
        return len(self._free)

    def allocate(self) -> int:
        if not self._free:
            raise PoolExhausted(f"all {self.num_blocks} blocks are in use")
        blk = self._free.popleft()
        assert self.ref[blk] == 0
        self.ref[blk] = 1
        return blk

    def _decref(self, blk: int) -> None:
        assert self.ref[blk] > 0
        self.ref[blk] -= 1
        if self.ref[blk] == 0:
            self._free.append(blk)

    # -- sequences --------------------------------------------------------
    def new_sequence(self) -> Sequence:
        s = Sequence(self._next_seq)
        self._next_seq += 1
        return s

    def append_slot(self, seq: Sequence) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Reserve the slot of the sequence's next token.

        Returns (slot, cow) where slot = physical_block * block_size + offset
        and cow is a (src, dst) block pair that must be copied before the
        token is written, or None.
        """
        off = seq.length % self.block_size
        cow = None
        if off == 0:
            seq.block_table.append(self.allocate())
        else:
            last = seq.block_table[-1]
            if self.ref[last] > 1:
                new = self.allocate()
                self._decref(last)
                seq.block_table[-1] = new
                cow = (last, new)
        seq.length += 1
        return seq.block_table[-1] * self.block_size + off, cow

    def fork(self, parent: Sequence) -> Sequence:
        """A child that shares every block of the parent (no copy)."""
        child = self.new_sequence()
        child.block_table = list(parent.block_table)
        child.length = parent.length
        for blk in child.block_table:
            self.ref[blk] += 1
        return child

    def free(self, seq: Sequence) -> None:
        for blk in seq.block_table:
            self._decref(blk)
        seq.block_table = []
        seq.length = 0

    # -- accounting -------------------------------------------------------
    def blocks_in_use(self) -> int:
        return sum(1 for r in self.ref if r > 0)

    def shared_blocks(self) -> int:
        return sum(1 for r in self.ref if r > 1)

    def shared_ratio(self) -> float:
        """shared blocks / blocks in use, the sharing metric the
        "KV-cache sharing article" (§5.2) suggests monitoring."""
        used = self.blocks_in_use()
        return self.shared_blocks() / used if used else 0.0
