"""A deliberately naive block manager, used to pin the oracle's on tiny pools.

It stores no free queue and no reference counts.  Everything the oracle keeps
in a structure is recomputed here by scanning:

* a block's reference count is the number of live block tables that contain it;
* a block is free when that count is zero;
* the free queue's order is the order in which blocks became free: the initial
  order counts as "freed" at times 0..N-1, and a block that a later free drops
  to zero is stamped with the next tick of a clock;
* taking a block takes the free block with the oldest stamp.

That is the first-in first-out pool of "PagedAttention: KV cache as virtual
memory (block manager & fragmentation)", section "Deep dive" (free queue, per
block reference counts, per request tables), and the sharing and copy-on-write
of "PagedAttention: Why Static Batching Wastes Your KV Cache", section "How
does copy-on-write eliminate duplicate prompt KV cache?", written as plainly as
possible and with every lookup a linear scan, so that it cannot share a bug
with the oracle's deque and counters.  It is only meant for pools of a few
blocks.

It models the calls the hot path makes (create, append with copy-on-write,
fork, free, table export).  The readings where the pages are silent are the
oracle's: copy-on-write only for a shared, partly filled last block, the copy
taken before the new blocks, and a freed sequence's blocks stamped in logical
order.
"""

from __future__ import annotations

from typing import Dict, List, Optional, Sequence


class NaivePool:
    def __init__(self, num_blocks: int, block_size: int,
                 init_free_order: Optional[Sequence[int]] = None):
        order = list(range(num_blocks)) if init_free_order is None else [int(x) for x in init_free_order]
        self.n = num_blocks
        self.bs = block_size
        self.stamp = [0] * num_blocks
        for t, b in enumerate(order):
            self.stamp[b] = t
        self.clock = num_blocks
        self.blocks: Dict[int, List[int]] = {}
        self.length: Dict[int, int] = {}
        self.next_id = 0

    # -- scans ---------------------------------------------------------------
    def holders(self, b: int) -> int:
        return sum(1 for tbl in self.blocks.values() for x in tbl if x == b)

    def free_blocks(self) -> List[int]:
        """Free blocks, oldest stamp first: the queue's order."""
        free = [b for b in range(self.n) if self.holders(b) == 0]
        return sorted(free, key=lambda b: self.stamp[b])

    def ref_cnt(self) -> List[int]:
        return [self.holders(b) for b in range(self.n)]

    def _take(self) -> int:
        return self.free_blocks()[0]

    # -- operations ------------------------------------------------------------
    def create(self) -> int:
        s = self.next_id
        self.next_id += 1
        self.blocks[s] = []
        self.length[s] = 0
        return s

    def append(self, s: int, n: int):
        """Returns ``(ok, slots, cow)`` like the oracle's ``alloc_append``."""
        tbl = self.blocks[s]
        length = self.length[s]
        if n == 0:
            return True, [], None
        have = len(tbl)
        want = 0
        while want * self.bs < length + n:   # blocks that cover length + n tokens
            want += 1
        shared_partial = length % self.bs != 0 and self.holders(tbl[-1]) > 1
        if (want - have) + (1 if shared_partial else 0) > len(self.free_blocks()):
            return False, [], None
        cow = None
        if shared_partial:
            dst = self._take()
            cow = (tbl[-1], dst)
            tbl[-1] = dst
        for _ in range(want - have):
            tbl.append(self._take())
        slots = []
        for pos in range(length, length + n):
            slots.append(tbl[pos // self.bs] * self.bs + pos % self.bs)
        self.length[s] = length + n
        return True, slots, cow

    def fork(self, parent: int) -> int:
        s = self.create()
        self.blocks[s] = list(self.blocks[parent])
        self.length[s] = self.length[parent]
        return s

    def free(self, s: int) -> None:
        tbl = self.blocks.pop(s)
        del self.length[s]
        for b in tbl:
            if self.holders(b) == 0:
                self.stamp[b] = self.clock
                self.clock += 1

    def table(self, s: int, width: int) -> List[int]:
        t = self.blocks[s]
        return t + [-1] * (width - len(t))
