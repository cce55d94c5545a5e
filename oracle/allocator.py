"""Block-manager model (test infrastructure only; see ``oracle/__init__``).

Follows [p2] "PagedAttention: KV cache as virtual memory", sections "Direct
answer" and "Deep dive", and [p3] "PagedAttention: Why Static Batching Wastes
Your KV Cache", sections "What does PagedAttention actually do differently?"
and "How does copy-on-write eliminate duplicate prompt KV cache?":

* one shared pool of fixed-size physical blocks; free blocks sit in a queue,
  allocation takes from the front and freeing appends at the back;
* each block carries a reference count; a block goes back to the queue when its
  count reaches zero;
* each sequence owns a block table (logical block index -> physical block id);
  a block is taken only when the sequence grows past a block boundary;
* forking a sequence shares every block (count + 1 each), like ``fork()``;
* writing new tokens into a shared, partly filled last block first copies that
  one block to a fresh one and repoints the table entry (copy-on-write).

Readings where the pages are silent (stated in the design notes as well):

* the initial queue order is 0..N-1 unless an explicit order is given;
* freeing a sequence walks its table in logical order, appending each block whose
  count drops to zero;
* inside one append the copy-on-write block is taken first, then new blocks in
  increasing logical index;
* copy-on-write fires only when tokens land in an existing partial last block
  whose count is above one; the last holder writes in place;
* every call is all-or-nothing: on any error the state is unchanged.

Prefix caching ([p2] "Deep dive", the prefix-caching bullet; [p1] "Automatic
Prefix Caching (APC)", "APC Mechanics" and "Evaluating APC Hit Rates"):

* a full block is identified by the token ids of the whole prefix up to its
  end (the pages key it by its own tokens plus its parent's key, which names
  the same prefix); only full blocks are cached;
* a new prompt walks its full blocks from the start and reuses every block
  whose prefix is cached, stopping at the first miss; a reused block's count
  goes up by one ("touch"), and a reused block that sat in the free queue
  leaves it from wherever it is;
* freed blocks keep their cache entry while they wait in the free queue, and
  lose it when the queue hands them out again (the queue front is the eviction
  order);
* the hit rate is reused prompt tokens over prompt tokens.

Readings where the pages are silent:

* a block enters the cache only when the caller says its K/V is written
  (``cache_commit``), so no request can reuse a block whose K/V is still
  being computed;
* the last prompt token is never served from the cache (its query starts the
  generation), so a prompt reuses at most ``(n - 1) // block_size`` blocks;
* a sequence's tokens are known only while every append supplied them; after
  an append without token ids its later blocks are never cached;
* if a prefix is already cached under another block, committing an identical
  block leaves it private (one cached copy per prefix);
* inside ``alloc_prompt`` the reused blocks are taken first (in logical
  order), then new blocks from the queue front.

Preemption by swapping ([p3] "What happens when the GPU runs out of KV
blocks?": copy the evicted blocks to CPU RAM, copy them back when the sequence
is rescheduled):

* host blocks form a second pool with its own first-in first-out queue;
* swapping out walks the table in logical order, takes a host block from the
  host queue front for each block and drops the sequence's reference to the
  device block (back of the device queue at zero);
* swapping in walks the host table in logical order, takes a device block from
  the queue front for each and returns the host block to the back of the host
  queue;
* a swapped-out sequence keeps its length and tokens but cannot grow, fork,
  commit or be exported until it is swapped in; its tokens count neither in
  ``tokens`` nor in ``waste_tokens`` (those describe device memory).
"""

from __future__ import annotations

import collections
from typing import Dict, List, Optional, Sequence, Tuple


class Status:
    OK = "ok"
    NO_BLOCKS = "no_blocks"
    BAD_SEQ = "bad_seq"
    BAD_ARG = "bad_arg"
    CAPACITY = "capacity"


class OraclePool:
    def __init__(self, num_blocks: int, block_size: int = 16,
                 init_free_order: Optional[Sequence[int]] = None):
        if num_blocks < 1 or block_size < 1:
            raise ValueError("bad pool shape")
        if init_free_order is None:
            order = list(range(num_blocks))
        else:
            order = [int(x) for x in init_free_order]
            if sorted(order) != list(range(num_blocks)):
                raise ValueError("init_free_order must be a permutation of 0..N-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = collections.deque(order)
        self.ref_cnt: List[int] = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}
        self.next_seq = 0
        self.cow_copies = 0
        # prefix cache
        self.tokens: Dict[int, List[int]] = {}   # known token ids per sequence
        self.cache: Dict[Tuple[int, ...], int] = {}  # prefix -> physical block
        self.block_key: Dict[int, Tuple[int, ...]] = {}  # physical block -> its prefix
        self.prompt_tokens = 0
        self.hit_tokens = 0
        self.evictions = 0
        # swap space
        self.host_n = 0
        self.host_free = collections.deque()
        self.swapped = set()

    # -- sequences -------------------------------------------------------
    def seq_create(self) -> Tuple[str, int]:
        sid = self.next_seq
        self.next_seq += 1
        self.tables[sid] = []
        self.lens[sid] = 0
        self.tokens[sid] = []
        return Status.OK, sid

    def _take_front(self) -> int:
        """Pop the queue front; a cached block loses its cache entry (evicted)."""
        b = self.free.popleft()
        key = self.block_key.pop(b, None)
        if key is not None:
            del self.cache[key]
            self.evictions += 1
        return b

    def alloc_append(self, sid: int, n: int, token_ids: Optional[List[int]] = None):
        """Reserve room for ``n`` new tokens of sequence ``sid``.

        Returns ``(status, slots, cow)`` where ``slots[i]`` is the flat cache
        slot (physical block * block_size + offset) of token ``len + i`` and
        ``cow`` is ``(src, dst)`` when a shared partial block was copied, else
        ``None``.  Without ``token_ids`` the sequence's later tokens are unknown
        and its later blocks are never cached.
        """
        if sid not in self.tables:
            return Status.BAD_SEQ, [], None
        if n < 0 or sid in self.swapped:
            return Status.BAD_ARG, [], None
        bs = self.block_size
        table = self.tables[sid]
        length = self.lens[sid]
        if n == 0:
            return Status.OK, [], None
        # blocks the sequence must hold after the append (one per started block)
        blocks_after = (length + n + bs - 1) // bs
        new_blocks = blocks_after - len(table)
        partial_last = (length % bs) != 0
        cow = partial_last and self.ref_cnt[table[-1]] > 1
        need = new_blocks + (1 if cow else 0)
        if need > len(self.free):
            return Status.NO_BLOCKS, [], None
        cow_pair = None
        if cow:
            src = table[-1]
            dst = self._take_front()
            self.ref_cnt[src] -= 1
            self.ref_cnt[dst] = 1
            table[-1] = dst
            cow_pair = (src, dst)
            self.cow_copies += 1
        for _ in range(new_blocks):
            b = self._take_front()
            self.ref_cnt[b] = 1
            table.append(b)
        slots = []
        for i in range(n):
            pos = length + i
            slots.append(table[pos // bs] * bs + pos % bs)
        self.lens[sid] = length + n
        if token_ids is not None and len(self.tokens[sid]) == length:
            self.tokens[sid].extend(int(t) for t in token_ids)
        return Status.OK, slots, cow_pair

    def append_tokens(self, sid: int, token_ids: Sequence[int]):
        """``alloc_append`` that also records the new tokens' ids."""
        return self.alloc_append(sid, len(token_ids), token_ids=list(token_ids))

    def alloc_prompt(self, sid: int, token_ids: Sequence[int]):
        """Admit a prompt into an empty sequence, reusing cached full blocks.

        Returns ``(status, slots, hit_tokens)``: the prompt's first
        ``hit_tokens`` tokens come from cached blocks, and ``slots`` holds the
        cache slots of the remaining tokens, in order.
        """
        if sid not in self.tables:
            return Status.BAD_SEQ, [], 0
        if self.lens[sid] != 0 or sid in self.swapped:
            return Status.BAD_ARG, [], 0
        toks = [int(t) for t in token_ids]
        n = len(toks)
        bs = self.block_size
        hits = []
        for i in range((n - 1) // bs if n > 0 else 0):
            b = self.cache.get(tuple(toks[:bs * (i + 1)]))
            if b is None:
                break
            hits.append(b)
        new_blocks = (n + bs - 1) // bs - len(hits)
        free_hits = sum(1 for b in hits if self.ref_cnt[b] == 0)
        if new_blocks > len(self.free) - free_hits:
            return Status.NO_BLOCKS, [], 0
        table = self.tables[sid]
        for b in hits:
            if self.ref_cnt[b] == 0:
                self.free.remove(b)
            self.ref_cnt[b] += 1
            table.append(b)
        for _ in range(new_blocks):
            b = self._take_front()
            self.ref_cnt[b] = 1
            table.append(b)
        hit = len(hits) * bs
        slots = [table[pos // bs] * bs + pos % bs for pos in range(hit, n)]
        self.lens[sid] = n
        self.tokens[sid] = toks
        self.prompt_tokens += n
        self.hit_tokens += hit
        return Status.OK, slots, hit

    def cache_commit(self, sid: int):
        """Enter the sequence's full, token-known blocks into the cache (their
        K/V is written).  Returns ``(status, newly cached blocks)``."""
        if sid not in self.tables:
            return Status.BAD_SEQ, 0
        if sid in self.swapped:
            return Status.BAD_ARG, 0
        bs = self.block_size
        toks = self.tokens[sid]
        table = self.tables[sid]
        added = 0
        for i in range(len(toks) // bs):
            key = tuple(toks[:bs * (i + 1)])
            if key in self.cache:
                continue
            b = table[i]
            if b in self.block_key:
                continue  # already cached under its own prefix
            self.cache[key] = b
            self.block_key[b] = key
            added += 1
        return Status.OK, added

    def fork(self, parent: int) -> Tuple[str, int]:
        if parent not in self.tables:
            return Status.BAD_SEQ, -1
        if parent in self.swapped:
            return Status.BAD_ARG, -1
        sid = self.next_seq
        self.next_seq += 1
        self.tables[sid] = list(self.tables[parent])
        self.lens[sid] = self.lens[parent]
        self.tokens[sid] = list(self.tokens[parent])
        for b in self.tables[sid]:
            self.ref_cnt[b] += 1
        return Status.OK, sid

    def seq_free(self, sid: int) -> str:
        if sid not in self.tables:
            return Status.BAD_SEQ
        if sid in self.swapped:
            self.host_free.extend(self.tables[sid])
            self.swapped.discard(sid)
        else:
            for b in self.tables[sid]:
                self.ref_cnt[b] -= 1
                if self.ref_cnt[b] == 0:
                    self.free.append(b)
        del self.tables[sid]
        del self.lens[sid]
        del self.tokens[sid]
        return Status.OK

    # -- export ------------------------------------------------------------
    def block_tables(self, sids: Sequence[int], max_blocks: int):
        """Padded ``[len(sids)][max_blocks]`` table (pad -1) and lengths."""
        for s in sids:
            if s not in self.tables:
                return Status.BAD_SEQ, None, None
            if s in self.swapped:
                return Status.BAD_ARG, None, None
            if len(self.tables[s]) > max_blocks:
                return Status.CAPACITY, None, None
        rows, lens = [], []
        for s in sids:
            t = self.tables[s]
            rows.append(list(t) + [-1] * (max_blocks - len(t)))
            lens.append(self.lens[s])
        return Status.OK, rows, lens

    # -- swapping ----------------------------------------------------------
    def set_swap_space(self, n: int) -> str:
        if n < 0 or self.swapped:
            return Status.BAD_ARG
        self.host_n = n
        self.host_free = collections.deque(range(n))
        return Status.OK

    def swap_out(self, sid: int):
        """Returns ``(status, [(device, host), ...])``."""
        if sid not in self.tables:
            return Status.BAD_SEQ, []
        if sid in self.swapped:
            return Status.BAD_ARG, []
        table = self.tables[sid]
        if len(table) > len(self.host_free):
            return Status.NO_BLOCKS, []
        pairs = []
        for i, b in enumerate(table):
            h = self.host_free.popleft()
            pairs.append((b, h))
            self.ref_cnt[b] -= 1
            if self.ref_cnt[b] == 0:
                self.free.append(b)
            table[i] = h
        self.swapped.add(sid)
        return Status.OK, pairs

    def swap_in(self, sid: int):
        """Returns ``(status, [(host, device), ...])``."""
        if sid not in self.tables:
            return Status.BAD_SEQ, []
        if sid not in self.swapped:
            return Status.BAD_ARG, []
        table = self.tables[sid]
        if len(table) > len(self.free):
            return Status.NO_BLOCKS, []
        pairs = []
        for i, h in enumerate(table):
            b = self._take_front()
            self.ref_cnt[b] = 1
            pairs.append((h, b))
            self.host_free.append(h)
            table[i] = b
        self.swapped.discard(sid)
        return Status.OK, pairs

    def stats(self) -> Dict[str, int]:
        free = len(self.free)
        dev = [s for s in self.tables if s not in self.swapped]
        tokens = sum(self.lens[s] for s in dev)
        waste = sum(len(self.tables[s]) * self.block_size - self.lens[s] for s in dev)
        return {
            "num_blocks": self.num_blocks,
            "free_blocks": free,
            "used_blocks": self.num_blocks - free,
            "shared_blocks": sum(1 for c in self.ref_cnt if c > 1),
            "total_refs": sum(self.ref_cnt),
            "cow_copies": self.cow_copies,
            "live_seqs": len(self.tables),
            "tokens": tokens,
            "waste_tokens": waste,
            "cached_blocks": len(self.cache),
            "prompt_tokens": self.prompt_tokens,
            "hit_tokens": self.hit_tokens,
            "evictions": self.evictions,
            "host_blocks": self.host_n,
            "host_free_blocks": len(self.host_free),
            "swapped_seqs": len(self.swapped),
        }

    def free_order(self) -> List[int]:
        return list(self.free)

    def table(self, sid: int) -> List[int]:
        return list(self.tables[sid])
