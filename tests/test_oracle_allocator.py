"""Pins for the oracle's block manager: invariants that hold whatever the op
sequence (conservation, reference counts = number of tables holding a block,
FIFO free queue, bounded waste), the pages' fork / copy-on-write behaviour, and
closed-form block counts for the shared-prefix workload."""

import math
import random

import pytest
from hypothesis import given, settings, strategies as st

from oracle import OraclePool, Status


def check_invariants(pool: OraclePool):
    N = pool.num_blocks
    held = {}
    for sid, t in pool.tables.items():
        # one block per started block of 16 tokens
        assert len(t) == -(-pool.lens[sid] // pool.block_size)
        assert len(set(t)) == len(t)
        for b in t:
            held[b] = held.get(b, 0) + 1
    free = pool.free_order()
    assert len(set(free)) == len(free)
    # conservation: a block is either free or held by >= 1 table, never both
    assert set(free).isdisjoint(held)
    assert len(free) + len(held) == N
    for b in range(N):
        assert pool.ref_cnt[b] == held.get(b, 0)
    s = pool.stats()
    assert s["free_blocks"] == len(free)
    assert s["total_refs"] == sum(held.values())
    assert s["shared_blocks"] == sum(1 for c in held.values() if c > 1)
    assert all(0 <= pool.block_size * len(t) - pool.lens[sid] < pool.block_size or pool.lens[sid] == 0
               for sid, t in pool.tables.items())


def test_free_queue_is_fifo():
    pool = OraclePool(8, 4)
    _, a = pool.seq_create()
    _, b = pool.seq_create()
    assert pool.alloc_append(a, 8)[0] == Status.OK      # takes 0, 1
    assert pool.alloc_append(b, 5)[0] == Status.OK      # takes 2, 3
    assert pool.table(a) == [0, 1] and pool.table(b) == [2, 3]
    assert pool.seq_free(a) == Status.OK                # 0, 1 appended at the back
    assert pool.free_order() == [4, 5, 6, 7, 0, 1]
    _, c = pool.seq_create()
    assert pool.alloc_append(c, 9)[1][0] == 4 * 4       # takes from the front
    assert pool.table(c) == [4, 5, 6]


def test_append_one_token_at_a_time_allocates_on_boundaries():
    pool = OraclePool(16, 16)
    _, s = pool.seq_create()
    taken = []
    for t in range(70):
        st_, slots, cow = pool.alloc_append(s, 1)
        assert st_ == Status.OK and cow is None
        if t % 16 == 0:
            taken.append(pool.table(s)[-1])
        assert slots == [pool.table(s)[t // 16] * 16 + t % 16]
    assert pool.table(s) == taken == [0, 1, 2, 3, 4]


def test_fork_shares_and_free_returns_only_at_zero():
    pool = OraclePool(10, 16)
    _, p = pool.seq_create()
    pool.alloc_append(p, 40)                       # blocks 0, 1, 2 (last partial)
    _, c = pool.fork(p)
    assert pool.table(c) == pool.table(p) == [0, 1, 2]
    assert [pool.ref_cnt[b] for b in range(3)] == [2, 2, 2]
    # nothing copied until someone writes into the shared partial block
    assert pool.stats()["used_blocks"] == 3
    st_, slots, cow = pool.alloc_append(c, 1)      # token 40 lands in block 2 (shared) -> CoW
    assert st_ == Status.OK and cow == (2, 3)
    assert pool.table(c) == [0, 1, 3] and pool.ref_cnt[2] == 1 and pool.ref_cnt[3] == 1
    assert slots == [3 * 16 + 8]
    # the last holder writes in place
    st_, slots, cow = pool.alloc_append(p, 1)
    assert cow is None and slots == [2 * 16 + 8]
    assert pool.seq_free(p) == Status.OK
    assert pool.free_order()[-1:] == [2]           # only the private block returned
    assert pool.ref_cnt[0] == 1 and pool.ref_cnt[1] == 1
    assert pool.seq_free(c) == Status.OK
    assert sorted(pool.free_order()) == list(range(10))
    check_invariants(pool)


def test_full_shared_blocks_never_copied():
    pool = OraclePool(10, 16)
    _, p = pool.seq_create()
    pool.alloc_append(p, 32)                       # two full blocks
    _, c = pool.fork(p)
    st_, slots, cow = pool.alloc_append(c, 5)      # new block, no copy
    assert cow is None and pool.table(c) == [0, 1, 2]
    assert pool.ref_cnt[0] == 2 and pool.ref_cnt[2] == 1


@pytest.mark.parametrize("prompt,expect_cow", [(800, 0), (808, 31)])
def test_shared_prompt_counts(prompt, expect_cow):
    """32 sequences share one system prompt (one writer, forked 31 times), then
    each appends its own tail in order 0..31."""
    rng = random.Random(5)
    tails = [rng.randint(1, 1024) for _ in range(32)]
    nblk_prompt = math.ceil(prompt / 16)
    pool = OraclePool(2000, 16)
    _, root = pool.seq_create()
    pool.alloc_append(root, prompt)
    seqs = [root] + [pool.fork(root)[1] for _ in range(31)]
    assert all(pool.ref_cnt[b] == 32 for b in pool.table(root))
    assert pool.stats()["used_blocks"] == nblk_prompt
    for s, t in zip(seqs, tails):
        assert pool.alloc_append(s, t)[0] == Status.OK
    st = pool.stats()
    assert st["cow_copies"] == expect_cow
    partial = prompt % 16
    if partial == 0:
        expect_used = nblk_prompt + sum(math.ceil(t / 16) for t in tails)
    else:
        # 31 copies of the partial block + the original; tails first fill the
        # 16 - partial free rows of their (copied or own) last block
        room = 16 - partial
        expect_used = nblk_prompt + 31 + sum(math.ceil(max(0, t - room) / 16) for t in tails)
    assert st["used_blocks"] == expect_used
    # the full prompt blocks are read by all 32, stored once
    full = prompt // 16
    assert all(pool.ref_cnt[b] == 32 for b in pool.table(root)[:full])
    check_invariants(pool)


def test_all_or_nothing():
    pool = OraclePool(4, 16)
    _, a = pool.seq_create()
    assert pool.alloc_append(a, 40)[0] == Status.OK     # 3 blocks
    before = (pool.free_order(), list(pool.ref_cnt), pool.table(a), pool.lens[a])
    st_, slots, cow = pool.alloc_append(a, 40)          # would need 3 more (5 total)
    assert st_ == Status.NO_BLOCKS and slots == [] and cow is None
    assert before == (pool.free_order(), list(pool.ref_cnt), pool.table(a), pool.lens[a])
    # CoW needs a block too: with no free block, the shared write fails cleanly
    _, c = pool.fork(a)
    assert pool.alloc_append(c, 1)[0] == Status.OK      # takes the last free block (CoW)
    _, d = pool.fork(c)
    assert pool.alloc_append(d, 1)[0] == Status.NO_BLOCKS
    assert pool.alloc_append(99, 1)[0] == Status.BAD_SEQ
    assert pool.seq_free(99) == Status.BAD_SEQ
    assert pool.alloc_append(a, -1)[0] == Status.BAD_ARG
    check_invariants(pool)


def test_block_tables_export():
    pool = OraclePool(8, 16, [7, 6, 5, 4, 3, 2, 1, 0])
    _, a = pool.seq_create()
    _, b = pool.seq_create()
    pool.alloc_append(a, 20)
    pool.alloc_append(b, 3)
    st_, rows, lens = pool.block_tables([b, a], 3)
    assert st_ == Status.OK and rows == [[5, -1, -1], [7, 6, -1]] and lens == [3, 20]
    assert pool.block_tables([a], 1)[0] == Status.CAPACITY
    assert pool.block_tables([42], 4)[0] == Status.BAD_SEQ


ops = st.lists(st.tuples(st.sampled_from(["new", "append", "fork", "free"]),
                         st.integers(0, 7), st.integers(0, 40)), min_size=1, max_size=60)


@settings(max_examples=150, deadline=None)
@given(ops=ops, n=st.integers(1, 12), bs=st.sampled_from([1, 2, 4, 16]), seed=st.integers(0, 99))
def test_random_ops_keep_invariants(ops, n, bs, seed):
    order = list(range(n))
    random.Random(seed).shuffle(order)
    pool = OraclePool(n, bs, order)
    live = []
    for op, i, k in ops:
        if op == "new" or not live:
            live.append(pool.seq_create()[1])
        elif op == "append":
            s = live[i % len(live)]
            before_free = len(pool.free)
            st_, slots, cow = pool.alloc_append(s, k)
            if st_ == Status.OK:
                # slots are distinct and land in the sequence's own blocks
                assert len(set(slots)) == len(slots) == k
                assert all(sl // bs in pool.table(s) for sl in slots)
            else:
                assert st_ == Status.NO_BLOCKS and len(pool.free) == before_free
        elif op == "fork":
            live.append(pool.fork(live[i % len(live)])[1])
        else:
            s = live.pop(i % len(live))
            assert pool.seq_free(s) == Status.OK
        check_invariants(pool)
    for s in live:
        pool.seq_free(s)
    assert sorted(pool.free_order()) == list(range(n))
    assert sum(pool.ref_cnt) == 0
