"""Pins of the oracle's swap model ([p3] "What happens when the GPU runs out of
KV blocks?": copy the evicted blocks to CPU RAM over PCIe, copy them back when
the sequence is rescheduled).  Worked cases written out by hand, and a
shadow-content property: after any interleaving of swaps, a swapped-in
sequence's blocks hold what they held before it was swapped out."""

import random

import pytest

from oracle import OraclePool, Status

BS = 16


def test_swap_out_and_in_worked_example():
    p = OraclePool(6, BS)                  # device queue 0..5
    p.set_swap_space(4)                    # host queue 0..3
    _, a = p.seq_create()
    p.alloc_append(a, 40)                  # blocks 0, 1, 2
    _, b = p.seq_create()
    p.alloc_append(b, 16)                  # block 3
    st, pairs = p.swap_out(a)
    assert st == Status.OK and pairs == [(0, 0), (1, 1), (2, 2)]
    assert p.free_order() == [4, 5, 0, 1, 2] and p.table(a) == [0, 1, 2]   # host ids now
    s = p.stats()
    assert (s["tokens"], s["swapped_seqs"], s["host_free_blocks"], s["waste_tokens"]) == (16, 1, 1, 0)
    p.alloc_append(b, 17)                  # b grows into 4 and 5 (block 4 is not full: 2 blocks)
    assert p.table(b) == [3, 4, 5]
    st, pairs = p.swap_in(a)
    assert st == Status.OK and pairs == [(0, 0), (1, 1), (2, 2)]
    assert p.table(a) == [0, 1, 2] and list(p.host_free) == [3, 0, 1, 2]
    assert p.stats()["tokens"] == 40 + 33


def test_swapping_a_forked_sequence_keeps_the_sibling():
    p = OraclePool(4, BS)
    p.set_swap_space(2)
    _, a = p.seq_create()
    p.alloc_append(a, 20)                  # blocks 0, 1
    _, c = p.fork(a)
    st, pairs = p.swap_out(c)
    assert st == Status.OK and pairs == [(0, 0), (1, 1)]
    assert p.ref_cnt[:2] == [1, 1] and p.free_order() == [2, 3]
    st, pairs = p.swap_in(c)               # c gets fresh device copies
    assert pairs == [(0, 2), (1, 3)] and p.table(c) == [2, 3]


def test_shortages_and_refusals_leave_state_unchanged():
    p = OraclePool(3, BS)
    p.set_swap_space(1)
    _, a = p.seq_create()
    p.alloc_append(a, 20)
    snap = (p.free_order(), list(p.ref_cnt), p.stats(), p.table(a))
    assert p.swap_out(a) == (Status.NO_BLOCKS, [])           # 2 blocks, 1 host block
    assert p.swap_in(a) == (Status.BAD_ARG, [])              # not swapped out
    assert snap == (p.free_order(), list(p.ref_cnt), p.stats(), p.table(a))
    p.set_swap_space(2)
    assert p.swap_out(a)[0] == Status.OK
    assert p.set_swap_space(5) == Status.BAD_ARG              # while swapped
    assert p.alloc_append(a, 1)[0] == Status.BAD_ARG
    assert p.fork(a)[0] == Status.BAD_ARG
    assert p.cache_commit(a)[0] == Status.BAD_ARG
    assert p.block_tables([a], 4)[0] == Status.BAD_ARG
    _, b = p.seq_create()
    p.alloc_append(b, 48)                                     # takes all 3 device blocks
    assert p.swap_in(a) == (Status.NO_BLOCKS, [])
    p.seq_free(a)                                             # host blocks go back
    assert list(p.host_free) == [0, 1] and p.stats()["swapped_seqs"] == 0


@pytest.mark.parametrize("seed", range(20))
def test_swapped_in_blocks_hold_what_was_swapped_out(seed):
    r = random.Random(seed)
    p = OraclePool(12, BS, init_free_order=r.sample(range(12), 12))
    p.set_swap_space(10)
    dev = {}                         # device block -> content tag
    host = {}                        # host block -> content tag
    expect = {}                      # sequence -> list of content tags per logical block
    live = []
    tag = 0
    for _ in range(150):
        op = r.random()
        if op < 0.3:
            _, s = p.seq_create()
            st, _, _ = p.alloc_append(s, r.randrange(1, 50))
            if st != Status.OK:
                p.seq_free(s)
                continue
            tags = []
            for b in p.table(s):
                tag += 1
                dev[b] = tag
                tags.append(tag)
            expect[s] = tags
            live.append(s)
        elif op < 0.45 and live:
            s = r.choice(live)
            if s in p.swapped:
                continue
            old = len(p.table(s))
            st, _, cow = p.alloc_append(s, r.randrange(1, 20))
            if st == Status.OK:
                if cow:
                    dev[cow[1]] = dev[cow[0]]
                for b in p.table(s)[old:]:
                    tag += 1
                    dev[b] = tag
                expect[s] = [dev[b] for b in p.table(s)]
        elif op < 0.6 and live:
            s = r.choice(live)
            if s in p.swapped:
                continue
            st, c = p.fork(s)
            live.append(c)
            expect[c] = list(expect[s])
        elif op < 0.75 and live:
            s = r.choice(live)
            if s in p.swapped:
                st, pairs = p.swap_in(s)
                for h, b in pairs:
                    dev[b] = host[h]
            else:
                st, pairs = p.swap_out(s)
                for b, h in pairs:
                    host[h] = dev[b]
        elif live:
            s = live.pop(r.randrange(len(live)))
            p.seq_free(s)
            del expect[s]
        for s in live:
            if s not in p.swapped:
                assert [dev[b] for b in p.table(s)] == expect[s]
            else:
                assert [host[h] for h in p.table(s)] == expect[s]
