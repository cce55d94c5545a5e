"""Pins of the oracle's prefix-cache model ([p2] "Deep dive", prefix-caching
bullet; [p1] "Automatic Prefix Caching (APC)"): worked cases written out from
the pages' description, and a shadow-content property -- a reused block always
holds exactly the K/V of the prefix it is reused for -- under random traffic."""

import random

import pytest

from oracle import OraclePool, Status

BS = 16


def prompt(seed, n, vocab=1000):
    r = random.Random(seed)
    return [r.randrange(vocab) for _ in range(n)]


def test_identical_prompts_share_full_blocks_only():
    p = OraclePool(16, BS)
    toks = prompt(1, 40)
    _, a = p.seq_create()
    st, slots, hit = p.alloc_prompt(a, toks)
    assert (st, hit, len(slots)) == (Status.OK, 0, 40)
    assert p.cache_commit(a) == (Status.OK, 2)          # blocks 0-15, 16-31; 32-39 is partial
    _, b = p.seq_create()
    st, slots, hit = p.alloc_prompt(b, toks)
    assert (st, hit, len(slots)) == (Status.OK, 32, 8)  # the partial block is never shared
    assert p.tables[b][:2] == p.tables[a][:2] and p.tables[b][2] != p.tables[a][2]
    assert [p.ref_cnt[x] for x in p.tables[a]] == [2, 2, 1]
    s = p.stats()
    assert (s["prompt_tokens"], s["hit_tokens"], s["cached_blocks"]) == (80, 32, 2)
    assert slots == [p.tables[b][2] * BS + i for i in range(8)]


def test_uncommitted_blocks_are_not_reused():
    p = OraclePool(8, BS)
    toks = prompt(2, 48)
    _, a = p.seq_create()
    p.alloc_prompt(a, toks)
    _, b = p.seq_create()
    assert p.alloc_prompt(b, toks)[2] == 0


def test_last_token_is_always_computed():
    p = OraclePool(8, BS)
    toks = prompt(3, 32)
    _, a = p.seq_create()
    p.alloc_prompt(a, toks)
    p.cache_commit(a)
    _, b = p.seq_create()
    assert p.alloc_prompt(b, toks)[2] == 16          # 2 full blocks cached, only 1 reused
    _, c = p.seq_create()
    assert p.alloc_prompt(c, toks[:16])[2] == 0       # a one-block prompt computes its block
    _, d = p.seq_create()
    assert p.alloc_prompt(d, toks[:17])[2] == 16


def test_divergence_stops_the_match():
    p = OraclePool(16, BS)
    toks = prompt(4, 64)
    _, a = p.seq_create()
    p.alloc_prompt(a, toks)
    p.cache_commit(a)
    other = list(toks)
    other[20] += 1                                    # differs inside block 1
    _, b = p.seq_create()
    assert p.alloc_prompt(b, other)[2] == 16
    other2 = list(toks)
    other2[3] += 1                                    # block 0 differs: later equal blocks do not match
    _, c = p.seq_create()
    assert p.alloc_prompt(c, other2)[2] == 0


def test_multi_turn_dialogue_reuses_the_history():
    """[p1] APC motivation: each turn starts with the conversation so far."""
    p = OraclePool(64, BS)
    history = prompt(5, 100)
    _, s1 = p.seq_create()
    p.alloc_prompt(s1, history)
    p.cache_commit(s1)
    reply = prompt(6, 30)
    p.append_tokens(s1, reply)                        # generated tokens, ids known
    p.cache_commit(s1)                                # blocks through token 127 are full
    p.seq_free(s1)
    turn2 = history + reply + prompt(7, 25)
    _, s2 = p.seq_create()
    st, slots, hit = p.alloc_prompt(s2, turn2)
    assert st == Status.OK and hit == 128 and len(slots) == 155 - 128


def test_freed_blocks_stay_cached_until_the_queue_hands_them_out():
    p = OraclePool(4, BS, init_free_order=[0, 1, 2, 3])
    toks = prompt(8, 33)
    _, a = p.seq_create()
    p.alloc_prompt(a, toks)                           # blocks 0, 1, 2
    p.cache_commit(a)                                 # 0 and 1 cached
    p.seq_free(a)
    assert p.free_order() == [3, 0, 1, 2]
    _, b = p.seq_create()
    p.alloc_prompt(b, prompt(9, 20))                  # takes 3 and 0: block 0 is evicted
    assert p.stats()["evictions"] == 1 and p.stats()["cached_blocks"] == 1
    _, c = p.seq_create()
    assert p.alloc_prompt(c, toks)[2] == 0            # its first block is gone, so nothing matches


def test_a_hit_takes_the_block_out_of_the_middle_of_the_queue():
    p = OraclePool(6, BS, init_free_order=[5, 4, 3, 2, 1, 0])
    toks = prompt(10, 40)
    _, a = p.seq_create()
    p.alloc_prompt(a, toks)                           # blocks 5, 4, 3
    p.cache_commit(a)
    p.seq_free(a)
    assert p.free_order() == [2, 1, 0, 5, 4, 3]
    _, b = p.seq_create()
    st, slots, hit = p.alloc_prompt(b, toks[:20])     # reuses 5 (middle of the queue), takes 2
    assert (st, hit) == (Status.OK, 16)
    assert p.tables[b] == [5, 2] and p.free_order() == [1, 0, 4, 3]


def test_no_blocks_counts_reused_free_blocks():
    p = OraclePool(3, BS)
    toks = prompt(11, 33)
    _, a = p.seq_create()
    p.alloc_prompt(a, toks)
    p.cache_commit(a)
    p.seq_free(a)
    _, b = p.seq_create()
    before = (p.free_order(), p.stats())
    # 3 blocks needed: 2 reused (both in the queue) + 1 new; the queue holds 3
    assert p.alloc_prompt(b, toks)[0] == Status.OK
    _, c = p.seq_create()
    st, _, _ = p.alloc_prompt(c, toks + [1])          # 2 reused (in use) + 1 new: none left
    assert st == Status.NO_BLOCKS
    assert before[0] != p.free_order()                # (b's admission changed it)


def test_errors_leave_the_cache_unchanged():
    p = OraclePool(4, BS)
    _, a = p.seq_create()
    p.alloc_prompt(a, prompt(12, 20))
    p.cache_commit(a)
    _, b = p.seq_create()
    snap = (dict(p.cache), p.free_order(), list(p.ref_cnt), p.stats())
    assert p.alloc_prompt(a, prompt(12, 20))[0] == Status.BAD_ARG    # not empty
    assert p.alloc_prompt(99, [1])[0] == Status.BAD_SEQ
    assert p.alloc_prompt(b, prompt(13, 100))[0] == Status.NO_BLOCKS
    assert snap == (dict(p.cache), p.free_order(), list(p.ref_cnt), p.stats())


@pytest.mark.parametrize("seed", range(25))
def test_reused_blocks_hold_exactly_their_prefix(seed):
    """Shadow model: every block remembers the token ids written into it; a
    reused block must hold the reusing prompt's tokens for that block, and the
    hit count must equal the longest run of cached, un-evicted full blocks."""
    r = random.Random(seed)
    p = OraclePool(40, BS, init_free_order=r.sample(range(40), 40))
    content = {}                       # block -> prefix tuple through its end, when written
    bases = [prompt(1000 + seed * 7 + k, 70, vocab=5) for k in range(3)]
    live = []
    for _ in range(120):
        op = r.random()
        if op < 0.45:
            base = r.choice(bases)
            toks = base[:r.randrange(1, 70)] + prompt(r.randrange(10**6), r.randrange(0, 20), vocab=5)
            _, s = p.seq_create()
            expect_hit = 0
            for i in range((len(toks) - 1) // BS):
                if tuple(toks[:BS * (i + 1)]) in p.cache:
                    expect_hit += BS
                else:
                    break
            st, slots, hit = p.alloc_prompt(s, toks)
            if st != Status.OK:
                p.seq_free(s)
                continue
            assert hit == expect_hit
            for i, b in enumerate(p.tables[s]):
                pre = tuple(toks[:min(len(toks), BS * (i + 1))])
                if BS * i < hit:
                    assert content[b] == pre          # reused: the K/V is this prefix's
                else:
                    content[b] = pre                  # written fresh
            if r.random() < 0.8:
                p.cache_commit(s)
            live.append(s)
        elif op < 0.65 and live:
            s = r.choice(live)
            n = r.randrange(1, 20)
            old_len = p.lens[s]
            add = prompt(r.randrange(10**6), n, vocab=5)
            st, slots, cow = p.append_tokens(s, add)
            if st == Status.OK:
                toks = p.tokens[s]
                for i in range(old_len // BS, len(p.tables[s])):
                    content[p.tables[s][i]] = tuple(toks[:min(len(toks), BS * (i + 1))])
                p.cache_commit(s)
        elif live:
            s = live.pop(r.randrange(len(live)))
            p.seq_free(s)
        # cached blocks are full and their cache key is what they hold
        for key, b in p.cache.items():
            assert len(key) % BS == 0 and content[b] == key and p.block_key[b] == key
