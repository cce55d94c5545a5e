"""Pins for the oracle's capacity arithmetic and allocator against the pages'
printed values (tests/golden, each file cites its passage)."""

import math

from conftest import load_golden
from oracle import OraclePool, Status
from oracle.capacity import (contiguous_fit, kv_bytes_per_token, paged_fit_skip,
                             paged_fit_stop_at_first_failure, reservation_waste)


def test_kv_bytes_per_token_13b():
    g = load_golden("kv_bytes.json")
    b = kv_bytes_per_token(g["num_layers"], g["num_kv_heads"], g["head_dim"], g["dtype_bytes"])
    assert b == g["bytes_per_token"] == 819200
    seq = b * g["seq_tokens"]
    assert seq == 1_677_721_600
    assert abs(seq / 1e9 - g["seq_gb_approx"]) < 0.1      # "about 1.6 GB"
    w = reservation_waste(g["reserved_tokens"], g["reply_tokens"])
    assert abs(w - g["waste_fraction_approx"]) < 0.01     # "~98%"
    assert w == 2018 / 2048


def test_kv_bytes_per_token_terms():
    # each factor enters linearly: doubling any one doubles the bytes
    base = kv_bytes_per_token(3, 5, 7, 2)
    assert base == 2 * 3 * 5 * 7 * 2
    assert kv_bytes_per_token(6, 5, 7, 2) == 2 * base
    assert kv_bytes_per_token(3, 10, 7, 2) == 2 * base
    assert kv_bytes_per_token(3, 5, 14, 2) == 2 * base
    assert kv_bytes_per_token(3, 5, 7, 1) * 2 == base     # fp8 halves the bytes


def test_contiguous_vs_paged_fit():
    g = load_golden("fragmentation_arithmetic.json")
    assert contiguous_fit(g["pool"], g["block"], g["max_len"]) == g["contiguous_fit"] == 4
    admitted, used = paged_fit_stop_at_first_failure(g["lens"], g["pool"], g["block"])
    assert admitted == g["paged_fit"] == 13
    # by hand: blocks of the first 13 lengths are 3+8+19+4+14+6+12+3+10+5+4+27+3
    assert used == 118
    # the printed loop skips the 256-token sequence (16 blocks > 10 left) but then
    # admits the 90-token one (6 blocks); 110 (7 blocks) no longer fits
    assert paged_fit_skip(g["lens"], g["pool"], g["block"]) == (14, 124)


def test_allocator_admission_matches_arithmetic():
    """The allocator model, admitting until its first NO_BLOCKS, reproduces 13."""
    g = load_golden("fragmentation_arithmetic.json")
    pool = OraclePool(g["pool"], g["block"])
    admitted = 0
    for L in g["lens"]:
        _, s = pool.seq_create()
        st, slots, cow = pool.alloc_append(s, L)
        if st != Status.OK:
            assert st == Status.NO_BLOCKS
            # all-or-nothing: nothing taken for the failed sequence
            assert pool.table(s) == [] and pool.lens[s] == 0
            break
        admitted += 1
    assert admitted == 13
    assert pool.stats()["used_blocks"] == 118 and pool.stats()["free_blocks"] == 10


def test_worked_block_tables():
    g = load_golden("worked_block_tables.json")
    head = [b for s in g["sequences"] for b in s["table"]]
    order = head + [i for i in range(g["pool_blocks"]) if i not in head]
    pool = OraclePool(g["pool_blocks"], g["block_size"], order)
    for s in g["sequences"]:
        _, sid = pool.seq_create()
        st, slots, cow = pool.alloc_append(sid, s["tokens"])
        assert st == Status.OK and cow is None
        assert len(pool.table(sid)) == s["blocks"] == math.ceil(s["tokens"] / 16)
        assert pool.table(sid) == s["table"]
        # the slot of token t is row t % 16 of physical block table[t // 16]
        assert slots[0] == s["table"][0] * 16
        assert slots[17] == s["table"][1] * 16 + 1
        assert slots[-1] == s["table"][-1] * 16 + (s["tokens"] - 1) % 16


def test_internal_waste_bound():
    g = load_golden("kv_bytes.json")
    for L in range(1, 400):
        pool = OraclePool(64, 16)
        _, s = pool.seq_create()
        assert pool.alloc_append(s, L)[0] == Status.OK
        nb = len(pool.table(s))
        assert nb == -(-L // 16)
        waste = pool.stats()["waste_tokens"]
        assert 0 <= waste <= g["max_internal_waste_tokens"]
        assert waste == nb * 16 - L


def test_fit_rules_brute_force_on_small_lists():
    """Both admission rules against a direct simulation of a pool on every
    list of up to 4 lengths from {1, 16, 17, 40} and pools of 0..9 blocks."""
    import itertools
    for k in range(5):
        for lens in itertools.product([1, 16, 17, 40], repeat=k):
            for pool_blocks in range(10):
                free, stop, skip, stopped = pool_blocks, [0, 0], [0, 0], False
                free_skip = pool_blocks
                for L in lens:
                    need = -(-L // 16)
                    if not stopped and need <= free:
                        free -= need
                        stop = [stop[0] + 1, stop[1] + need]
                    else:
                        stopped = True
                    if need <= free_skip:
                        free_skip -= need
                        skip = [skip[0] + 1, skip[1] + need]
                assert paged_fit_stop_at_first_failure(lens, pool_blocks, 16) == tuple(stop)
                assert paged_fit_skip(lens, pool_blocks, 16) == tuple(skip)
