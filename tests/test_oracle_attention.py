"""Pins for the oracle's attention: closed forms, an independent library routine
(torch's scaled_dot_product_attention in float64 on the CPU), the pages'
"paged equals dense" statement, invariance under physical placement, and the
chunked-prefill identities."""

import numpy as np
import pytest
import torch

import workloads
from oracle import (OracleCache, OraclePool, Status, attention_fp64, dense_decode,
                    dense_prefill_row, gather_paged, paged_decode, paged_prefill)


def test_single_key_returns_its_value():
    rng = np.random.default_rng(0)
    q, K, V = rng.standard_normal(8), rng.standard_normal((1, 8)), rng.standard_normal((1, 8))
    assert np.array_equal(attention_fp64(q, K, V, 0.3), V[0])


def test_equal_scores_average_values():
    rng = np.random.default_rng(1)
    V = rng.standard_normal((7, 5))
    out = attention_fp64(rng.standard_normal(5), np.zeros((7, 5)), V, 1.0)
    assert np.allclose(out, V.mean(axis=0), rtol=0, atol=1e-15)
    # scale 0 flattens any scores to the mean as well
    out0 = attention_fp64(rng.standard_normal(5), rng.standard_normal((7, 5)), V, 0.0)
    assert np.allclose(out0, V.mean(axis=0), rtol=0, atol=1e-15)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(2)
    K = rng.standard_normal((9, 4)) * 0.01
    K[5] = [100.0, 0, 0, 0]
    V = rng.standard_normal((9, 4))
    out = attention_fp64(np.array([100.0, 0, 0, 0]), K, V, 1.0)
    assert np.array_equal(out, V[5])


def test_two_keys_logistic_form():
    # with two keys the weights are logistic in the score difference
    q = np.array([0.5, -1.0, 2.0])
    K = np.array([[1.0, 0.0, 0.5], [-0.5, 1.0, 0.0]])
    V = np.array([[1.0, 2.0, 3.0], [-3.0, 0.0, 1.0]])
    scale = 0.7
    d = scale * ((0.5 * 1.0 + 2.0 * 0.5) - (0.5 * -0.5 + -1.0 * 1.0))   # s0 - s1, by hand
    w0 = 1.0 / (1.0 + np.exp(-d))
    expect = w0 * V[0] + (1.0 - w0) * V[1]
    assert np.allclose(attention_fp64(q, K, V, scale), expect, rtol=0, atol=1e-15)


def test_matches_torch_sdpa_float64():
    rng = np.random.default_rng(3)
    for L, D in [(1, 4), (17, 64), (300, 128)]:
        q = rng.standard_normal(D)
        K = rng.standard_normal((L, D))
        V = rng.standard_normal((L, D))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, None, None, :], torch.from_numpy(K)[None, None],
            torch.from_numpy(V)[None, None], scale=1.0 / np.sqrt(D))[0, 0, 0].numpy()
        assert np.allclose(attention_fp64(q, K, V, 1.0 / np.sqrt(D)), ref, rtol=1e-12, atol=1e-12)


def _paged_setup(w, fp8=False, seqs=None):
    pool = OraclePool(w.num_blocks, 16, w.init_free_order)
    cache = OracleCache(w.num_blocks, w.num_kv_heads, w.head_dim, fp8=fp8)
    tables, Ks, Vs = [], [], []
    for b in (seqs if seqs is not None else range(w.batch)):
        _, s = pool.seq_create()
        k, v = w.kv(b)
        st, slots, cow = pool.alloc_append(s, int(w.lens[b]))
        assert st == Status.OK and cow is None
        cache.write(slots, k, v)
        tables.append(pool.table(s))
        Ks.append(k)
        Vs.append(v)
    return pool, cache, tables, Ks, Vs


def test_paged_equals_dense_bitwise():
    """The pages: paging changes where K/V live, not the attention result."""
    for w in (workloads.tiny_decode(), workloads.tiny_decode_worked_example(),
              workloads.custom_decode(11, [1, 15, 16, 17, 33, 64], 4, 2, 64)):
        pool, cache, tables, Ks, Vs = _paged_setup(w)
        got = paged_decode(cache, tables, w.lens, w.q, w.scale)
        ref = dense_decode(w.q, Ks, Vs, w.scale)
        assert np.array_equal(got, ref)


def test_worked_example_tables_reach_the_kernel_inputs():
    w = workloads.tiny_decode_worked_example()
    _, cache, tables, Ks, _ = _paged_setup(w)
    assert tables == [[10, 25], [3, 7, 12, 18]]
    # token 17 of the 50-token sequence sits in row 1 of physical block 7
    assert np.array_equal(cache.k[7, :, 1, :], Ks[1][17])
    assert np.array_equal(gather_paged(cache.values("k"), tables[1], 50, 2), Ks[1][:, 2, :].astype(np.float64))


def test_physical_placement_does_not_change_output():
    w1 = workloads.custom_decode(21, [5, 40, 77], 2, 2, 64, shuffle=False)
    w2 = workloads.custom_decode(21, [5, 40, 77], 2, 2, 64, shuffle=True)
    assert w1.init_free_order is None and w2.init_free_order is not None
    _, c1, t1, _, _ = _paged_setup(w1)
    _, c2, t2, _, _ = _paged_setup(w2)
    assert t1 != t2
    assert np.array_equal(paged_decode(c1, t1, w1.lens, w1.q, w1.scale),
                          paged_decode(c2, t2, w2.lens, w2.q, w2.scale))


def test_grouped_heads_read_their_kv_head():
    w = workloads.custom_decode(31, [9, 20], 6, 2, 64)
    _, cache, tables, Ks, Vs = _paged_setup(w)
    out = paged_decode(cache, tables, w.lens, w.q, w.scale)
    for b in range(2):
        for h in range(6):
            kh = h // 3
            ref = attention_fp64(w.q[b, h], Ks[b][:, kh], Vs[b][:, kh], w.scale)
            assert np.array_equal(out[b, h], ref)


def test_fp8_cache_stores_codes_and_dequantises():
    w = workloads.custom_decode(41, [20], 2, 2, 64)
    k, v = w.kv(0)
    ks, vs = workloads.fp8_scale(k), workloads.fp8_scale(v)
    pool = OraclePool(w.num_blocks, 16)
    cache = OracleCache(w.num_blocks, 2, 64, fp8=True, k_scale=ks, v_scale=vs)
    _, s = pool.seq_create()
    _, slots, _ = pool.alloc_append(s, 20)
    cache.write(slots, k, v)
    assert cache.k.dtype == np.uint8
    # each stored value is within half an e4m3 step (2^-4 relative) of the source
    vals = gather_paged(cache.values("k"), pool.table(s), 20, 1)
    src = k[:, 1].astype(np.float64)
    big = np.abs(src) > 64 * ks          # normal range of the scaled values
    assert np.all(np.abs(vals - src)[big] <= np.abs(src)[big] * 2.0 ** -4 * 1.0000001)


def _prefill_setup(w):
    pool = OraclePool(w.num_blocks, 16, w.init_free_order)
    cache = OracleCache(w.num_blocks, w.num_kv_heads, w.head_dim)
    tables = []
    for b in range(w.batch):
        _, s = pool.seq_create()
        k, v = w.kv(b)
        P = int(w.prior[b])
        st, slots, _ = pool.alloc_append(s, P)            # prior context
        cache.write(slots, k[:P], v[:P])
        st, slots, _ = pool.alloc_append(s, int(w.chunk[b]))   # the chunk
        assert st == Status.OK
        cache.write(slots, k[P:], v[P:])
        tables.append(pool.table(s))
    return cache, tables


def test_prefill_zero_prior_is_causal_sdpa():
    w = workloads.custom_prefill(51, [0], [40], 2, 2, 64)
    cache, tables = _prefill_setup(w)
    out = paged_prefill(cache, tables, w.prior, w.chunk, w.q, w.scale)
    k, v = w.kv(0)
    qt = torch.from_numpy(w.q.astype(np.float64)).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                           scale=w.scale)[0].permute(1, 0, 2).numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_prefill_with_prior_is_masked_sdpa():
    w = workloads.custom_prefill(52, [37], [21], 2, 2, 64)
    cache, tables = _prefill_setup(w)
    out = paged_prefill(cache, tables, w.prior, w.chunk, w.q, w.scale)
    k, v = w.kv(0)
    P, C = 37, 21
    mask = np.zeros((C, P + C), dtype=bool)
    for i in range(C):
        mask[i, :P + i + 1] = True
    qt = torch.from_numpy(w.q.astype(np.float64)).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.from_numpy(mask), scale=w.scale)[0].permute(1, 0, 2).numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_prefill_single_row_is_decode():
    w = workloads.custom_prefill(53, [45, 0], [1, 1], 2, 2, 64)
    cache, tables = _prefill_setup(w)
    out = paged_prefill(cache, tables, w.prior, w.chunk, w.q, w.scale)
    dec = paged_decode(cache, tables, w.prior + 1, w.q.reshape(2, 2, 64), w.scale)
    assert np.array_equal(out.reshape(2, 2, 64), dec)


def test_prefill_chunk_split_equivalence():
    """One 48-row chunk == two 24-row chunks run back to back (same keys seen)."""
    w = workloads.custom_prefill(54, [19], [48], 2, 2, 64)
    cache, tables = _prefill_setup(w)
    whole = paged_prefill(cache, tables, w.prior, w.chunk, w.q, w.scale)
    first = paged_prefill(cache, tables, [19], [24], w.q[:24], w.scale)
    second = paged_prefill(cache, tables, [19 + 24], [24], w.q[24:], w.scale)
    assert np.allclose(whole, np.concatenate([first, second]), rtol=1e-13, atol=1e-13)
    k, v = w.kv(0)
    row = dense_prefill_row(w.q[30, 1], k[:, 1], v[:, 1], 19 + 30, w.scale)
    assert np.array_equal(row, whole[30, 1])


def test_all_heads_form_matches_sdpa_and_the_single_head_form():
    """attention_heads_fp64 against torch's float64 SDPA (grouped heads expanded
    by hand) and against attention_fp64 head by head."""
    from oracle import attention_heads_fp64
    rng = np.random.default_rng(31)
    for L, Hq, Hkv, D in [(1, 4, 4, 8), (37, 8, 2, 64), (300, 6, 3, 128), (0, 2, 2, 4)]:
        q = rng.standard_normal((Hq, D))
        K = rng.standard_normal((L, Hkv, D))
        V = rng.standard_normal((L, Hkv, D))
        got = attention_heads_fp64(q, K, V, 0.2)
        assert got.shape == (Hq, D)
        if L == 0:
            assert np.all(got == 0)
            continue
        g = Hq // Hkv
        Ke = torch.from_numpy(np.repeat(K, g, axis=1).transpose(1, 0, 2).copy())   # [Hq][L][D]
        Ve = torch.from_numpy(np.repeat(V, g, axis=1).transpose(1, 0, 2).copy())
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, :, None, :], Ke[None], Ve[None], scale=0.2)[0, :, 0].numpy()
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
        for h in range(Hq):
            one = attention_fp64(q[h], K[:, h // g], V[:, h // g], 0.2)
            assert np.allclose(got[h], one, rtol=1e-13, atol=1e-13)


def test_causal_chunk_matches_masked_sdpa_and_row_form():
    """causal_chunk_fp64 against torch SDPA with an explicit boolean mask
    (row i sees keys 0..P+i), against dense_prefill_row row by row, and with
    P = 0 against SDPA's own causal flag."""
    from oracle import causal_chunk_fp64
    rng = np.random.default_rng(32)
    for P, C, D in [(0, 1, 8), (0, 40, 16), (33, 17, 64), (200, 129, 128)]:
        Q = rng.standard_normal((C, D))
        K = rng.standard_normal((P + C, D))
        V = rng.standard_normal((P + C, D))
        got = causal_chunk_fp64(Q, K, V, P, 0.3)
        mask = torch.from_numpy(np.arange(P + C)[None, :] <= (P + np.arange(C))[:, None])
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q)[None, None], torch.from_numpy(K)[None, None],
            torch.from_numpy(V)[None, None], attn_mask=mask, scale=0.3)[0, 0].numpy()
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
        for i in (0, C // 2, C - 1):
            assert np.allclose(got[i], dense_prefill_row(Q[i], K, V, P + i, 0.3), rtol=1e-13, atol=1e-13)
        if P == 0:
            causal = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(Q)[None, None], torch.from_numpy(K)[None, None],
                torch.from_numpy(V)[None, None], is_causal=True, scale=0.3)[0, 0].numpy()
            assert np.allclose(got, causal, rtol=1e-12, atol=1e-12)
        # the last row sees every key: plain attention
        assert np.allclose(got[-1], attention_fp64(Q[-1], K, V, 0.3), rtol=1e-13, atol=1e-13)


def test_causal_chunk_planted_off_by_one_is_caught():
    """A mask that lets row i see key P+i+1 (or hides key P+i) changes the
    rows the SDPA comparison checks."""
    from oracle import causal_chunk_fp64
    rng = np.random.default_rng(33)
    P, C, D = 5, 9, 8
    Q, K, V = rng.standard_normal((C, D)), rng.standard_normal((P + C, D)), rng.standard_normal((P + C, D))
    good = causal_chunk_fp64(Q, K, V, P, 0.3)
    late = causal_chunk_fp64(Q, K, V, P + 1, 0.3)[:-1]
    early = causal_chunk_fp64(Q, K, V, P - 1, 0.3)
    assert not np.allclose(good[:-1], late, rtol=1e-6, atol=1e-6)
    assert not np.allclose(good, early, rtol=1e-6, atol=1e-6)
