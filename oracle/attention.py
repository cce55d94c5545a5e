"""Paged attention in float64 (test infrastructure only; see ``oracle/__init__``).

What is computed follows [p1] "vLLM PagedAttention Deep Dive", section
"PagedAttention Mechanism": for each query, look the sequence's physical blocks
up in its block table, gather the K and V rows from those (non-contiguous)
blocks, then run ordinary softmax attention over the gathered rows.  [p2]
"PagedAttention: KV cache as virtual memory" ("Direct answer" and the
follow-ups) and [p3] "PagedAttention: Why Static Batching Wastes Your KV
Cache" state that the result is the same as attention over the tokens stored
contiguously; ``dense_decode`` is that contiguous computation and the tests
assert the two agree bit for bit.

Chunked prefill follows [p1], section "Mechanics of Chunked Prefill": a chunk's
K/V are added to the paged cache, and each chunk query attends to the whole
cached prior context plus the chunk tokens up to and including its own
position (causal inside the chunk).

Cache layout modelled here (the pages do not fix one): K and V each
``[num_blocks][num_kv_heads][block_size][head_dim]``; token ``t`` of a sequence
lives at physical block ``table[t // block_size]``, row ``t % block_size``.
A flat slot is ``block * block_size + row``.

Query head ``h`` reads KV head ``h // (Hq // Hkv)`` (grouped heads; with
``Hq == Hkv`` this is plain multi-head attention as on the pages).
"""

from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np

from .fp8 import e4m3_dequantize, e4m3_quantize


def attention_fp64(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * K q) V for one query, all in float64.

    ``q`` [D], ``K``/``V`` [L][D].  L = 0 returns zeros (no keys to attend to).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if K.shape[0] == 0:
        return np.zeros(V.shape[1], dtype=np.float64)
    s = (K @ q) * float(scale)
    s = s - s.max()
    p = np.exp(s)
    return (p @ V) / p.sum()


def attention_heads_fp64(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """``attention_fp64`` for every query head of one sequence at once.

    ``q`` [Hq][D]; ``K``/``V`` [L][Hkv][D], the sequence's rows in token order;
    query head ``h`` reads KV head ``h // (Hq // Hkv)``.  Returns [Hq][D]
    float64.  The same definition as ``attention_fp64``, with the per-head
    products written as two batched matrix products (a library step).
    """
    q = np.asarray(q, dtype=np.float64)
    Hq, D = q.shape
    L, Hkv = K.shape[0], K.shape[1]
    if L == 0:
        return np.zeros((Hq, D), dtype=np.float64)
    kv = np.arange(Hq) // (Hq // Hkv)
    Kh = np.asarray(K, dtype=np.float64)[:, kv, :].transpose(1, 0, 2)   # [Hq][L][D]
    Vh = np.asarray(V, dtype=np.float64)[:, kv, :].transpose(1, 0, 2)
    s = np.matmul(Kh, q[:, :, None])[:, :, 0] * float(scale)           # [Hq][L]
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return np.matmul(p[:, None, :], Vh)[:, 0, :] / p.sum(axis=1)[:, None]


def causal_chunk_fp64(Q: np.ndarray, K: np.ndarray, V: np.ndarray, prior: int,
                      scale: float) -> np.ndarray:
    """One head of a chunk: row ``i`` of ``Q`` [C][D] sits at position
    ``prior + i`` and attends to keys ``0 .. prior + i`` of ``K``/``V``
    [prior + C][D] ([p1] "Mechanics of Chunked Prefill": full attention to the
    cached prior context, causal inside the chunk).  All rows at once: the
    scores of keys past a row's position are set to minus infinity before the
    softmax, so they get weight zero.  Returns [C][D] float64.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    C, L = Q.shape[0], K.shape[0]
    if C == 0:
        return np.zeros((0, V.shape[1]), dtype=np.float64)
    s = (Q @ K.T) * float(scale)                                        # [C][L]
    visible = np.arange(L)[None, :] <= (int(prior) + np.arange(C))[:, None]
    s = np.where(visible, s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ V) / p.sum(axis=1, keepdims=True)


class OracleCache:
    """Paged K/V arrays plus the two writes the path performs on them."""

    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int,
                 block_size: int = 16, fp8: bool = False,
                 k_scale: float = 1.0, v_scale: float = 1.0):
        dt = np.uint8 if fp8 else np.float16
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        self.k = np.zeros(shape, dtype=dt)
        self.v = np.zeros(shape, dtype=dt)
        self.block_size = block_size
        self.fp8 = fp8
        self.k_scale = float(np.float32(k_scale))
        self.v_scale = float(np.float32(v_scale))

    def write(self, slots: Sequence[int], k_new: np.ndarray, v_new: np.ndarray) -> None:
        """Scatter token ``i``'s rows ``k_new[i][h]`` to slot ``slots[i]``.

        Negative slots are padding and are skipped.  FP8 caches store the
        quantised codes.
        """
        bs = self.block_size
        if self.fp8:
            k_new = e4m3_quantize(k_new, self.k_scale)
            v_new = e4m3_quantize(v_new, self.v_scale)
        for i, s in enumerate(slots):
            s = int(s)
            if s < 0:
                continue
            self.k[s // bs, :, s % bs, :] = k_new[i]
            self.v[s // bs, :, s % bs, :] = v_new[i]

    def copy_block(self, src: int, dst: int) -> None:
        """Copy-on-write: duplicate one whole physical block ([p3], section "How
        does copy-on-write eliminate duplicate prompt KV cache?")."""
        self.k[dst] = self.k[src]
        self.v[dst] = self.v[src]

    def values(self, which: str) -> np.ndarray:
        """Cache contents as float64 (dequantised for FP8)."""
        arr = self.k if which == "k" else self.v
        if self.fp8:
            return e4m3_dequantize(arr, self.k_scale if which == "k" else self.v_scale)
        return arr.astype(np.float64)


def gather_paged(cache_vals: np.ndarray, table: Sequence[int], length: int, kv_head: int,
                 block_size: int = 16) -> np.ndarray:
    """Rows 0..length-1 of one KV head of one sequence, looked up token by token
    through the block table (logical block ``t // bs`` -> physical block)."""
    rows = []
    for t in range(length):
        phys = int(table[t // block_size])
        rows.append(cache_vals[phys, kv_head, t % block_size, :])
    if not rows:
        return np.zeros((0, cache_vals.shape[-1]), dtype=np.float64)
    return np.stack(rows).astype(np.float64)


def paged_decode(cache: OracleCache, tables: Sequence[Sequence[int]], lens: Sequence[int],
                 q: np.ndarray, scale: float, only: Optional[Sequence[tuple]] = None) -> np.ndarray:
    """One query per sequence over its paged context.

    ``q`` [B][Hq][D]; returns [B][Hq][D] float64.  ``only``: optional list of
    ``(b, h)`` pairs to compute (others left zero).
    """
    B, Hq, D = q.shape
    Hkv = cache.k.shape[1]
    group = Hq // Hkv
    kv_k = cache.values("k")
    kv_v = cache.values("v")
    out = np.zeros((B, Hq, D), dtype=np.float64)
    pairs = only if only is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in pairs:
        K = gather_paged(kv_k, tables[b], int(lens[b]), h // group, cache.block_size)
        V = gather_paged(kv_v, tables[b], int(lens[b]), h // group, cache.block_size)
        out[b, h] = attention_fp64(q[b, h], K, V, scale)
    return out


def dense_decode(q: np.ndarray, Ks: List[np.ndarray], Vs: List[np.ndarray], scale: float,
                 only: Optional[Sequence[tuple]] = None) -> np.ndarray:
    """Same attention over contiguous per-sequence arrays ``Ks[b]`` [L][Hkv][D]."""
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D), dtype=np.float64)
    pairs = only if only is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in pairs:
        Hkv = Ks[b].shape[1]
        kh = h // (Hq // Hkv)
        out[b, h] = attention_fp64(q[b, h], Ks[b][:, kh, :], Vs[b][:, kh, :], scale)
    return out


def paged_prefill(cache: OracleCache, tables: Sequence[Sequence[int]], prior: Sequence[int],
                  chunk: Sequence[int], q: np.ndarray, scale: float,
                  only_rows: Optional[Sequence[tuple]] = None) -> np.ndarray:
    """Chunked-prefill attention over the paged cache.

    ``q`` [sum C][Hq][D]: the chunks of all sequences back to back.  Row ``i``
    of sequence ``b`` sits at absolute position ``prior[b] + i`` and attends to
    tokens ``0 .. prior[b] + i`` (the chunk's own K/V are already in the
    cache).  ``only_rows``: optional ``(b, i, h)`` triples to compute.
    """
    _, Hq, D = q.shape
    Hkv = cache.k.shape[1]
    group = Hq // Hkv
    kv_k = cache.values("k")
    kv_v = cache.values("v")
    starts = np.concatenate([[0], np.cumsum(np.asarray(chunk, dtype=np.int64))])
    out = np.zeros(q.shape, dtype=np.float64)
    if only_rows is None:
        only_rows = [(b, i, h) for b in range(len(chunk)) for i in range(int(chunk[b]))
                     for h in range(Hq)]
    gathered = {}
    for b, i, h in only_rows:
        key = (b, h // group)
        if key not in gathered:
            L = int(prior[b]) + int(chunk[b])
            gathered[key] = (gather_paged(kv_k, tables[b], L, h // group, cache.block_size),
                             gather_paged(kv_v, tables[b], L, h // group, cache.block_size))
        K, V = gathered[key]
        n = int(prior[b]) + i + 1
        r = int(starts[b]) + i
        out[r, h] = attention_fp64(q[r, h], K[:n], V[:n], scale)
    return out


def dense_prefill_row(q_row: np.ndarray, K: np.ndarray, V: np.ndarray, position: int,
                      scale: float) -> np.ndarray:
    """One chunk query at absolute ``position`` over contiguous ``K``/``V``
    [L][D]: keys ``0..position``."""
    n = int(position) + 1
    return attention_fp64(q_row, K[:n], V[:n], scale)
