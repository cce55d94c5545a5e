"""Seeded synthetic inputs for the paged-attention hot path.

This module only draws numbers: context lengths, pool sizes, initial free-queue
orders and Q/K/V values.  It holds none of the method's arithmetic (no slot
mapping, no allocation, no attention, no fp8 encoding), so the oracle and the
HIP path can both be fed from it without sharing any of their logic.

Seeding
-------
Each workload has a base seed ``s``.  ``numpy.random.default_rng(s)`` draws, in
this order: the lengths (where random), the free-queue permutation (where
random), then Q.  The K/V rows of sequence ``b`` come from their own stream,
``default_rng((s, b + 1))`` (K first, then V), so any one sequence can be
regenerated on its own; this is what lets a full-size run be checked on a
sample of sequences.  Values are drawn in float32 and rounded to float16
(round-to-nearest-even, numpy's ``astype``).

Shapes follow the pages' workloads: 16-token blocks; the 16 request lengths of
the fragmentation arithmetic example; a Llama-2-13B-shaped layer (40 heads of
128); an 800-token shared system prompt; long prompts split into chunks.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Tuple

import numpy as np

BLOCK_SIZE = 16

# The 16 request lengths of the pure-Python fragmentation example
# ("PagedAttention: KV cache as virtual memory", section "Code").
FRAGMENTATION_LENS = (40, 128, 300, 64, 210, 96, 180, 48, 150, 80, 60, 420, 33, 256, 90, 110)


def _ceil_div(a: int, b: int) -> int:
    return -(-int(a) // int(b))


def _draw(rng: np.random.Generator, shape, dist: str) -> np.ndarray:
    if dist == "normal":
        x = rng.standard_normal(size=shape, dtype=np.float32)
    elif dist == "uniform":
        x = rng.random(size=shape, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
    else:
        raise ValueError(dist)
    return x.astype(np.float16)


@dataclass
class Workload:
    """One synthetic batch.

    ``kv(b)`` returns ``(K, V)`` for sequence ``b``, each ``[n_tokens][Hkv][D]``
    float16, covering every token the sequence will hold (for prefill: prior
    context followed by the chunk).  For the shared-prefix workload the rows are
    ``prompt ++ tail_b`` and the prompt rows come from ``prompt_kv()``.
    """

    name: str
    seed: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    lens: np.ndarray                       # int64 [B]: tokens in the cache at attention time
    q: np.ndarray                          # float16: [B][Hq][D] (decode) or [sum C][Hq][D] (prefill)
    dist: str
    init_free_order: Optional[np.ndarray] = None  # int32 [num_blocks] or None (ascending)
    block_size: int = BLOCK_SIZE
    # prefill only
    prior: Optional[np.ndarray] = None     # int64 [B]
    chunk: Optional[np.ndarray] = None     # int64 [B]
    # shared-prefix only
    prompt_len: int = 0
    tails: Optional[np.ndarray] = None     # int64 [B]
    _kv_fn: Optional[Callable[[int], Tuple[np.ndarray, np.ndarray]]] = None
    _prompt_fn: Optional[Callable[[], Tuple[np.ndarray, np.ndarray]]] = None
    _cache: Dict[int, Tuple[np.ndarray, np.ndarray]] = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(len(self.lens))

    @property
    def scale(self) -> float:
        # softmax scale 1/sqrt(head_dim) for every workload
        return float(1.0 / np.sqrt(self.head_dim))

    def kv(self, b: int, cache: bool = False) -> Tuple[np.ndarray, np.ndarray]:
        if b in self._cache:
            return self._cache[b]
        out = self._kv_fn(b)
        if cache:
            self._cache[b] = out
        return out

    def prompt_kv(self) -> Tuple[np.ndarray, np.ndarray]:
        return self._prompt_fn()


def _per_seq_kv(seed: int, ntok: Callable[[int], int], hkv: int, d: int, dist: str):
    def fn(b: int):
        rng = np.random.default_rng((seed, b + 1))
        n = int(ntok(b))
        k = _draw(rng, (n, hkv, d), dist)
        v = _draw(rng, (n, hkv, d), dist)
        return k, v
    return fn


def tiny_decode(seed: int = 1001) -> Workload:
    """2 sequences of 30 and 50 tokens, a 32-block pool whose free queue is a
    seeded permutation, 4 heads of 64, U[-1,1] values."""
    rng = np.random.default_rng(seed)
    lens = np.array([30, 50], dtype=np.int64)
    perm = rng.permutation(32).astype(np.int32)
    h, d = 4, 64
    q = _draw(rng, (2, h, d), "uniform")
    return Workload("tiny_decode", seed, h, h, d, 32, lens, q, "uniform", perm,
                    _kv_fn=_per_seq_kv(seed, lambda b: lens[b], h, d, "uniform"))


def tiny_decode_worked_example(seed: int = 1001) -> Workload:
    """Same as ``tiny_decode`` but with the free queue ordered so the two
    sequences receive physical blocks {10, 25} and {3, 7, 12, 18}, the worked
    block tables of "vLLM PagedAttention Deep Dive", section "PagedAttention
    Mechanism" (its code comments)."""
    w = tiny_decode(seed)
    head = [10, 25, 3, 7, 12, 18]
    rest = [i for i in range(32) if i not in head]
    w.init_free_order = np.array(head + rest, dtype=np.int32)
    w.name = "tiny_decode_worked_example"
    return w


def alloc_decode(seed: int = 1002) -> Workload:
    """The 16 lengths of the fragmentation example, a 128-block pool (ascending
    free queue), 8 heads of 128, N(0,1) values.  Values are drawn for all 16
    sequences; the harness admits in order until the pool is full."""
    rng = np.random.default_rng(seed)
    lens = np.array(FRAGMENTATION_LENS, dtype=np.int64)
    h, d = 8, 128
    q = _draw(rng, (len(lens), h, d), "normal")
    return Workload("alloc_decode", seed, h, h, d, 128, lens, q, "normal", None,
                    _kv_fn=_per_seq_kv(seed, lambda b: lens[b], h, d, "normal"))


def llama13b_decode(seed: int = 1003, batch: int = 64, max_len: int = 2048,
                    num_heads: int = 40, head_dim: int = 128,
                    pool_slack: float = 0.10) -> Workload:
    """Llama-2-13B-shaped single layer: 40 query heads = 40 KV heads of 128,
    ``batch`` sequences with lengths uniform in [1, max_len], a pool of the
    blocks needed plus 10% whose free queue is a seeded shuffle, N(0,1)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, max_len + 1, size=batch).astype(np.int64)
    need = sum(_ceil_div(L, BLOCK_SIZE) for L in lens)
    nblocks = int(np.ceil((1.0 + pool_slack) * need))
    perm = rng.permutation(nblocks).astype(np.int32)
    q = _draw(rng, (batch, num_heads, head_dim), "normal")
    return Workload("llama13b_decode", seed, num_heads, num_heads, head_dim, nblocks, lens, q,
                    "normal", perm,
                    _kv_fn=_per_seq_kv(seed, lambda b: lens[b], num_heads, head_dim, "normal"))


def prefix_cow(seed: int = 1004, prompt_len: int = 800, batch: int = 32, max_tail: int = 1024,
               num_heads: int = 40, head_dim: int = 128) -> Workload:
    """``batch`` sequences sharing one ``prompt_len``-token system prompt, each
    followed by a private tail of uniform [1, max_tail] tokens; N(0,1).
    ``kv(b)`` returns the tail rows only; ``prompt_kv()`` the shared rows."""
    rng = np.random.default_rng(seed)
    tails = rng.integers(1, max_tail + 1, size=batch).astype(np.int64)
    q = _draw(rng, (batch, num_heads, head_dim), "normal")
    lens = tails + prompt_len
    need = _ceil_div(prompt_len, BLOCK_SIZE) + sum(_ceil_div(t, BLOCK_SIZE) + 1 for t in tails)
    nblocks = int(need + 16)

    def prompt_fn():
        prng = np.random.default_rng((seed, 0))
        k = _draw(prng, (prompt_len, num_heads, head_dim), "normal")
        v = _draw(prng, (prompt_len, num_heads, head_dim), "normal")
        return k, v

    w = Workload("prefix_cow", seed, num_heads, num_heads, head_dim, nblocks, lens, q, "normal",
                 None, prompt_len=prompt_len, tails=tails,
                 _kv_fn=_per_seq_kv(seed, lambda b: tails[b], num_heads, head_dim, "normal"),
                 _prompt_fn=prompt_fn)
    return w


def chunked_prefill(seed: int = 1005, batch: int = 8, max_prior: int = 4096, chunk: int = 512,
                    num_heads: int = 40, head_dim: int = 128, pool_slack: float = 0.10) -> Workload:
    """``batch`` sequences, each with a prior context of uniform [0, max_prior]
    tokens already cached plus one new ``chunk``-token chunk; N(0,1).
    ``q`` holds the chunk queries of all sequences back to back."""
    rng = np.random.default_rng(seed)
    prior = rng.integers(0, max_prior + 1, size=batch).astype(np.int64)
    chunks = np.full(batch, chunk, dtype=np.int64)
    lens = prior + chunks
    need = sum(_ceil_div(L, BLOCK_SIZE) for L in lens)
    nblocks = int(np.ceil((1.0 + pool_slack) * need)) + 1
    perm = rng.permutation(nblocks).astype(np.int32)
    q = _draw(rng, (int(chunks.sum()), num_heads, head_dim), "normal")
    return Workload("chunked_prefill", seed, num_heads, num_heads, head_dim, nblocks, lens, q,
                    "normal", perm, prior=prior, chunk=chunks,
                    _kv_fn=_per_seq_kv(seed, lambda b: lens[b], num_heads, head_dim, "normal"))


def custom_decode(seed: int, lens, num_heads: int, num_kv_heads: int, head_dim: int,
                  num_blocks: Optional[int] = None, shuffle: bool = True,
                  dist: str = "normal") -> Workload:
    """Free-form decode batch for edge cases (ragged tails, GQA, empty lengths)."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    need = sum(_ceil_div(L, BLOCK_SIZE) for L in lens) + 1
    nblocks = int(num_blocks if num_blocks is not None else need + 8)
    perm = rng.permutation(nblocks).astype(np.int32)   # drawn either way: Q stays the same
    q = _draw(rng, (len(lens), num_heads, head_dim), dist)
    return Workload("custom_decode", seed, num_heads, num_kv_heads, head_dim, nblocks, lens, q,
                    dist, perm if shuffle else None,
                    _kv_fn=_per_seq_kv(seed, lambda b: lens[b], num_kv_heads, head_dim, dist))


def custom_prefill(seed: int, prior, chunk, num_heads: int, num_kv_heads: int, head_dim: int,
                   dist: str = "normal") -> Workload:
    """Free-form chunked-prefill batch for edge cases (P = 0, short or ragged chunks)."""
    rng = np.random.default_rng(seed)
    prior = np.asarray(prior, dtype=np.int64)
    chunks = np.asarray(chunk, dtype=np.int64)
    lens = prior + chunks
    need = sum(_ceil_div(L, BLOCK_SIZE) for L in lens) + 1
    nblocks = int(need + 8)
    perm = rng.permutation(nblocks).astype(np.int32)
    q = _draw(rng, (int(chunks.sum()), num_heads, head_dim), dist)
    return Workload("custom_prefill", seed, num_heads, num_kv_heads, head_dim, nblocks, lens, q,
                    dist, perm, prior=prior, chunk=chunks,
                    _kv_fn=_per_seq_kv(seed, lambda b: lens[b], num_kv_heads, head_dim, dist))


def fp8_scale(x: np.ndarray) -> np.float32:
    """Per-tensor calibration input for an e4m3 cache: amax / 448 in float32
    (448 is the largest finite e4m3 magnitude).  A caller's choice of scale, not
    part of the method; both sides receive the same value."""
    amax = np.float32(np.max(np.abs(x.astype(np.float32)))) if x.size else np.float32(0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / np.float32(448.0))


WORKLOADS = {
    "tiny_decode": tiny_decode,
    "alloc_decode": alloc_decode,
    "llama13b_decode": llama13b_decode,
    "prefix_cow": prefix_cow,
    "chunked_prefill": chunked_prefill,
}


@dataclass
class Dialogue:
    """Multi-turn conversations for prefix caching ([p1] "Automatic Prefix
    Caching (APC)": each turn's prompt starts with the conversation so far).

    ``turns[c][t]`` is ``(prompt, reply)``: token-id lists; the prompt of turn
    t + 1 is the prompt of turn t, its reply, then a new user message.  K/V rows
    depend only on the token id and its position (an embedding-plus-position
    stand-in for a model), so identical prefixes carry identical K/V, as the
    pages require of a reusable block; ``kv(tokens, lo, hi)`` gives rows lo..hi-1.
    """
    seed: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    vocab: int
    turns: List[List[Tuple[List[int], List[int]]]]
    num_blocks: int
    _tok_k: np.ndarray = field(repr=False, default=None)
    _tok_v: np.ndarray = field(repr=False, default=None)
    _pos_k: np.ndarray = field(repr=False, default=None)
    _pos_v: np.ndarray = field(repr=False, default=None)

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.head_dim))

    def kv(self, tokens, lo: int, hi: int) -> Tuple[np.ndarray, np.ndarray]:
        ids = np.asarray(tokens[lo:hi], dtype=np.int64)
        pos = np.arange(lo, hi)
        k = (self._tok_k[ids] + self._pos_k[pos]).astype(np.float16)
        v = (self._tok_v[ids] + self._pos_v[pos]).astype(np.float16)
        return k, v

    def query(self, c: int, t: int) -> np.ndarray:
        rng = np.random.default_rng((self.seed, 1000 + c, t))
        return _draw(rng, (self.num_heads, self.head_dim), "normal")


def dialogue(seed: int = 1006, conversations: int = 16, turns: int = 4, num_heads: int = 8,
             num_kv_heads: int = 8, head_dim: int = 128, vocab: int = 512,
             first=(200, 600), reply=(20, 200), message=(10, 100)) -> Dialogue:
    """``conversations`` dialogues of ``turns`` turns: first prompts U[first],
    replies U[reply], user messages U[message] tokens (inclusive bounds)."""
    rng = np.random.default_rng(seed)
    convs = []
    max_len = 0
    for _ in range(conversations):
        prompt = rng.integers(0, vocab, size=int(rng.integers(first[0], first[1] + 1))).tolist()
        conv = []
        for t in range(turns):
            rep = rng.integers(0, vocab, size=int(rng.integers(reply[0], reply[1] + 1))).tolist()
            conv.append((list(prompt), rep))
            max_len = max(max_len, len(prompt) + len(rep))
            msg = rng.integers(0, vocab, size=int(rng.integers(message[0], message[1] + 1))).tolist()
            prompt = prompt + rep + msg
        convs.append(conv)
    tok_k = _draw(rng, (vocab, num_kv_heads, head_dim), "normal") * np.float32(0.7)
    tok_v = _draw(rng, (vocab, num_kv_heads, head_dim), "normal")
    pos_k = _draw(rng, (max_len + 1, num_kv_heads, head_dim), "normal") * np.float32(0.7)
    pos_v = _draw(rng, (max_len + 1, num_kv_heads, head_dim), "normal") * np.float32(0.1)
    # room for every conversation's longest turn at once, plus slack for cached blocks
    need = sum(_ceil_div(len(c[-1][0]) + len(c[-1][1]), BLOCK_SIZE) for c in convs)
    return Dialogue(seed, num_heads, num_kv_heads, head_dim, vocab, convs, int(need * 2 + 16),
                    tok_k, tok_v, pos_k, pos_v)
