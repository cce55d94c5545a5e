"""Capacity arithmetic of the pages (test infrastructure only; see
``oracle/__init__``).

* KV bytes per token: [p3] "PagedAttention: Why Static Batching Wastes Your KV
  Cache", section "Why does static KV cache allocation waste so much memory?":
  K and V, for every layer and KV head, ``head_dim`` values of ``dtype_bytes``.
* Contiguous vs paged fit: [p2] "PagedAttention: KV cache as virtual memory",
  section "Code": a contiguous engine reserves ``ceil(MAX_LEN / BLOCK)`` blocks
  for every sequence; a paged engine needs ``ceil(L / BLOCK)`` blocks.
* Reservation waste of a short reply in a long slab: [p3], "TL;DR".

The expected figures for the 16 listed lengths in a 128-block pool come from
[p2] "Code": 4 sequences under contiguous reservation and 13 under paging.
Read literally, the admission rule printed there (a sequence that does not fit
is passed over and later ones are still tried) admits 14, not 13.  The reading
taken for the admission workload is "admit in order and stop at the first
sequence that does not fit" (13).  Both rules are written here, each from its
definition, so the tests pin the discrepancy instead of hiding it.
"""

from __future__ import annotations

import math
from typing import Sequence, Tuple

import numpy as np


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    return 2 * num_layers * num_kv_heads * head_dim * dtype_bytes


def contiguous_fit(pool_blocks: int, block: int, max_len: int) -> int:
    """Sequences that fit when each reserves a whole MAX_LEN slab of blocks."""
    slab = math.ceil(max_len / block)
    return pool_blocks // slab


def _blocks(lens: Sequence[int], block: int) -> np.ndarray:
    return np.array([math.ceil(int(L) / block) for L in lens], dtype=np.int64)


def paged_fit_stop_at_first_failure(lens: Sequence[int], pool_blocks: int, block: int) -> Tuple[int, int]:
    """Admission in order until the first sequence that does not fit: the
    admitted sequences are the longest leading run whose block counts sum to at
    most the pool.  Returns (sequences admitted, blocks used)."""
    totals = np.cumsum(_blocks(lens, block))
    admitted = int(np.searchsorted(totals, pool_blocks, side="right"))
    return admitted, int(totals[admitted - 1]) if admitted else 0


def paged_fit_skip(lens: Sequence[int], pool_blocks: int, block: int) -> Tuple[int, int]:
    """Admission in order that passes over a sequence that does not fit and
    keeps trying later ones: the leading run that fits is admitted, the first
    sequence after it is passed over, and the rest are admitted the same way
    into the blocks still free."""
    lens = list(lens)
    n, used = paged_fit_stop_at_first_failure(lens, pool_blocks, block)
    if n >= len(lens):
        return n, used
    n_rest, used_rest = paged_fit_skip(lens[n + 1:], pool_blocks - used, block)
    return n + n_rest, used + used_rest


def reservation_waste(reserved_tokens: int, used_tokens: int) -> float:
    return (reserved_tokens - used_tokens) / reserved_tokens
