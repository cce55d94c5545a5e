"""Capacity arithmetic of the pages (test infrastructure only; see
``oracle/__init__``).

* KV bytes per token: [p3] "PagedAttention: Why Static Batching Wastes Your KV
  Cache", section "Why does static KV cache allocation waste so much memory?":
  K and V, for every layer and KV head, ``head_dim`` values of ``dtype_bytes``.
* Contiguous vs paged fit: [p2] "PagedAttention: KV cache as virtual memory",
  section "Code": a contiguous engine reserves ``ceil(MAX_LEN / BLOCK)`` blocks
  for every sequence; a paged engine needs ``ceil(L / BLOCK)`` blocks.
* Reservation waste of a short reply in a long slab: [p3], "TL;DR".

The page's printed loop keeps admitting shorter sequences after one has not
fitted, which admits 14 of the 16 lengths, while its comment says 13.  The
reading taken for the admission workload is "admit in order and stop at the
first sequence that does not fit" (13); both variants are kept so the tests
pin the discrepancy instead of hiding it.
"""

from __future__ import annotations

import math
from typing import Sequence, Tuple


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    return 2 * num_layers * num_kv_heads * head_dim * dtype_bytes


def contiguous_fit(pool_blocks: int, block: int, max_len: int) -> int:
    reserve = math.ceil(max_len / block)
    return pool_blocks // reserve


def paged_fit_stop_at_first_failure(lens: Sequence[int], pool_blocks: int, block: int) -> Tuple[int, int]:
    """Returns (sequences admitted, blocks used)."""
    used = admitted = 0
    for L in lens:
        need = math.ceil(L / block)
        if used + need > pool_blocks:
            break
        used += need
        admitted += 1
    return admitted, used


def paged_fit_skip(lens: Sequence[int], pool_blocks: int, block: int) -> Tuple[int, int]:
    """The printed loop: a sequence that does not fit is skipped, later ones
    are still tried."""
    used = admitted = 0
    for L in lens:
        need = math.ceil(L / block)
        if used + need <= pool_blocks:
            used += need
            admitted += 1
    return admitted, used


def reservation_waste(reserved_tokens: int, used_tokens: int) -> float:
    return (reserved_tokens - used_tokens) / reserved_tokens
