"""Plain CPU oracle for the paged KV-cache attention path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link
anything in this package: only the test suite, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
and imports nothing from it; both sides are fed from ``workloads``.

It is deliberately slow and literal: Python lists and a ``deque`` for the block
manager, float64 numpy for attention, a table lookup for the fp8 format.  Each
function cites the passage of the pages it follows:

* [p1] "vLLM PagedAttention Deep Dive: KV Cache Memory Fragmentation, Chunked
  Prefill & Prefix Caching"
* [p2] "PagedAttention: KV cache as virtual memory (block manager &
  fragmentation)"
* [p3] "PagedAttention: Why Static Batching Wastes Your KV Cache"

Pins (what each function is checked against, other than itself) live in
``tests/test_oracle_*.py``.  Every function here has at least one pin; none is
"parity unpinned".
"""

from .allocator import OraclePool, Status  # noqa: F401
from .attention import (  # noqa: F401
    attention_fp64,
    attention_heads_fp64,
    causal_chunk_fp64,
    dense_decode,
    paged_decode,
    paged_prefill,
    dense_prefill_row,
    gather_paged,
    OracleCache,
)
from .fp8 import e4m3_decode, e4m3_encode, e4m3_quantize  # noqa: F401
from .capacity import (  # noqa: F401
    kv_bytes_per_token,
    contiguous_fit,
    paged_fit_stop_at_first_failure,
    paged_fit_skip,
    reservation_waste,
)
