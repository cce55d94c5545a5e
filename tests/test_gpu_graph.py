"""The device calls under HIP graph capture: a captured decode step (one
launch, and the two-call form), a captured split-path decode (split kernel +
merge kernel) and a captured chunked prefill are replayed several times, with
eager work and synchronisations between the replays, and every replay must
equal the eager result bit for bit.  None of the calls records a memset or
allocates, so they can sit inside a caller's graph."""

import numpy as np
import pytest
import torch

import paged_kv_cache_394_amd as pa
import workloads
from gpu_harness import PrefillCase

pytestmark = pytest.mark.gpu

REPLAYS = 4


def replay_equals_eager(fn, out: torch.Tensor, disturb):
    """Eager result of fn, then REPLAYS graph replays of it, each checked
    against the eager bits after the output was overwritten."""
    fn()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on the capture stream, as torch asks
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for i in range(REPLAYS):
        out.fill_(float("nan"))
        disturb(i)                  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), f"replay {i}"


def test_captured_decode_step_and_two_call_form():
    rng = np.random.default_rng(501)
    lens = rng.integers(1, 1500, size=64)
    w = workloads.custom_decode(501, lens, 32, 8, 128)
    pool = pa.pa_pool_create(w.num_blocks, 16, w.init_free_order)
    cache = pa.KvCache(w.num_blocks, w.num_kv_heads, w.head_dim, fill=float("nan"))
    ids, slots, kn, vn = [], [], [], []
    for b in range(w.batch):
        s = pa.pa_seq_create(pool)
        ids.append(s)
        k, v = w.kv(b)
        L = int(lens[b])
        sl, _ = pa.pa_alloc_append(pool, s, L - 1)
        if L > 1:
            pa.pa_write_kv(cache, torch.from_numpy(k[:L - 1]).cuda(), torch.from_numpy(v[:L - 1]).cuda(),
                           torch.from_numpy(sl).cuda())
        sl, _ = pa.pa_alloc_append(pool, s, 1)
        slots.append(int(sl[0]))
        kn.append(k[L - 1])
        vn.append(v[L - 1])
    max_ctx = int(lens.max())
    tables, ll = pa.pa_block_tables(pool, ids, -(-max_ctx // 16))
    tt, ll = torch.from_numpy(tables).cuda(), torch.from_numpy(ll).cuda()
    kn = torch.from_numpy(np.stack(kn)).cuda()
    vn = torch.from_numpy(np.stack(vn)).cuda()
    sl = torch.tensor(slots, dtype=torch.int32, device="cuda")
    q = torch.from_numpy(w.q).cuda()
    out = torch.empty((w.batch, w.num_heads, w.head_dim), device="cuda")
    ws = torch.empty(max(16, pa.pa_decode_workspace_bytes(w.batch, w.num_heads, w.head_dim, max_ctx)),
                     dtype=torch.uint8, device="cuda")
    junk = torch.empty(1 << 20, device="cuda")

    def disturb(i):
        junk.normal_()
        junk.sum()

    replay_equals_eager(lambda: pa.pa_decode_append(cache, q, kn, vn, tt, ll, max_ctx, w.scale, out, ws),
                        out, disturb)

    def two_calls():
        pa.pa_write_kv(cache, kn, vn, sl)
        pa.pa_decode(cache, q, tt, ll, max_ctx, w.scale, out, ws)

    replay_equals_eager(two_calls, out, disturb)


def test_captured_split_path_decode():
    """A narrow batch with long contexts: split kernel and merge kernel."""
    w = workloads.custom_decode(511, [9000, 3000, 17, 0, 4100], 8, 2, 128)
    from gpu_harness import DecodeCase
    case = DecodeCase(w)
    junk = torch.empty(1 << 18, device="cuda")
    replay_equals_eager(lambda: pa.pa_decode(case.cache, case.q, case.tables, case.lens, case.max_ctx,
                                             w.scale, case.out, case.ws),
                        case.out, lambda i: junk.uniform_())


def test_captured_prefill():
    w = workloads.custom_prefill(521, [0, 37, 300, 900], [1, 130, 200, 64], 4, 2, 128)
    case = PrefillCase(w)
    junk = torch.empty(1 << 18, device="cuda")
    replay_equals_eager(lambda: pa.pa_prefill_chunk(case.cache, case.q, case.cu, case.prior, case.tables,
                                                    int(w.chunk.max()), w.scale, case.out),
                        case.out, lambda i: junk.uniform_())
