"""Every output of the full-size workloads against the float64 oracle.

* the Llama-2-13B-shaped decode step (64 sequences, lengths U[1, 2048], 40
  heads of 128): as one launch (new token written by the attention launch) and
  as two calls (KV write, then decode), fp16 and e4m3 caches;
* the shared-prompt batch (32 forks of an 800- and of an 808-token prompt,
  private tails U[1, 1024]), fp16 and e4m3, with and without the shared-prefix
  read hint, one launch and two calls; the shared full blocks are stored once;
* the chunked prefill (8 sequences, prior context U[0, 4096], 512-row chunks),
  fp16 and e4m3.

Each compares all B x Hq (or sum C x Hq) output vectors element by element:
2e-3 absolute + 2e-3 relative against the oracle over what the cache holds
(the dequantised codes for e4m3), and for e4m3 also 5e-2 + 5e-2 relative
against the oracle over the fp16 source for contexts of 200 tokens and more
(a shorter context can miss that by the format's rounding alone).  The pages
state that the paged result is the dense one ("PagedAttention: KV cache as
virtual memory (block manager & fragmentation)", "Interviewer follow-ups").
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_394_amd as pa
import workloads
from gpu_harness import (ATOL8, PrefillCase, Twin, close, oracle_decode_all, oracle_prefill_all,
                         parallel_map, same_bytes, scales_of)

pytestmark = pytest.mark.gpu


def _warm(w, n):
    # draw every sequence's rows once and keep them (all later reads reuse them)
    parallel_map(lambda b: w.kv(b, cache=True), range(n))


@pytest.mark.parametrize("fp8", [False, True], ids=["fp16", "e4m3"])
def test_llama13b_step_every_output(fp8):
    w = workloads.llama13b_decode()
    _warm(w, w.batch)
    t = Twin(w, fp8=fp8)
    two, two_cache = t.two_calls()
    one, one_cache = t.one_call()
    assert np.array_equal(one.view(np.uint32), two.view(np.uint32))
    same_bytes(one_cache, two_cache)
    ref = oracle_decode_all(w.q, w.kv, w.batch, w.scale, t.scales if fp8 else None)
    close(one, ref)
    if fp8:
        src = oracle_decode_all(w.q, w.kv, w.batch, w.scale)
        long_ = w.lens >= 200
        close(one[long_], src[long_], ATOL8, ATOL8)


class SharedPrompt:
    """32 forks of one prompt, each with its private tail but the last token
    written; the last token's slot reserved (copy-on-write pairs kept)."""

    def __init__(self, w, fp8):
        self.w = w
        pk, pv = w.prompt_kv()
        self.rows = [(np.concatenate([pk, w.kv(b)[0]]), np.concatenate([pv, w.kv(b)[1]]))
                     for b in range(w.batch)]
        self.scales = scales_of(self.rows) if fp8 else (1.0, 1.0)
        ks, vs = self.scales
        self.pool = pa.pa_pool_create(w.num_blocks, 16)
        self.cache = pa.KvCache(w.num_blocks, w.num_kv_heads, w.head_dim, fp8=fp8, k_scale=ks,
                                v_scale=vs, fill=(255 if fp8 else float("nan")))
        root = pa.pa_seq_create(self.pool)
        sl, _ = pa.pa_alloc_append(self.pool, root, w.prompt_len)
        pa.pa_write_kv(self.cache, torch.from_numpy(pk).cuda(), torch.from_numpy(pv).cuda(),
                       torch.from_numpy(sl).cuda())
        self.seqs = [root] + [pa.pa_fork_cow(self.pool, root) for _ in range(w.batch - 1)]
        self.copies = 0
        for b, s in enumerate(self.seqs):
            n = int(w.tails[b]) - 1
            if n:
                k, v = w.kv(b)
                sl, cow = pa.pa_alloc_append(self.pool, s, n)
                self.copies += cow is not None
                pa.pa_write_kv(self.cache, torch.from_numpy(k[:n]).cuda(), torch.from_numpy(v[:n]).cuda(),
                               torch.from_numpy(sl).cuda(), [cow] if cow else None)
        self.new_slots, self.pairs = [], []
        for s in self.seqs:
            sl, cow = pa.pa_alloc_append(self.pool, s, 1)
            self.new_slots.append(int(sl[0]))
            if cow:
                self.pairs.append(cow)
        self.copies += len(self.pairs)
        self.max_ctx = int(w.lens.max())
        tables, lens = pa.pa_block_tables(self.pool, self.seqs, -(-self.max_ctx // 16))
        assert np.array_equal(lens, w.lens.astype(np.int32))
        self.tables_np = tables
        self.tables, self.lens = torch.from_numpy(tables).cuda(), torch.from_numpy(lens).cuda()
        self.hint = torch.from_numpy(pa.pa_shared_prefix(self.pool, self.seqs)).cuda()
        self.k_new = torch.from_numpy(np.stack([w.kv(b)[0][-1] for b in range(w.batch)])).cuda()
        self.v_new = torch.from_numpy(np.stack([w.kv(b)[1][-1] for b in range(w.batch)])).cuda()
        self.q = torch.from_numpy(w.q).cuda()
        self.ws = torch.empty(max(16, pa.pa_decode_workspace_bytes(w.batch, w.num_heads, w.head_dim,
                                                                   self.max_ctx)),
                              dtype=torch.uint8, device="cuda")

    def out(self):
        w = self.w
        return torch.full((w.batch, w.num_heads, w.head_dim), float("nan"), device="cuda")

    def two_calls(self):
        a, b = self.out(), self.out()
        pa.pa_write_kv(self.cache, self.k_new, self.v_new,
                       torch.tensor(self.new_slots, dtype=torch.int32, device="cuda"), self.pairs or None)
        pa.pa_decode(self.cache, self.q, self.tables, self.lens, self.max_ctx, self.w.scale, a, self.ws)
        pa.pa_decode(self.cache, self.q, self.tables, self.lens, self.max_ctx, self.w.scale, b, self.ws,
                     cached_blocks=self.hint)
        torch.cuda.synchronize()
        return a.cpu().numpy(), b.cpu().numpy()

    def one_call(self):
        o = self.out()
        pa.pa_decode_append(self.cache, self.q, self.k_new, self.v_new, self.tables, self.lens,
                            self.max_ctx, self.w.scale, o, self.ws, cow_pairs=self.pairs or None,
                            cached_blocks=self.hint)
        torch.cuda.synchronize()
        return o.cpu().numpy()


@pytest.mark.parametrize("prompt", [800, 808])
@pytest.mark.parametrize("fp8", [False, True], ids=["fp16", "e4m3"])
def test_shared_prompt_every_output(prompt, fp8):
    w = workloads.prefix_cow(prompt_len=prompt)
    _warm(w, w.batch)
    one_side, two_side = SharedPrompt(w, fp8), SharedPrompt(w, fp8)
    full = prompt // 16
    # one stored copy of the prompt's full blocks, held by all 32 tables
    assert (one_side.tables_np[:, :full] == one_side.tables_np[0, :full]).all()
    assert (one_side.hint.cpu().numpy() == full).all()
    assert one_side.copies == (0 if prompt % 16 == 0 else w.batch - 1)
    plain, hinted = two_side.two_calls()
    fused = one_side.one_call()
    assert np.array_equal(plain.view(np.uint32), hinted.view(np.uint32))
    assert np.array_equal(plain.view(np.uint32), fused.view(np.uint32))
    same_bytes(one_side.cache, two_side.cache)
    rows = one_side.rows
    ref = oracle_decode_all(w.q, lambda b: rows[b], w.batch, w.scale,
                            one_side.scales if fp8 else None)
    close(fused, ref)
    if fp8:
        src = oracle_decode_all(w.q, lambda b: rows[b], w.batch, w.scale)
        close(fused, src, ATOL8, ATOL8)     # every context here is over 200 tokens


@pytest.mark.parametrize("fp8", [False, True], ids=["fp16", "e4m3"])
def test_chunked_prefill_every_output(fp8):
    w = workloads.chunked_prefill()
    _warm(w, w.batch)
    case = PrefillCase(w, fp8=fp8)
    got = case.run()
    ref = oracle_prefill_all(w, case.cu_np, w.kv, case.scales)
    close(got, ref)
    if fp8:
        src = oracle_prefill_all(w, case.cu_np, w.kv)
        ctx = np.concatenate([int(w.prior[b]) + 1 + np.arange(int(w.chunk[b])) for b in range(w.batch)])
        long_ = ctx >= 200
        close(got[long_], src[long_], ATOL8, ATOL8)
