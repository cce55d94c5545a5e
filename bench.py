"""Benchmark of the paged KV-cache attention hot path on one MI355X.

Step (timed): one decode iteration of the Llama-2-13B-shaped batch -- 64
sequences, context lengths uniform in [1, 2048], 40 heads of 128, fp16 K/V in
16-token blocks scattered over the pool.  The step writes the 64 new tokens'
K/V into their slots and runs the paged decode over every context, in one
launch (pa_decode_append; the same bits as pa_write_kv then pa_decode, which
is timed beside it).  The block-manager work of the iteration (allocation,
table export) is host work, done before the timed region and timed on its own.
Each of the K timed steps starts with cold caches: 1 GiB of unrelated writes
evicts L2 and the last-level cache, then one HIP event pair on the library's
stream brackets the step's launch; the K steps sit between two
synchronisations.  `value` uses the median step, the roofline the mean (the
step kernel's average launch duration).

Reported on one JSON line:
  value        KV-read GB/s of the step: K+V bytes of the contexts / median
               cold step time
  roofline     the step kernel against 8 TB/s (algorithmic bytes / mean cold
               launch time)
  warm_step    the same step run back to back (caches warm from the previous
               step), one event pair over the K steps
  ceiling      a plain device copy of 1 GiB (read + write GB/s), for context
  read_ceiling torch's fastest read-bound reduction over 1 GiB, for context
  achievable_mfma  the library's matrix-core probe (fp16 MFMAs on register
               operands): the matrix throughput the part sustains, for context
               beside the prefill's MFMA utilisation
  achievable_read  the library's read-only probe kernel with the decode's
               access pattern (random 4 KiB tiles, 1.35 GB): the practical
               read ceiling, and the step's fraction of it
  fp8_decode   the same batch with an e4m3 cache
  prefix_cow   32 sequences sharing an 800-token prompt: GB/s on unique and on
               logical K/V bytes
  prefix_cache multi-turn dialogues through the prefix cache: hit rate and
               block-manager call times (host only)
  mixed_step   the prefill and decode batches over one cache in one launch
               (pa_mixed_step) against two launches
  preemption   one 2048-token sequence swapped to pinned host memory and back
               (PCIe GB/s), against its attention-side recomputation
  prefill      chunked prefill, 8 x 512-token chunks over 0..4096 cached tokens,
               causal-valid FLOPs / time against the 2.5 PFLOP/s fp16 MFMA peak
  host         block-manager call times (admission per sequence, the step's
               batched reservation for all 64 sequences, table export)
  capacity     13B-shaped requests that fit beside the weights: reserving the
               maximum length per request against the library's block pool
  cpu_baseline the float64 oracle on a bounded sample of the batch (one core)
  cpu_baseline_pool  the same oracle over the whole batch in a pool of
               single-threaded processes (one per host core, 16 at most)

Every leg first runs its own work untimed for SETTLE_S seconds, so that the
GPU is at its steady clock when the W warm-up steps and the timed region
start (after the host-side set-up of a leg the clock has dropped).

Counter runs: ``--pmc-run [WORKLOAD]`` does only a 256 MiB device copy
(torch.neg, one elementwise kernel that reads and writes 256 MiB) and a few
decode calls of one workload (the 13B-shaped step in fp16 or e4m3, or the
shared-prompt decode), for ``rocprofv3 --pmc FETCH_SIZE`` / ``WRITE_SIZE``;
``--summarize-pmc FETCH_DIR WRITE_DIR [WORKLOAD]`` turns the two counter CSVs
into that workload's profiles/decode_*_traffic.md, scaling the decode
kernels' counts by the copy's (known bytes / counted bytes).
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak
METRIC = "paged decode KV-read GB/s and % of HBM peak; tokens/s; prefill MFMA util"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_llama13b_fp16_traffic.md")
PMC_COPY_BYTES = 256 << 20
PMC_DECODE_STEPS = 5


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in ("decode.hip", "decode_impl.hpp", "device_common.hpp"):
        with open(os.path.join(ROOT, "paged_kv_cache_394_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def prefill_source_hash() -> str:
    h = hashlib.sha256()
    for name in ("prefill.hip", "prefill_pp_impl.hpp", "prefill_impl.hpp", "device_common.hpp"):
        with open(os.path.join(ROOT, "paged_kv_cache_394_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes (read, written) per pa_decode launch from the committed counter
    summary, if it was taken on the current kernel source (else None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m_src = re.search(r"kernel source hash: `([0-9a-f]+)`", text)
    m_rd = re.search(r"HBM bytes read per decode-step launch: `([0-9.eE+]+)`", text)
    m_wr = re.search(r"HBM bytes written per decode-step launch: `([0-9.eE+]+)`", text)
    if not (m_src and m_rd and m_wr) or m_src.group(1) != kernel_source_hash():
        return None
    return float(m_rd.group(1)), float(m_wr.group(1))


def fp8_scales(w, np):
    ka = va = np.float32(0)
    for b in range(w.batch):
        k, v = w.kv(b)
        ka = max(ka, np.abs(k.astype(np.float32)).max())
        va = max(va, np.abs(v.astype(np.float32)).max())
    return float(np.float32(ka / np.float32(448))), float(np.float32(va / np.float32(448)))


def pool_geometry(w, block_size, np):
    """(num_blocks, free order) holding ``w``'s tokens at ``block_size``: the
    workloads size their pools in 16-token blocks; other sizes keep the
    capacity in tokens plus one spare block per sequence, freshly shuffled."""
    if block_size == 16:
        return w.num_blocks, w.init_free_order
    nb = -(-w.num_blocks * 16 // block_size) + w.batch + 8
    return nb, np.random.default_rng(1000 + w.seed + block_size).permutation(nb).astype(np.int32)


def capacity(pa, np, hbm_bytes=288e9, weight_bytes=26e9, max_len=2048, block_size=16, seed=2048):
    """How many requests of a Llama-2-13B-shaped model (40 layers x 40 KV heads
    x 128 dims, fp16: 819,200 KV bytes a token) fit in the memory left after the
    fp16 weights, admitted in arrival order until the first that does not fit:
    reserving max_len tokens per request up front, against the library's block
    pool (one block id spans every layer, so a block is 16 tokens of all
    layers).  Request lengths are U[1, max_len], the decode workload's mix.
    Host only; the same arithmetic for a 40 GB device is reported as context."""
    per_token = 2 * 40 * 40 * 128 * 2
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, max_len + 1, size=4096)

    def fit(total_bytes):
        budget = total_bytes - weight_bytes
        naive = int(budget // (max_len * per_token))
        n_blocks = int(budget // (block_size * per_token))
        pool = pa.pa_pool_create(n_blocks, block_size, None)
        admitted, tokens = 0, 0
        for L in lens:
            s = pa.pa_seq_create(pool)
            try:
                pa.pa_alloc_append(pool, s, int(L))
            except pa.PaError as e:
                if e.status != pa.PA_ERR_NO_BLOCKS:
                    raise
                break
            admitted += 1
            tokens += int(L)
        used_blocks = n_blocks - pa.pa_pool_state(pool)[0]["free_blocks"]
        return {"kv_budget_gb": round(budget / 1e9, 2), "blocks": n_blocks,
                "reserve_max_len_fit": naive, "paged_fit": admitted,
                "gain": round(admitted / max(naive, 1), 2),
                "reserve_waste_frac": round(1 - float(lens[:naive].sum()) / (naive * max_len), 4) if naive else None,
                "paged_waste_frac": round(1 - tokens / (used_blocks * block_size), 5) if used_blocks else None}

    return {"workload": f"Llama-2-13B shape, {per_token} KV bytes a token, fp16 weights {weight_bytes / 1e9:.0f} GB, "
                        f"requests U[1,{max_len}] tokens in arrival order, block {block_size}",
            "mi355x_288gb": fit(hbm_bytes), "context_40gb_device": fit(40e9)}


def host_timings(w, pa, np, trials=7):
    """Block-manager call times of one decode iteration of the batch, through
    the Python binding, as medians over `trials` fresh pools: admitting a
    context (per sequence), reserving the step's 64 new tokens in one batched
    call, and exporting the tables."""
    admit, reserve, export = [], [], []
    max_blocks = -(-int(w.lens.max()) // 16)
    for _ in range(trials):
        pool = pa.pa_pool_create(w.num_blocks, 16, w.init_free_order)
        ids = []
        for b in range(w.batch):
            s = pa.pa_seq_create(pool)
            ids.append(s)
            t0 = time.perf_counter()
            pa.pa_alloc_append(pool, s, int(w.lens[b]) - 1)
            admit.append(time.perf_counter() - t0)
        t0 = time.perf_counter()
        pa.pa_alloc_append_batch(pool, ids, [1] * len(ids))
        reserve.append(time.perf_counter() - t0)
        for _ in range(3):
            t0 = time.perf_counter()
            pa.pa_block_tables(pool, ids, max_blocks)
            export.append(time.perf_counter() - t0)
    return {"admit_us_per_seq": round(1e6 * float(np.median(admit)), 2),
            "step_reserve_us": round(1e6 * float(np.median(reserve)), 2),
            "table_export_us": round(1e6 * float(np.median(export)), 2),
            "timing": f"medians over {trials} fresh pools, Python binding included"}


def setup_decode(w, fp8: bool, pa, torch, np, block_size=16):
    """Admit every sequence with its context minus the newest token, write that
    KV, then allocate the newest token (the step's write target)."""
    nb, order = pool_geometry(w, block_size, np)
    pool = pa.pa_pool_create(nb, block_size, order)
    ks, vs = fp8_scales(w, np) if fp8 else (1.0, 1.0)
    cache = pa.KvCache(nb, w.num_kv_heads, w.head_dim, block_size=block_size, fp8=fp8, k_scale=ks,
                       v_scale=vs)
    ids, new_k, new_v, new_slots = [], [], [], []
    for b in range(w.batch):
        s = pa.pa_seq_create(pool)
        ids.append(s)
        k, v = w.kv(b)
        L = int(w.lens[b])
        slots, _ = pa.pa_alloc_append(pool, s, L - 1)
        if L > 1:
            pa.pa_write_kv(cache, torch.from_numpy(k[:L - 1]).cuda(), torch.from_numpy(v[:L - 1]).cuda(),
                           torch.from_numpy(slots).cuda())
        new_k.append(k[L - 1:])
        new_v.append(v[L - 1:])
    # the step's reservations: one batched call for every sequence
    slots, _ = pa.pa_alloc_append_batch(pool, ids, [1] * len(ids))
    new_slots = [int(x) for x in slots]
    max_ctx = int(w.lens.max())
    max_blocks = -(-max_ctx // block_size)
    tables, lens = pa.pa_block_tables(pool, ids, max_blocks)
    torch.cuda.synchronize()
    d = {
        "pool": pool, "cache": cache,
        "k_new": torch.from_numpy(np.ascontiguousarray(np.concatenate(new_k))).cuda(),
        "v_new": torch.from_numpy(np.ascontiguousarray(np.concatenate(new_v))).cuda(),
        "slots": torch.tensor(new_slots, dtype=torch.int32, device="cuda"),
        "tables": torch.from_numpy(tables).cuda(), "lens": torch.from_numpy(lens).cuda(),
        "q": torch.from_numpy(w.q).cuda(), "max_ctx": max_ctx,
        "out": torch.empty((w.batch, w.num_heads, w.head_dim), dtype=torch.float32, device="cuda"),
    }
    nbytes = pa.pa_decode_workspace_bytes(w.batch, w.num_heads, w.head_dim, max_ctx)
    d["ws"] = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    return d


SETTLE_S = 0.25  # seconds of untimed work that bring the GPU to its steady clock


def settle(torch, fn, seconds=SETTLE_S):
    """Run fn back to back until `seconds` have passed.  After a pause (the
    host-side set-up of a leg), the GPU needs tens of milliseconds of load to
    return to its steady clock; without this a short timed region measures
    the ramp (the prefill leg reads about 25% slow)."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


def decode_call(pa, w, d):
    pa.pa_decode(d["cache"], d["q"], d["tables"], d["lens"], d["max_ctx"], w.scale, d["out"], d["ws"],
                 cached_blocks=d.get("cached"))


def append_call(pa, w, d):
    pa.pa_decode_append(d["cache"], d["q"], d["k_new"], d["v_new"], d["tables"], d["lens"], d["max_ctx"],
                        w.scale, d["out"], d["ws"], cached_blocks=d.get("cached"))


def time_region(torch, fn, steps, warmup):
    """Untimed settle and warm-up, then `steps` calls of fn back to back,
    bracketed by a synchronisation and one HIP event pair on the current
    stream (the stream the library launches on).  No event sits between two
    calls, so the region holds only the calls' own work and launch gaps
    (recording an event pair around every call added about 7 us per call).
    Returns (wall-clock ms per call, event ms per call)."""
    settle(torch, fn)
    for _ in range(warmup):
        fn()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return 1e3 * (t1 - t0) / steps, start.elapsed_time(end) / steps


def run_decode(pa, torch, w, d, steps, warmup, fused=True):
    """Decode steps back to back: each writes the new tokens' K/V and attends
    over every context.  fused: one pa_decode_append launch per step (so the
    event time per step is that kernel's average launch duration); else
    pa_write_kv then pa_decode.  Returns (wall ms per step, event ms per step)."""
    if fused:
        return time_region(torch, lambda: append_call(pa, w, d), steps, warmup)

    def step():
        pa.pa_write_kv(d["cache"], d["k_new"], d["v_new"], d["slots"])
        decode_call(pa, w, d)

    return time_region(torch, step, steps, warmup)


def decode_bytes(w, elem_bytes, lens=None, block_size=16, fused=False):
    """(KV bytes of the contexts, algorithmic bytes of one launch).  pa_decode:
    K and V rows of every cached token read once, q read, fp32 output written,
    block tables and lengths read (split partials, when used, are not
    algorithmic).  pa_decode_append: the same, except that each sequence's new
    token is read from k_new / v_new (fp16) and written to the cache instead
    of read from it."""
    lens = w.lens if lens is None else lens
    row = w.num_kv_heads * w.head_dim * 2        # K and V values of one token
    kv = int(lens.sum()) * row * elem_bytes
    io = w.batch * w.num_heads * w.head_dim * (2 + 4)
    tables = w.batch * (-(-int(lens.max()) // block_size)) * 4 + w.batch * 4
    if not fused:
        return kv, kv + io + tables
    new = int((lens > 0).sum())
    return kv, kv - new * row * elem_bytes + new * row * (2 + elem_bytes) + io + tables


def time_events(torch, fn, reps, warmup=3):
    """Event ms per call of fn over `reps` back-to-back calls (time_region)."""
    return time_region(torch, fn, reps, warmup)[1]


def copy_ceiling(torch, nbytes=1 << 30, reps=20):
    """A plain device copy (one elementwise kernel) as the bandwidth context."""
    src = torch.ones(nbytes // 2, dtype=torch.float16, device="cuda")
    dst = torch.empty_like(src)
    mean = time_events(torch, lambda: torch.neg(src, out=dst), reps)
    del src, dst
    return {"kind": "torch.neg over 1 GiB fp16 (read 1 GiB + write 1 GiB)",
            "gbs_read_plus_write": round(2 * nbytes / (mean * 1e-3) / 1e9, 1), "ms": round(mean, 4)}


def read_ceiling(torch, nbytes=1 << 30, reps=20):
    """A read-bound device kernel for context: torch's row sums over 1 GiB of
    fp16 laid out as 8192 rows of 65536 (reads 1 GiB, writes 16 KiB).  Of the
    torch reductions and products over this buffer it is the fastest reader
    on this part; a full-length sum reaches only about 60% of its rate."""
    src = torch.ones(nbytes // 2, dtype=torch.float16, device="cuda").view(-1, 65536)
    acc = torch.empty(src.shape[0], dtype=torch.float16, device="cuda")
    mean = time_events(torch, lambda: torch.sum(src, dim=1, out=acc), reps)
    del src, acc
    return {"kind": "torch.sum over rows of a 1 GiB fp16 matrix (8192 x 65536): read 1 GiB",
            "gbs_read": round(nbytes / (mean * 1e-3) / 1e9, 1), "ms": round(mean, 4)}


def achievable_read(pa, torch, np, reps=20, n_tiles=330000, per_wave=8, cold=False):
    """The library's read-only probe kernel (pa_probe_tile_gather) with the
    decode's access pattern: 4 KiB tiles in a seeded random order over 1.35 GB,
    8 tiles per wave, non-temporal loads -- the practical read ceiling.  Timed
    back to back (gbs_read), and with cold=True also as the headline step is,
    a 1 GiB flush before each call (gbs_read_cold, the median)."""
    base = torch.empty(n_tiles * 4096, dtype=torch.uint8, device="cuda")
    base.fill_(1)
    ids = torch.from_numpy(np.random.default_rng(7).permutation(n_tiles).astype(np.int32)).cuda()
    sink = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    fn = lambda: pa.pa_probe_tile_gather(base, ids, per_wave, sink)
    mean = time_events(torch, fn, reps)
    nbytes = n_tiles * 4096
    res = {"kind": f"pa_probe_tile_gather: {n_tiles} 4 KiB tiles ({nbytes / 1e9:.2f} GB) in random order, "
                   f"{per_wave} per wave, non-temporal loads",
           "gbs_read": round(nbytes / (mean * 1e-3) / 1e9, 1), "ms": round(mean, 4)}
    if cold:
        per, _ = cold_region(torch, np, fn, reps, 3)
        ms_cold = float(np.median(per))
        res["gbs_read_cold"] = round(nbytes / (ms_cold * 1e-3) / 1e9, 1)
        res["ms_cold"] = round(ms_cold, 4)
    del base, ids, sink
    return res


def achievable_mfma(pa, torch, n_workgroups=1024, iters=20000, reps=5):
    """The library's matrix-core probe (pa_probe_mfma): fp16 16x16x32 MFMAs on
    register operands, 4 waves per SIMD -- the fp16 matrix throughput the part
    sustains, clock under matrix load included."""
    sink = torch.zeros(64, dtype=torch.float32, device="cuda")
    mean = time_events(torch, lambda: pa.pa_probe_mfma(n_workgroups, iters, sink), reps, warmup=2)
    flop = float(n_workgroups) * iters * pa.PA_PROBE_MFMA_FLOP
    tf = flop / (mean * 1e-3) / 1e12
    return {"kind": f"pa_probe_mfma: {n_workgroups} x 4 waves, {iters} x 8 MFMAs a wave (fp16 16x16x32, "
                    "register operands)",
            "tflops": round(tf, 1), "frac_of_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4), "ms": round(mean, 4)}


FLUSH_BYTES = 1 << 30


def cold_region(torch, np, fn, steps, warmup):
    """The headline timing: every step starts with cold caches.  Before each
    step 1 GiB of unrelated writes (four times the 256 MB last-level cache)
    evicts what the previous step left in L2 and the MALL, then an event pair
    brackets the step's launch alone.  The K timed steps sit between two
    synchronisations.  Returns (per-step event ms array, wall ms of the whole
    region per step, including the flushes).  Per-launch event pairs read
    about 2 us long on this part, so the figure is conservative."""
    junk = torch.empty(FLUSH_BYTES // 2, dtype=torch.float16, device="cuda")
    settle(torch, fn)
    for _ in range(warmup):
        junk.fill_(1.0)
        fn()
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in pairs:
        junk.fill_(1.0)
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    del junk
    return np.array([a.elapsed_time(b) for a, b in pairs]), 1e3 * (t1 - t0) / steps


def setup_prefix(w, fp8, pa, torch, np):
    """``w.batch`` sequences fork one ``w.prompt_len``-token prompt and append
    private tails; one decode query each.  The prompt's blocks are stored once
    and read by every sequence.  e4m3 caches take per-tensor scales from the
    largest |K| and |V| over the prompt and the tails."""
    pool = pa.pa_pool_create(w.num_blocks, 16)
    pk, pv = w.prompt_kv()
    ks = vs = 1.0
    if fp8:
        ka, va = np.abs(pk.astype(np.float32)).max(), np.abs(pv.astype(np.float32)).max()
        for b in range(w.batch):
            k, v = w.kv(b)
            ka = max(ka, np.abs(k.astype(np.float32)).max())
            va = max(va, np.abs(v.astype(np.float32)).max())
        ks, vs = float(np.float32(ka / np.float32(448))), float(np.float32(va / np.float32(448)))
    cache = pa.KvCache(w.num_blocks, w.num_kv_heads, w.head_dim, fp8=fp8, k_scale=ks, v_scale=vs)
    root = pa.pa_seq_create(pool)
    slots, _ = pa.pa_alloc_append(pool, root, w.prompt_len)
    pa.pa_write_kv(cache, torch.from_numpy(pk).cuda(), torch.from_numpy(pv).cuda(), torch.from_numpy(slots).cuda())
    seqs = [root] + [pa.pa_fork_cow(pool, root) for _ in range(w.batch - 1)]
    for b, s in enumerate(seqs):
        k, v = w.kv(b)
        slots, cow = pa.pa_alloc_append(pool, s, int(w.tails[b]))
        pa.pa_write_kv(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(),
                       torch.from_numpy(slots).cuda(), [cow] if cow else None)
    max_ctx = int(w.lens.max())
    tables, lens = pa.pa_block_tables(pool, seqs, -(-max_ctx // 16))
    stats, _, _ = pa.pa_pool_state(pool)
    d = {"pool": pool, "seqs": seqs, "stats": stats, "cache": cache, "q": torch.from_numpy(w.q).cuda(),
         "tables": torch.from_numpy(tables).cuda(), "lens": torch.from_numpy(lens).cuda(), "max_ctx": max_ctx,
         "out": torch.empty((w.batch, w.num_heads, w.head_dim), dtype=torch.float32, device="cuda"),
         "ws": torch.empty(max(16, pa.pa_decode_workspace_bytes(w.batch, w.num_heads, w.head_dim, max_ctx)),
                           dtype=torch.uint8, device="cuda")}
    return d


def prefix_hint(pa, torch, d):
    """Turn on the shared-prefix hint: the prompt's blocks are read through the caches."""
    d["cached"] = torch.from_numpy(pa.pa_shared_prefix(d["pool"], d["seqs"])).cuda()


def bench_prefix(pa, torch, np, workloads, reps, fp8=False):
    """The shared-prompt decode (32 sequences over one 800-token prompt):
    warm (back to back) without and with the shared-prefix hint, and cold
    (1 GiB flush before each call) with the hint."""
    w = workloads.prefix_cow()
    d = setup_prefix(w, fp8, pa, torch, np)
    mean_nt = time_events(torch, lambda: decode_call(pa, w, d), reps)
    prefix_hint(pa, torch, d)
    mean = time_events(torch, lambda: decode_call(pa, w, d), reps)
    cold, _ = cold_region(torch, np, lambda: decode_call(pa, w, d), reps, 5)
    cold_med = float(np.median(cold))
    per_tok = w.num_kv_heads * w.head_dim * 2 * (1 if fp8 else 2)
    logical = int(w.lens.sum()) * per_tok
    unique = (w.prompt_len + int(w.tails.sum())) * per_tok
    return {"workload": "prefix_cow: 32 seqs share an 800-token prompt (50 blocks, ref_cnt 32), "
                        f"tails U[1,1024], 40 heads x 128, {'e4m3' if fp8 else 'fp16'}",
            "pa_decode_ms": round(mean, 5),
            "pa_decode_ms_without_hint": round(mean_nt, 5),
            "pa_decode_ms_cold": round(cold_med, 5),
            "unique_kv_bytes": unique, "logical_kv_bytes": logical,
            "unique_gbs": round(unique / (mean * 1e-3) / 1e9, 2),
            "unique_gbs_cold": round(unique / (cold_med * 1e-3) / 1e9, 2),
            "logical_gbs": round(logical / (mean * 1e-3) / 1e9, 2),
            "used_blocks": d["stats"]["used_blocks"], "shared_blocks": d["stats"]["shared_blocks"],
            "timing": "warm: one event pair over back-to-back calls; cold: median of per-call "
                      "event pairs, 1 GiB flush before each"}


def bench_prefix_cache(pa, np, workloads):
    """Host-side prefix caching over multi-turn dialogues: every turn admits its
    prompt with pa_alloc_prompt (reusing the conversation's cached blocks),
    commits, appends the reply with pa_append_tokens, commits and finishes.
    Reports the hit rate (reused prompt tokens / prompt tokens) and the block
    manager's call times; the K/V writes are not part of this leg."""
    d = workloads.dialogue()
    t_prompt, t_other = [], []
    for rep in range(5):  # the same replay on a fresh pool; per-call medians over all of them
        pool = pa.pa_pool_create(d.num_blocks, 16)
        for t in range(len(d.turns[0])):
            for c in range(len(d.turns)):
                prompt, reply = d.turns[c][t]
                s = pa.pa_seq_create(pool)
                t0 = time.perf_counter()
                pa.pa_alloc_prompt(pool, s, prompt)
                t1 = time.perf_counter()
                pa.pa_cache_commit(pool, s)
                pa.pa_append_tokens(pool, s, reply)
                pa.pa_cache_commit(pool, s)
                pa.pa_seq_free(pool, s)
                t2 = time.perf_counter()
                t_prompt.append(t1 - t0)
                t_other.append(t2 - t1)
        st, _, _ = pa.pa_pool_state(pool)
    return {"workload": f"dialogue: {len(d.turns)} conversations x {len(d.turns[0])} turns, first prompt "
                        "U[200,600], replies U[20,200], messages U[10,100] tokens",
            "prompt_tokens": st["prompt_tokens"], "hit_tokens": st["hit_tokens"],
            "hit_rate": round(st["hit_tokens"] / max(1, st["prompt_tokens"]), 4),
            "cached_blocks": st["cached_blocks"], "evictions": st["evictions"],
            "alloc_prompt_us": round(1e6 * float(np.median(t_prompt)), 2),
            "commit_append_free_us": round(1e6 * float(np.median(t_other)), 2),
            "timing": "median per call over 5 replays, Python binding included"}


def bench_preemption(pa, torch, np, workloads, reps=10):
    """Preemption of one 2048-token sequence at the 13B shape (128 blocks, 40 MiB
    of fp16 K/V per layer): swap out to pinned host memory and back in
    (pa_swap_out / pa_swap_in + pa_swap_blocks), against the attention-side
    part of recomputing it (K/V write + chunked prefill, 4 x 512 tokens) for one
    layer.  The model's own projections, which recomputation also repeats, are
    not part of this library and not timed."""
    L, H, D = 2048, 40, 128
    nblk = L // 16
    pool = pa.pa_pool_create(nblk + 16, 16)
    cache = pa.KvCache(nblk + 16, H, D)
    rng = np.random.default_rng(1007)
    k = torch.from_numpy(rng.standard_normal((L, H, D), dtype=np.float32).astype(np.float16)).cuda()
    v = torch.from_numpy(rng.standard_normal((L, H, D), dtype=np.float32).astype(np.float16)).cuda()
    q = torch.from_numpy(rng.standard_normal((L, H, D), dtype=np.float32).astype(np.float16)).cuda()
    s = pa.pa_seq_create(pool)
    slots, _ = pa.pa_alloc_append(pool, s, L)
    pa.pa_write_kv(cache, k, v, torch.from_numpy(slots).cuda())
    host_k = torch.empty((nblk, H, 16, D), dtype=torch.float16, pin_memory=True)
    host_v = torch.empty_like(host_k, pin_memory=True)
    pa.pa_swap_space(pool, nblk)

    def swap_cycle():
        t0 = time.perf_counter()
        pa.pa_swap_blocks(cache, host_k, host_v, pa.pa_swap_out(pool, s), 0)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        pa.pa_swap_blocks(cache, host_k, host_v, pa.pa_swap_in(pool, s), 1)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        return t1 - t0, t2 - t1

    for _ in range(3):
        swap_cycle()
    outs, ins = zip(*[swap_cycle() for _ in range(reps)])
    t_out, t_in = sorted(outs)[reps // 2], sorted(ins)[reps // 2]
    nbytes = 2 * nblk * H * 16 * D * 2
    tables, _ = pa.pa_block_tables(pool, [s], nblk)
    tables = torch.from_numpy(tables).cuda()
    out = torch.empty((512, H, D), dtype=torch.float32, device="cuda")
    cu = torch.tensor([0, 512], dtype=torch.int32, device="cuda")
    priors = [torch.tensor([c * 512], dtype=torch.int32, device="cuda") for c in range(4)]
    slots_d = torch.from_numpy(slots).cuda()
    scale = 1.0 / np.sqrt(D)

    def recompute():
        pa.pa_write_kv(cache, k, v, slots_d)
        for c in range(4):
            pa.pa_prefill_chunk(cache, q[c * 512:(c + 1) * 512], cu, priors[c], tables, 512, scale, out)

    mean = time_events(torch, recompute, reps)
    return {"workload": "one 2048-token sequence, 40 KV heads x 128, fp16: 128 blocks, "
                        f"{nbytes / 2**20:.0f} MiB of K/V per layer",
            "swap_out_ms": round(1e3 * t_out, 3), "swap_in_ms": round(1e3 * t_in, 3),
            "swap_out_gbs": round(nbytes / t_out / 1e9, 2), "swap_in_gbs": round(nbytes / t_in / 1e9, 2),
            "recompute_attention_ms_per_layer": round(mean, 3)}


def bench_mixed(pa, torch, np, workloads, reps, fp8=False):
    """A continuous-batching step: the chunked-prefill batch (8 x 512 rows) and
    the 13B-shaped decode batch (64 sequences) over one cache, as one
    pa_mixed_step call against pa_prefill_chunk followed by pa_decode."""
    wp, wd = workloads.chunked_prefill(), workloads.llama13b_decode()
    n = wp.num_blocks + wd.num_blocks
    pool = pa.pa_pool_create(n, 16)
    ks = vs = 1.0
    if fp8:
        (k1, v1), (k2, v2) = fp8_scales(wp, np), fp8_scales(wd, np)
        ks, vs = max(k1, k2), max(v1, v2)
    cache = pa.KvCache(n, wd.num_kv_heads, wd.head_dim, fp8=fp8, k_scale=ks, v_scale=vs)
    pids, dids = [], []
    for b in range(wp.batch):
        s = pa.pa_seq_create(pool)
        pids.append(s)
        k, v = wp.kv(b)
        slots, _ = pa.pa_alloc_append(pool, s, int(wp.lens[b]))
        pa.pa_write_kv(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), torch.from_numpy(slots).cuda())
    for b in range(wd.batch):
        s = pa.pa_seq_create(pool)
        dids.append(s)
        k, v = wd.kv(b)
        slots, _ = pa.pa_alloc_append(pool, s, int(wd.lens[b]))
        pa.pa_write_kv(cache, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), torch.from_numpy(slots).cuda())
    tp, _ = pa.pa_block_tables(pool, pids, -(-int(wp.lens.max()) // 16))
    max_ctx = int(wd.lens.max())
    td, lens = pa.pa_block_tables(pool, dids, -(-max_ctx // 16))
    cu = np.concatenate([[0], np.cumsum(wp.chunk)]).astype(np.int32)
    prefill = dict(q=torch.from_numpy(wp.q).cuda(), cu_q=torch.from_numpy(cu).cuda(),
                   prior=torch.from_numpy(wp.prior.astype(np.int32)).cuda(), tables=torch.from_numpy(tp).cuda(),
                   max_chunk=int(wp.chunk.max()),
                   out=torch.empty((int(cu[-1]), wp.num_heads, wp.head_dim), dtype=torch.float32, device="cuda"))
    decode = dict(q=torch.from_numpy(wd.q).cuda(), tables=torch.from_numpy(td).cuda(),
                  lens=torch.from_numpy(lens).cuda(), max_context_len=max_ctx,
                  out=torch.empty((wd.batch, wd.num_heads, wd.head_dim), dtype=torch.float32, device="cuda"),
                  workspace=torch.empty(max(16, pa.pa_decode_workspace_bytes(wd.batch, wd.num_heads, wd.head_dim,
                                                                             max_ctx)), dtype=torch.uint8,
                                        device="cuda"))
    scale = wp.scale

    def separate():
        pa.pa_prefill_chunk(cache, prefill["q"], prefill["cu_q"], prefill["prior"], prefill["tables"],
                            prefill["max_chunk"], scale, prefill["out"])
        pa.pa_decode(cache, decode["q"], decode["tables"], decode["lens"], max_ctx, scale, decode["out"],
                     decode["workspace"])

    mixed_ms = time_events(torch, lambda: pa.pa_mixed_step(cache, scale, prefill, decode), reps)
    sep_ms = time_events(torch, separate, reps)
    return {"workload": "chunked_prefill (8 x 512 rows) + llama13b_decode (64 seqs) over one "
                        f"{'e4m3' if fp8 else 'fp16'} cache",
            "mixed_ms": round(mixed_ms, 4), "separate_ms": round(sep_ms, 4),
            "speedup": round(sep_ms / mixed_ms, 3)}


def bench_prefill(pa, torch, np, workloads, reps, block_size=16, fp8=False):
    w = workloads.chunked_prefill()
    nb, order = pool_geometry(w, block_size, np)
    pool = pa.pa_pool_create(nb, block_size, order)
    ks, vs = fp8_scales(w, np) if fp8 else (1.0, 1.0)
    cache = pa.KvCache(nb, w.num_kv_heads, w.head_dim, block_size=block_size, fp8=fp8, k_scale=ks,
                       v_scale=vs)
    ids = []
    for b in range(w.batch):
        s = pa.pa_seq_create(pool)
        ids.append(s)
        k, v = w.kv(b)
        P, C = int(w.prior[b]), int(w.chunk[b])
        for lo, n in ((0, P), (P, C)):
            slots, _ = pa.pa_alloc_append(pool, s, n)
            if n:
                pa.pa_write_kv(cache, torch.from_numpy(np.ascontiguousarray(k[lo:lo + n])).cuda(),
                               torch.from_numpy(np.ascontiguousarray(v[lo:lo + n])).cuda(),
                               torch.from_numpy(slots).cuda())
    max_blocks = -(-int(w.lens.max()) // block_size)
    tables, _ = pa.pa_block_tables(pool, ids, max_blocks)
    tables = torch.from_numpy(tables).cuda()
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(w.chunk)]).astype(np.int32)).cuda()
    prior = torch.from_numpy(w.prior.astype(np.int32)).cuda()
    q = torch.from_numpy(w.q).cuda()
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    mean = time_events(
        torch, lambda: pa.pa_prefill_chunk(cache, q, cu, prior, tables, int(w.chunk.max()), w.scale, out), reps)
    C = w.chunk.astype(np.float64)
    P = w.prior.astype(np.float64)
    flops = 4.0 * w.head_dim * w.num_heads * float(np.sum(C * P + C * (C + 1) / 2))
    tflops = flops / (mean * 1e-3) / 1e12
    return {"workload": "chunked_prefill: 8 seqs, prior U[0,4096], chunk 512, 40 heads x 128, "
                        + ("e4m3 cache" if fp8 else "fp16"),
            "ms": round(mean, 4),
            "causal_gflop": round(flops / 1e9, 3), "tflops": round(tflops, 2),
            "mfma_util": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
            "peak_tflops": MFMA_F16_PEAK_TFLOPS}


def bench_block_sizes(pa, torch, np, workloads, w, steps, warmup, at16):
    """The 13B decode batch and the chunked-prefill batch at block sizes 8, 32
    and 64 (16 is the headline line): pa_decode bandwidth, the slots lost to
    partly filled last blocks, and prefill time."""
    res = {}
    for bs in (8, 16, 32, 64):
        if bs == 16:
            d_ms, p_ms = at16
        else:
            d = setup_decode(w, False, pa, torch, np, block_size=bs)
            _, d_ms = time_region(torch, lambda: decode_call(pa, w, d), steps, warmup)
            del d
            torch.cuda.empty_cache()
            p_ms = bench_prefill(pa, torch, np, workloads, 20, block_size=bs)["ms"]
        _, alg = decode_bytes(w, 2, block_size=bs)
        blocks = int(np.sum(-(-w.lens // bs)))
        res[str(bs)] = {"pa_decode_ms": round(d_ms, 5),
                        "pa_decode_gbs": round(alg / (d_ms * 1e-3) / 1e9, 2),
                        "hbm_frac": round(alg / (d_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "blocks": blocks, "waste_tokens": blocks * bs - int(w.lens.sum()),
                        "waste_frac": round(1.0 - int(w.lens.sum()) / (blocks * bs), 5),
                        "prefill_ms": round(p_ms, 4)}
    return {"workload": "llama13b_decode (64 seqs, fp16) and chunked_prefill (8 x 512 rows)", **res}


def _oracle_warm(_):
    """Worker start-up of cpu_baseline_pool, kept out of its timed region."""
    import oracle  # noqa: F401
    import workloads
    workloads.llama13b_decode()
    return os.getpid()


def _oracle_seqs(bs):
    """Worker of cpu_baseline_pool: the oracle for sequences bs of the batch."""
    from threadpoolctl import threadpool_limits
    from oracle import OracleCache, OraclePool, paged_decode
    import workloads as wl
    w = wl.llama13b_decode()
    done = 0
    with threadpool_limits(limits=1):
        for b in bs:
            k, v = w.kv(b)
            L = int(w.lens[b])
            nblk = -(-L // 16)
            pool = OraclePool(nblk, 16)
            cache = OracleCache(nblk, w.num_kv_heads, w.head_dim)
            _, s = pool.seq_create()
            _, slots, _ = pool.alloc_append(s, L)
            cache.write(slots, k, v)
            paged_decode(cache, [pool.table(s)], [L], w.q[b:b + 1], w.scale)
            done += L * w.num_kv_heads * w.head_dim * 2 * 2
    return done


def cpu_baseline_pool(w, np, procs=None):
    """The same oracle over all 64 sequences with a process pool (one
    single-threaded process per core of the host share, 16 at most)."""
    import multiprocessing as mp
    procs = procs or max(1, min(16, len(os.sched_getaffinity(0))))
    order = list(np.argsort(-w.lens))                  # longest first, dealt round robin
    parts = [[int(b) for b in order[i::procs]] for i in range(procs)]
    ctx = mp.get_context("spawn")                      # no fork of a process that holds the GPU
    with ctx.Pool(procs) as pool:
        pool.map(_oracle_warm, range(procs), chunksize=1)
        t0 = time.perf_counter()
        done = sum(pool.map(_oracle_seqs, parts, chunksize=1))
        elapsed = time.perf_counter() - t0
    return {"value": round(done / elapsed / 1e9, 5), "unit": "GB/s", "cores": procs, "kind": "oracle",
            "tokens_per_s": round(w.batch / elapsed, 2),
            "sample": f"all {w.batch} sequences, {procs} processes x 1 thread, float64 numpy, "
                      f"{elapsed:.1f} s after worker start-up",
            "seconds": round(elapsed, 2)}


def cpu_baseline(w, np, target_s=15.0):
    """The float64 oracle, as it stands, on a bounded sample of the batch:
    allocator model + cache model + paged gather + attention for the first
    sequences (in batch order) until about target_s of CPU time."""
    from threadpoolctl import threadpool_limits
    from oracle import OracleCache, OraclePool, paged_decode

    with threadpool_limits(limits=1):
        t_start = time.perf_counter()
        done_bytes = 0
        done_seqs = 0
        tokens = 0
        for b in range(w.batch):
            k, v = w.kv(b)
            L = int(w.lens[b])
            nblk = -(-L // 16)
            pool = OraclePool(nblk, 16)
            cache = OracleCache(nblk, w.num_kv_heads, w.head_dim)
            _, s = pool.seq_create()
            _, slots, _ = pool.alloc_append(s, L)
            cache.write(slots, k, v)
            paged_decode(cache, [pool.table(s)], [L], w.q[b:b + 1], w.scale)
            done_bytes += L * w.num_kv_heads * w.head_dim * 2 * 2
            tokens += L
            done_seqs += 1
            if time.perf_counter() - t_start > target_s:
                break
        elapsed = time.perf_counter() - t_start
    return {"value": round(done_bytes / elapsed / 1e9, 5), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "tokens_per_s": round(done_seqs / elapsed, 2),
            "sample": f"first {done_seqs} of {w.batch} sequences ({tokens} tokens, all 40 heads), "
                      f"{elapsed:.1f} s, float64 numpy, BLAS limited to 1 thread",
            "seconds": round(elapsed, 2)}


PMC_WORKLOADS = {
    # name: (description, tracked summary file)
    "step_fp16": ("pa_decode_append on llama13b_decode (64 seqs, L ~ U[1,2048], 40 x 128, fp16)",
                  "decode_llama13b_fp16_traffic.md"),
    "step_e4m3": ("pa_decode_append on llama13b_decode (64 seqs, L ~ U[1,2048], 40 x 128, e4m3 cache)",
                  "decode_llama13b_e4m3_traffic.md"),
    "prefix_fp16": ("pa_decode with the shared-prefix hint on prefix_cow (32 seqs over one 800-token "
                    "prompt, tails U[1,1024], 40 x 128, fp16)", "decode_prefix_cow_fp16_traffic.md"),
    "prefix_e4m3": ("pa_decode with the shared-prefix hint on prefix_cow (32 seqs over one 800-token "
                    "prompt, tails U[1,1024], 40 x 128, e4m3 cache)", "decode_prefix_cow_e4m3_traffic.md"),
}


def pmc_run(pa, torch, np, workloads, name):
    """Only what the counter runs need: one copy of known size, then
    PMC_DECODE_STEPS decode calls of one workload (PMC_WORKLOADS)."""
    src = torch.ones(PMC_COPY_BYTES // 2, dtype=torch.float16, device="cuda")
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    fp8 = name.endswith("e4m3")
    if name.startswith("step"):
        w = workloads.llama13b_decode()
        d = setup_decode(w, fp8, pa, torch, np)
        call = lambda: append_call(pa, w, d)
    else:
        w = workloads.prefix_cow()
        d = setup_prefix(w, fp8, pa, torch, np)
        prefix_hint(pa, torch, d)
        call = lambda: decode_call(pa, w, d)
    torch.cuda.synchronize()
    for _ in range(PMC_DECODE_STEPS):
        call()
    torch.cuda.synchronize()
    log(f"pmc run done: copy {PMC_COPY_BYTES} B, {PMC_DECODE_STEPS} decode calls of {name}")


def pmc_reference_bytes(name, np, workloads):
    """(label, bytes) pairs the counted traffic is compared with."""
    elt = 1 if name.endswith("e4m3") else 2
    if name.startswith("step"):
        w = workloads.llama13b_decode()
        kv, alg = decode_bytes(w, elt, fused=True)
        return [("K/V bytes of the contexts", kv), ("algorithmic bytes of the launch", alg)]
    w = workloads.prefix_cow()
    per_tok = w.num_kv_heads * w.head_dim * 2 * elt
    return [("unique K/V bytes (prompt stored once)", (w.prompt_len + int(w.tails.sum())) * per_tok),
            ("logical K/V bytes (prompt counted per sequence)", int(w.lens.sum()) * per_tok)]


def _read_counter_csv(path, counter):
    """{kernel name: [value per dispatch]} for one counter of a rocprofv3 CSV."""
    out = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return out


def _short_kernel(n):
    if n.startswith("void at::native::vectorized_elementwise_kernel<8, at::native::neg"):
        return "torch neg (elementwise copy)"
    if "FillFunctor" in n:
        return "torch fill"
    m = re.match(r"_ZN2pa12_GLOBAL__N_1\d+(\w+?)(I.*)$", n)
    if m:
        return f"pa::{m.group(1)} {m.group(2)[:60]}"
    return n[:70]


def summarize_trace(trace_dir, bench_log, out_md):
    """Write the kernel-time summary from a rocprofv3 --kernel-trace run of this
    script (its kernel_trace CSV) and the JSON line the same run printed."""
    trace_csv = sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True),
                       key=os.path.getmtime)[-1]
    with open(trace_csv) as f:
        recs = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    # one row per kernel, grid size (one kernel's workloads stay apart) and
    # whether the dispatch right before it was the cold legs' 1 GiB fill
    groups = {}
    prev = None
    for r in recs:
        wgs = int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"])
        cold = prev is not None and "FillFunctor" in prev["Kernel_Name"] and \
            int(prev["Grid_Size_X"]) >= 1 << 22   # the flush, not a small zero fill
        key = (r["Kernel_Name"], wgs, cold)
        groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        prev = r
    rows = [{"name": n, "wgs": w, "cold": c, "calls": len(d), "avg": sum(d) / len(d), "min": min(d),
             "max": max(d), "total": sum(d)} for (n, w, c), d in groups.items()]
    rows.sort(key=lambda r: -r["total"])
    everything = sum(r["total"] for r in rows)
    rows = [r for r in rows if r["cold"] or r["total"] > 0.002 * everything]
    total = sum(r["total"] for r in rows)
    with open(bench_log) as f:
        b = json.loads([line for line in f if line.startswith("{")][-1])
    roof, pc, pf, f8 = b["roofline"], b.get("prefix_cow", {}), b.get("prefill", {}), b.get("fp8_decode", {})
    body = f"""# Kernel trace: bench.py on llama13b_decode (+ fp8, prefix-sharing, mixed, prefill, block-size legs)

Commands (repository root, on the MI355X):

    rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_decode -o run -- python -u bench.py --steps 20 --warmup 3 --no-cpu-baseline > gpurun_out/prof_decode.log
    python bench.py --summarize-trace gpurun_out/prof_decode gpurun_out/prof_decode.log {out_md}

Template arguments of the decode kernels: <head_dim, e4m3, units per step, pipelined, waves per
workgroup, block-id registers, block size, appending>.  decode_seq_kernel<128,0,2,0,4,1,16,1> is
the fp16 13B-shaped decode step (pa_decode_append, the roofline kernel) and <...,16,0> the same
batch through pa_decode after pa_write_kv; <128,1,1,0,4,1,16,1> the e4m3 step; <128,0,2,0,8,1,16,0> the
800-token shared-prompt decode (32 x 40 pairs, 8 waves per workgroup; timed without and with the
shared-prefix hint, so its row averages both); the block-size legs add the same kernels at block
sizes 8, 32 and 64.  prefill_pp_kernel<head_dim, block size> with 640 workgroups is the 8 x 512-row
chunked prefill over an fp16 cache, prefill_kernel<head_dim, block size, 1> with 1280 the same over
an e4m3 cache; mixed_step_kernel runs the prefill and the 13B-shaped decode in one launch.
tile_gather_kernel is the read probe of the achievable-bandwidth figure (pa_probe_tile_gather),
mfma_loop_kernel the matrix-core probe of the achievable-MFMA figure (pa_probe_mfma).

One row per kernel, grid size (workgroups) and cache state; warm rows under 0.2% of GPU time are
left out.  "cold" rows hold the dispatches that directly follow the 1 GiB fill of a cold-timed leg
(the warm-up and timed steps of the headline step, of the e4m3 step and of the shared-prompt
decode); "warm" rows the rest, including each leg's untimed settle phase.  The headline
roofline's kernel time is the cold row of decode_seq_kernel<128,0,2,0,4,1,16,1>.

| kernel | workgroups | caches | calls | average us | min us | max us | share of GPU time |
|---|---|---|---|---|---|---|---|
"""
    for r in rows:
        body += (f"| `{_short_kernel(r['name'])}` | {r['wgs']} | {'cold' if r['cold'] else 'warm'} | "
                 f"{r['calls']} | {r['avg'] / 1e3:.1f} | "
                 f"{r['min'] / 1e3:.1f} | {r['max'] / 1e3:.1f} | {100 * r['total'] / total:.1f}% |\n")
    body += f"""
bench.py's HIP-event figures in the same profiled session:
- fp16 decode step (roofline kernel): {roof['ms_mean'] * 1e3:.1f} us per launch (mean of the cold steps' event pairs)
- fp16 decode step, warm: {b.get('warm_step', {}).get('ms_per_step', 0) * 1e3:.1f} us per launch (one event pair over back-to-back steps)
- fp16 pa_decode after pa_write_kv: mean {b.get('two_call_step', {}).get('pa_decode_ms', 0) * 1e3:.1f} us
- e4m3 decode step (pa_decode_append): mean {f8.get('kernel_ms', 0) * 1e3:.1f} us cold, {f8.get('warm_kernel_ms', 0) * 1e3:.1f} us warm
- shared-prompt decode: {pc.get('pa_decode_ms_without_hint', 0) * 1e3:.1f} us streaming every block, {pc.get('pa_decode_ms', 0) * 1e3:.1f} us with the shared-prefix hint (warm), {pc.get('pa_decode_ms_cold', 0) * 1e3:.1f} us cold
- chunked prefill: mean {pf.get('ms', 0) * 1e3:.1f} us

The write_kv and copyBuffer rows are dominated by the set-up writes of whole contexts, not by the
64-token step writes.
"""
    with open(out_md, "w") as f:
        f.write(body)
    print(body)


PREFILL_PMC_PASSES = (
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU "
    "SQ_VALU_MFMA_COEXEC_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE",
    "SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU "
    "SQ_ACTIVE_INST_LDS SQ_INSTS_VALU_TRANS_F32 SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE",
)


def summarize_prefill_pmc(dir1, dir2, out_md):
    """Counter summary of the 8 x 512-row chunked prefill over an fp16 cache
    (prefill_pp_kernel<128, 16>) from two rocprofv3 --pmc runs of
    --prefill-only."""
    def latest(d):
        hits = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not hits:
            raise SystemExit(f"no counter_collection.csv under {d}")
        return max(hits, key=os.path.getmtime)

    vals = {}
    for d, names in zip((dir1, dir2), PREFILL_PMC_PASSES):
        path = latest(d)
        for c in names.split():
            table = _read_counter_csv(path, c)
            keys = [k for k in table if "prefill_pp_kernel" in k and "ILi128ELi16E" in k]
            if not keys:
                raise SystemExit(f"no fp16 prefill dispatch with {c} in {path}")
            v = table[keys[0]]
            vals[c] = sum(v) / len(v)
    simds, xcds = 1024, 8
    grbm = vals["GRBM_GUI_ACTIVE"] / xcds          # the counter sums the 8 XCDs
    mfma_busy = vals["SQ_VALU_MFMA_BUSY_CYCLES"]
    wave = vals["SQ_WAVE_CYCLES"]
    rows = [
        ("kernel duration (GRBM_GUI_ACTIVE per XCD)", f"{grbm:,.0f} cycles"),
        ("MFMA busy / (duration x 1024 SIMDs)", f"{mfma_busy / (grbm * simds):.3f}"),
        ("MFMA instructions per dispatch", f"{vals['SQ_INSTS_MFMA']:,.0f}"),
        ("SQ_INSTS_VALU / SQ_INSTS_MFMA", f"{vals['SQ_INSTS_VALU'] / vals['SQ_INSTS_MFMA']:.2f}"),
        ("of which transcendental (exp2) per MFMA", f"{vals['SQ_INSTS_VALU_TRANS_F32'] / vals['SQ_INSTS_MFMA']:.2f}"),
        ("SALU / LDS instructions per MFMA",
         f"{vals['SQ_INSTS_SALU'] / vals['SQ_INSTS_MFMA']:.2f} / {vals['SQ_INSTS_LDS'] / vals['SQ_INSTS_MFMA']:.2f}"),
        ("VALU and MFMA co-issue cycles / MFMA busy cycles",
         f"{vals['SQ_VALU_MFMA_COEXEC_CYCLES'] / mfma_busy:.3f}"),
        ("wave time issuing any instruction (ACTIVE_INST_ANY / WAVE_CYCLES)", f"{vals['SQ_ACTIVE_INST_ANY'] / wave:.3f}"),
        ("wave time waiting on s_waitcnt (WAIT_ANY / WAVE_CYCLES)", f"{vals['SQ_WAIT_ANY'] / wave:.3f}"),
        ("wave time waiting to issue (WAIT_INST_ANY / WAVE_CYCLES)", f"{vals['SQ_WAIT_INST_ANY'] / wave:.3f}"),
        ("LDS bank conflicts per LDS instruction", f"{vals['SQ_LDS_BANK_CONFLICT'] / vals['SQ_INSTS_LDS']:.3f}"),
    ]
    body = f"""# Chunked-prefill counters: prefill_pp_kernel<128, 16> (fp16 cache), 8 x 512-row chunks over 0..4096 cached tokens

Commands (repository root, on the MI355X; one pass per counter set):

    rocprofv3 --pmc {PREFILL_PMC_PASSES[0]} --output-format csv -d gpurun_out/pf_pmc1 -- python bench.py --prefill-only
    rocprofv3 --pmc {PREFILL_PMC_PASSES[1]} --output-format csv -d gpurun_out/pf_pmc2 -- python bench.py --prefill-only
    python bench.py --summarize-prefill-pmc gpurun_out/pf_pmc1 gpurun_out/pf_pmc2 {out_md}

Averages over every dispatch of the kernel in the run (settle, warm-up and timed calls).  The
SQ counters sum over all SIMDs; GRBM_GUI_ACTIVE sums the 8 XCDs.

- kernel source hash: `{prefill_source_hash()}`

| quantity | value |
|---|---|
"""
    for k, v in rows:
        body += f"| {k} | {v} |\n"
    body += "\nRaw per-dispatch averages:\n\n"
    for k in sorted(vals):
        body += f"- {k}: {vals[k]:,.0f}\n"
    with open(out_md, "w") as f:
        f.write(body)
    print(body)


DECODE_PMC_PASSES = (
    "SQ_WAVES SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU "
    "SQ_ACTIVE_INST_VMEM SQ_BUSY_CYCLES GRBM_GUI_ACTIVE",
    "SQ_INSTS_VALU SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR SQ_INSTS_SALU SQ_INSTS_SMEM SQ_INSTS_LDS "
    "SQ_INST_LEVEL_VMEM GRBM_GUI_ACTIVE",
)


def summarize_decode_pmc(dir1, dir2, out_md):
    """Counter summary of the decode-step kernel (pa_decode_append on the
    13B-shaped batch) from two rocprofv3 --pmc runs of --pmc-run."""
    def latest(d):
        hits = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not hits:
            raise SystemExit(f"no counter_collection.csv under {d}")
        return max(hits, key=os.path.getmtime)

    vals = {}
    for d, names in zip((dir1, dir2), DECODE_PMC_PASSES):
        path = latest(d)
        for c in names.split():
            table = _read_counter_csv(path, c)
            keys = [k for k in table if "decode_seq_kernel" in k and "ILi128ELb0ELi2ELb0ELi4ELi1ELi16ELb1E" in k]
            if not keys:
                raise SystemExit(f"no decode-step dispatch with {c} in {path}")
            v = table[keys[0]]
            vals[c] = sum(v) / len(v)
    xcds = 8
    grbm = vals["GRBM_GUI_ACTIVE"] / xcds          # the counter sums the 8 XCDs
    wave = vals["SQ_WAVE_CYCLES"]
    alg = 1354661376                               # algorithmic bytes of one step launch
    rows = [
        ("kernel duration (GRBM_GUI_ACTIVE per XCD)", f"{grbm:,.0f} cycles"),
        ("waves per dispatch", f"{vals['SQ_WAVES']:,.0f}"),
        ("wave time issuing any instruction (ACTIVE_INST_ANY / WAVE_CYCLES)", f"{vals['SQ_ACTIVE_INST_ANY'] / wave:.3f}"),
        ("wave time issuing VALU (ACTIVE_INST_VALU / WAVE_CYCLES)", f"{vals['SQ_ACTIVE_INST_VALU'] / wave:.3f}"),
        ("wave time waiting on s_waitcnt (WAIT_ANY / WAVE_CYCLES)", f"{vals['SQ_WAIT_ANY'] / wave:.3f}"),
        ("wave time waiting to issue (WAIT_INST_ANY / WAVE_CYCLES)", f"{vals['SQ_WAIT_INST_ANY'] / wave:.3f}"),
        ("VMEM read instructions per dispatch", f"{vals['SQ_INSTS_VMEM_RD']:,.0f}"),
        ("algorithmic bytes per VMEM read instruction", f"{alg / vals['SQ_INSTS_VMEM_RD']:,.0f}"),
        ("VALU / SALU / SMEM / LDS instructions per VMEM read",
         f"{vals['SQ_INSTS_VALU'] / vals['SQ_INSTS_VMEM_RD']:.1f} / {vals['SQ_INSTS_SALU'] / vals['SQ_INSTS_VMEM_RD']:.1f}"
         f" / {vals['SQ_INSTS_SMEM'] / vals['SQ_INSTS_VMEM_RD']:.2f} / {vals['SQ_INSTS_LDS'] / vals['SQ_INSTS_VMEM_RD']:.3f}"),
    ]
    body = f"""# Decode-step counters: pa_decode_append, decode_seq_kernel<128,0,2,0,4,1,16,1>, llama13b_decode (64 seqs, L ~ U[1,2048], 40 x 128, fp16)

Commands (repository root, on the MI355X; one pass per counter set):

    rocprofv3 --pmc {DECODE_PMC_PASSES[0]} --output-format csv -d gpurun_out/dec_pmc1 -- python bench.py --pmc-run
    rocprofv3 --pmc {DECODE_PMC_PASSES[1]} --output-format csv -d gpurun_out/dec_pmc2 -- python bench.py --pmc-run
    python bench.py --summarize-decode-pmc gpurun_out/dec_pmc1 gpurun_out/dec_pmc2 {out_md}

Averages over the {PMC_DECODE_STEPS} step launches of the run.  The SQ counters sum over all
CUs; GRBM_GUI_ACTIVE sums the 8 XCDs.  The three wave-time shares (issuing, waiting on
s_waitcnt, waiting to issue) are ratios of counters in the same units and sum to one.  Waves
of this memory-bound kernel issue an instruction in under a tenth of their time; the rest they
wait, on their own loads (s_waitcnt) or for the memory pipeline and the other waves of their
SIMD to let the next load issue.  SQ_ACTIVE_INST_VMEM reads 0 on this part, and
SQ_INST_LEVEL_VMEM gives no usable latency here; both stay in the raw list only.

- kernel source hash: `{kernel_source_hash()}`

| quantity | value |
|---|---|
"""
    for k, v in rows:
        body += f"| {k} | {v} |\n"
    body += "\nRaw per-dispatch averages:\n\n"
    for k in sorted(vals):
        body += f"- {k}: {vals[k]:,.0f}\n"
    with open(out_md, "w") as f:
        f.write(body)
    print(body)


def summarize_pmc(fetch_dir, write_dir, name="step_fp16"):
    """Write profiles/<PMC_WORKLOADS[name] file> from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE) of --pmc-run NAME."""
    import numpy as np

    import workloads

    desc, fname = PMC_WORKLOADS[name]

    def find(d):
        hits = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not hits:
            raise SystemExit(f"no counter_collection.csv under {d}")
        return max(hits, key=os.path.getmtime)  # the latest run

    fetch = _read_counter_csv(find(fetch_dir), "FETCH_SIZE")
    write = _read_counter_csv(find(write_dir), "WRITE_SIZE")

    def pick(table, key):
        names = [n for n in table if key in n]
        if not names:
            raise SystemExit(f"no kernel matching {key!r} in {sorted(table)}")
        return names[0], table[names[0]]

    copy_name, copy_f = pick(fetch, "neg")
    _, copy_w = pick(write, "neg")
    pick(fetch, "decode_")
    known_kib = PMC_COPY_BYTES / 1024.0
    f_scale = known_kib / copy_f[0]
    w_scale = known_kib / copy_w[0]
    dec_kernels = [n for n in fetch if "decode_" in n]
    per_call_f = sum(sum(fetch[n]) for n in dec_kernels) / PMC_DECODE_STEPS
    per_call_w = sum(sum(write.get(n, [0.0])) for n in dec_kernels) / PMC_DECODE_STEPS
    rd = per_call_f * f_scale * 1024.0
    wr = per_call_w * w_scale * 1024.0
    refs = "\n".join(f"- {label}: `{b:.6e}` (read / this: {rd / b:.3f})"
                      for label, b in pmc_reference_bytes(name, np, workloads))
    text = f"""# Decode HBM traffic: {desc}

Commands (from the repository root, on the MI355X):

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch_{name} -- python bench.py --pmc-run {name}
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write_{name} -- python bench.py --pmc-run {name}
    python bench.py --summarize-pmc gpurun_out/pmc_fetch_{name} gpurun_out/pmc_write_{name} {name}

FETCH_SIZE and WRITE_SIZE count the L2's traffic to the memory fabric (the
last-level cache and HBM behind it), in KiB per dispatch.  Calibration:
`{copy_name[:60]}` copies {PMC_COPY_BYTES} B; FETCH_SIZE read {copy_f[0]:.1f} KiB
(scale {f_scale:.4f}), WRITE_SIZE {copy_w[0]:.1f} KiB (scale {w_scale:.4f}).
The {PMC_DECODE_STEPS} decode calls run back to back after the set-up writes.

Decode kernels counted: {", ".join(sorted(set(n[:70] for n in dec_kernels)))}
FETCH_SIZE per call (raw): {per_call_f:.1f} KiB; WRITE_SIZE per call (raw): {per_call_w:.1f} KiB

- kernel source hash: `{kernel_source_hash()}`
- HBM bytes read per decode-step launch: `{rd:.6e}`
- HBM bytes written per decode-step launch: `{wr:.6e}`

Compared with:

{refs}
"""
    out = os.path.join(ROOT, "profiles", fname)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with open(out, "w") as f:
        f.write(text)
    print(text)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="decode step only (for profiling)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--pmc-run", nargs="?", const="step_fp16", choices=sorted(PMC_WORKLOADS),
                    help="copy + one decode workload only, for counter runs")
    ap.add_argument("--prefill-only", action="store_true", help="the chunked-prefill leg only (for profiling)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="FETCH_DIR WRITE_DIR [WORKLOAD]")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("TRACE_DIR", "BENCH_LOG", "OUT_MD"))
    ap.add_argument("--summarize-prefill-pmc", nargs=3, metavar=("PASS1_DIR", "PASS2_DIR", "OUT_MD"))
    ap.add_argument("--summarize-decode-pmc", nargs=3, metavar=("PASS1_DIR", "PASS2_DIR", "OUT_MD"))
    args = ap.parse_args()
    if args.summarize_pmc:
        if len(args.summarize_pmc) not in (2, 3):
            ap.error("--summarize-pmc FETCH_DIR WRITE_DIR [WORKLOAD]")
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_prefill_pmc:
        summarize_prefill_pmc(*args.summarize_prefill_pmc)
        return
    if args.summarize_decode_pmc:
        summarize_decode_pmc(*args.summarize_decode_pmc)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this library runs on a single MI355X and has no "
              f"multi-GPU path (asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_394_amd as pa
    import workloads

    torch.cuda.set_device(0)
    if args.pmc_run:
        pmc_run(pa, torch, np, workloads, args.pmc_run)
        return
    if args.prefill_only:
        print(json.dumps({"prefill": bench_prefill(pa, torch, np, workloads, 20)}), flush=True)
        return
    log("generating the 13B-shaped decode batch")
    w = workloads.llama13b_decode()
    d = setup_decode(w, False, pa, torch, np)
    log("decode fp16, cold caches (the headline)")
    cold_ms, wall_ms = cold_region(torch, np, lambda: append_call(pa, w, d), args.steps, args.warmup)
    ms_step = float(np.median(cold_ms))
    dec_ms = float(cold_ms.mean())
    kv_bytes, alg_bytes = decode_bytes(w, 2, fused=True)
    log("decode fp16, warm (back to back)")
    _, warm_ms = run_decode(pa, torch, w, d, args.steps, args.warmup)
    log("decode fp16, two calls (pa_write_kv + pa_decode)")
    ms_step2, _ = run_decode(pa, torch, w, d, args.steps, args.warmup, fused=False)
    log("pa_decode alone")
    _, dec_ms2 = time_region(torch, lambda: decode_call(pa, w, d), args.steps, args.warmup)
    _, alg_bytes2 = decode_bytes(w, 2)
    value = kv_bytes / (ms_step * 1e-3) / 1e9
    achieved = alg_bytes / (dec_ms * 1e-3) / 1e9
    traffic = read_traffic()
    srt = np.sort(cold_ms)
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "llama13b_decode: 64 seqs, context U[1,2048], 40 q heads = 40 kv heads, "
                               "head_dim 128, block 16, fp16 KV scattered over a pool of needed+10% blocks",
                   "batch": w.batch, "kv_tokens": int(w.lens.sum()), "num_heads": w.num_heads,
                   "head_dim": w.head_dim, "block_size": 16, "num_blocks": w.num_blocks,
                   "kv_bytes_per_step": kv_bytes},
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(w.batch / (ms_step * 1e-3), 1),
        "roofline": {"kernel": "pa_decode_append (decode_seq_kernel, appending)", "bound": "hbm",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic[0] + traffic[1], 0),
                     "traffic_read": None if traffic is None else round(traffic[0], 0),
                     "traffic_write": None if traffic is None else round(traffic[1], 0),
                     "algorithmic_bytes": alg_bytes, "ms_mean": round(dec_ms, 5),
                     "timing": "mean of the K cold steps' event pairs, one launch per step"},
        "timing": {"flush": "1 GiB fill before every step", "step_ms_median": round(ms_step, 5),
                   "step_ms_p10": round(float(srt[len(srt) // 10]), 5),
                   "step_ms_p90": round(float(srt[(9 * len(srt)) // 10]), 5),
                   "region_wall_ms_per_step": round(wall_ms, 5)},
        "warm_step": {"ms_per_step": round(warm_ms, 5), "kv_gbs": round(kv_bytes / (warm_ms * 1e-3) / 1e9, 2),
                      "kernel_hbm_frac": round(alg_bytes / (warm_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "timing": "one HIP event pair over K back-to-back steps"},
        "two_call_step": {"ms_per_step": round(ms_step2, 5),
                          "kv_gbs": round(kv_bytes / (ms_step2 * 1e-3) / 1e9, 2),
                          "pa_decode_ms": round(dec_ms2, 5),
                          "pa_decode_gbs": round(alg_bytes2 / (dec_ms2 * 1e-3) / 1e9, 2),
                          "pa_decode_hbm_frac": round(alg_bytes2 / (dec_ms2 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "host": host_timings(w, pa, np),
        "capacity": capacity(pa, np),
    }
    del d
    torch.cuda.empty_cache()
    if not args.no_extras:
        log("copy and read ceilings")
        res["ceiling"] = copy_ceiling(torch)
        res["read_ceiling"] = read_ceiling(torch)
        ach = achievable_read(pa, torch, np, cold=True)
        # cold against cold, warm against warm
        ach["step_frac"] = round(value / ach["gbs_read_cold"], 4)
        ach["roofline_kernel_frac"] = round(achieved / ach["gbs_read_cold"], 4)
        ach["warm_step_frac"] = round(res["warm_step"]["kv_gbs"] / ach["gbs_read"], 4)
        res["achievable_read"] = ach
        # the same pattern at the e4m3 step's size (0.68 GB), for the fp8 leg below
        res["achievable_read_fp8_size"] = achievable_read(pa, torch, np, n_tiles=165800, cold=True)
        log("decode e4m3")
        d8 = setup_decode(w, True, pa, torch, np)
        cold8, _ = cold_region(torch, np, lambda: append_call(pa, w, d8), args.steps, args.warmup)
        ms8c = float(np.median(cold8))
        ms8, dec8 = run_decode(pa, torch, w, d8, args.steps, args.warmup)
        kv8, alg8 = decode_bytes(w, 1, fused=True)
        res["fp8_decode"] = {"kv_gbs": round(kv8 / (ms8c * 1e-3) / 1e9, 2), "ms_per_step": round(ms8c, 5),
                             "kernel_ms": round(float(cold8.mean()), 5),
                             "kernel_hbm_frac": round(alg8 / (float(cold8.mean()) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                             "timing": "cold steps as the headline: median per step, mean for the kernel; "
                                       "warm_*: one event pair over back-to-back steps",
                             "warm_ms_per_step": round(ms8, 5), "warm_kernel_ms": round(dec8, 5),
                             "warm_kernel_gbs": round(alg8 / (dec8 * 1e-3) / 1e9, 2),
                             "warm_hbm_frac": round(alg8 / (dec8 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if "achievable_read_fp8_size" in res:   # cold against cold, warm against warm
            a8 = res["achievable_read_fp8_size"]
            res["fp8_decode"]["warm_achievable_frac"] = round(res["fp8_decode"]["warm_kernel_gbs"] / a8["gbs_read"], 4)
            res["fp8_decode"]["achievable_frac"] = round(
                alg8 / (float(cold8.mean()) * 1e-3) / 1e9 / a8["gbs_read_cold"], 4)
        del d8
        torch.cuda.empty_cache()
        log("prefix sharing decode")
        res["prefix_cow"] = bench_prefix(pa, torch, np, workloads, args.steps)
        log("shared-prompt decode, e4m3")
        res["prefix_cow_fp8"] = bench_prefix(pa, torch, np, workloads, args.steps, fp8=True)
        torch.cuda.empty_cache()
        log("prefix cache (host)")
        res["prefix_cache"] = bench_prefix_cache(pa, np, workloads)
        log("mixed prefill + decode step")
        res["mixed_step"] = bench_mixed(pa, torch, np, workloads, 20)
        res["mixed_step_fp8"] = bench_mixed(pa, torch, np, workloads, 20, fp8=True)
        torch.cuda.empty_cache()
        log("preemption: swap vs recompute")
        res["preemption"] = bench_preemption(pa, torch, np, workloads)
        torch.cuda.empty_cache()
        log("chunked prefill")
        res["prefill"] = bench_prefill(pa, torch, np, workloads, 20)
        torch.cuda.empty_cache()
        log("achievable matrix-core rate (probe)")
        res["achievable_mfma"] = achievable_mfma(pa, torch)
        res["prefill"]["achievable_frac"] = round(res["prefill"]["tflops"] / res["achievable_mfma"]["tflops"], 4)
        log("chunked prefill, e4m3 cache")
        res["prefill_fp8"] = bench_prefill(pa, torch, np, workloads, 20, fp8=True)
        torch.cuda.empty_cache()
        log("block sizes 8 / 32 / 64")
        res["block_sizes"] = bench_block_sizes(pa, torch, np, workloads, w, args.steps, args.warmup,
                                               (dec_ms2, res["prefill"]["ms"]))
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(w, np, args.cpu_seconds)
        if not args.no_extras:
            log("cpu baseline (oracle, process pool)")
            res["cpu_baseline_pool"] = cpu_baseline_pool(w, np)
        for key in ("cpu_baseline", "cpu_baseline_pool"):
            if key in res:
                res[key]["host_cores"] = len(os.sched_getaffinity(0))
                res[key]["gpu_over_oracle"] = round(value / res[key]["value"], 1)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
