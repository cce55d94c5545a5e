/*
 * pa.h -- C ABI of libpa: paged KV-cache attention for AMD Instinct MI355X (gfx950).
 *
 * The library follows the block-manager model of the pages:
 *   [p1] "vLLM PagedAttention Deep Dive: KV Cache Memory Fragmentation, Chunked
 *        Prefill & Prefix Caching"
 *   [p2] "PagedAttention: KV cache as virtual memory (block manager & fragmentation)"
 *   [p3] "PagedAttention: Why Static Batching Wastes Your KV Cache"
 * A pool of fixed-size physical blocks is shared by all sequences; each sequence
 * maps its logical blocks to physical blocks through a block table; blocks are
 * taken one at a time as a sequence grows, returned when their reference count
 * drops to zero, shared between forked sequences and copied per block on write.
 * Attention reads K/V through the block table from scattered blocks.
 *
 * Conventions
 * -----------
 * Ownership.  A pool (pa_pool) holds host bookkeeping only.  Every device pointer
 *   (caches, q, out, tables, slots, lens, workspace) is allocated and owned by the
 *   caller.  The library never allocates or frees device memory and never
 *   synchronises a stream.  hip_stream is a hipStream_t (NULL = the null stream).
 * Errors.  Every call returns a pa_status; pa_last_error() gives a message for the
 *   calling thread.  Host calls are all-or-nothing: on any non-OK status the pool
 *   is bit-identical to its state before the call.  Device calls check their
 *   arguments on the host and return PA_ERR_HIP if a launch fails; faults during
 *   execution surface at the caller's next synchronisation.
 * Threads.  A pool is used by one thread at a time (no internal locking).
 * Limits.  block_size * num_blocks < 2^31 (slots are int32).  Device byte offsets
 *   are computed in 64 bits.
 * Device input checks.  Kernels never read or write outside the buffers the sizes
 *   describe: slots outside [0, num_blocks*block_size) are skipped, context lengths
 *   are clamped to [0, max_blocks*block_size], block ids outside [0, num_blocks)
 *   are read as block 0.  Results for such inputs are unspecified but safe.
 *
 * Cache layout (the pages leave it open; chosen here).  K and V are two separate
 *   device arrays, each [num_blocks][num_kv_heads][block_size][head_dim]: one
 *   (block, head) is a contiguous block_size*head_dim tile (4 KiB for 16 x 128
 *   fp16, 2 KiB for e4m3).  Token t of a sequence is row t % block_size of physical
 *   block table[t / block_size]; its flat slot is block * block_size + row.
 * Block size ([p1] "Tuning Block Size and GPU Memory Utilization"; [p3] "How do I
 *   configure vLLM to use this well?": smaller blocks waste fewer slots at the tail
 *   of each sequence, larger ones mean shorter tables and longer contiguous reads).
 *   The host pool takes any block_size >= 1; the device kernels are compiled for
 *   block_size 8, 16, 32 and 64, and an e4m3 tile must be at least 1 KiB
 *   (block_size * head_dim >= 1024: block_size 8 with e4m3 needs head_dim 128).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pa_status;
#define PA_OK 0
#define PA_ERR_NO_BLOCKS 1   /* not enough free blocks; nothing was taken        */
#define PA_ERR_BAD_SEQ 2     /* unknown (or already freed) sequence id            */
#define PA_ERR_BAD_ARG 3     /* null pointer, negative size, bad shape or order   */
#define PA_ERR_CAPACITY 4    /* an output buffer is too small for the request     */
#define PA_ERR_HIP 5         /* a HIP launch or copy reported an error            */
#define PA_ERR_UNSUPPORTED 6 /* shape / dtype combination not compiled in         */

#define PA_KV_F16 0          /* IEEE binary16                                     */
#define PA_KV_FP8_E4M3 1     /* OCP 8-bit E4M3 (bias 7, max 448, no inf), scaled */

typedef struct pa_pool pa_pool;

/* Device-side description of one layer's paged K/V cache (caller-owned). */
typedef struct {
  void *k_cache;          /* [num_blocks][num_kv_heads][block_size][head_dim]        */
  void *v_cache;          /* same shape as k_cache                                   */
  int32_t num_blocks;
  int32_t block_size;     /* tokens per block: 8, 16, 32 or 64 for the device calls  */
  int32_t num_kv_heads;   /* >= 1; one block (num_kv_heads*block_size*head_dim) < 2 GiB */
  int32_t head_dim;       /* 64 or 128                                               */
  int32_t dtype;          /* PA_KV_F16 or PA_KV_FP8_E4M3                             */
  float k_scale;          /* e4m3 only: stored code * k_scale = value                */
  float v_scale;          /* e4m3 only                                               */
} pa_kv_cache;

typedef struct {
  int64_t num_blocks;
  int64_t free_blocks;
  int64_t used_blocks;    /* num_blocks - free_blocks                                */
  int64_t shared_blocks;  /* blocks with ref_cnt > 1                                 */
  int64_t total_refs;     /* sum of ref_cnt                                          */
  int64_t cow_copies;     /* copy-on-write copies made since creation                */
  int64_t live_seqs;
  int64_t tokens;         /* sum of live sequence lengths                            */
  int64_t waste_tokens;   /* sum over live sequences of blocks*block_size - length   */
  int64_t cached_blocks;  /* blocks in the prefix cache (in use or waiting in the queue) */
  int64_t prompt_tokens;  /* tokens admitted through pa_alloc_prompt                  */
  int64_t hit_tokens;     /* of those, tokens served from cached blocks (hit rate =
                             hit_tokens / prompt_tokens)                              */
  int64_t evictions;      /* cached blocks handed out again by the free queue         */
  int64_t host_blocks;    /* size of the host swap space (pa_swap_space)              */
  int64_t host_free_blocks;
  int64_t swapped_seqs;   /* live sequences whose blocks are in host memory           */
} pa_pool_stats;

/* ---------------------------------------------------------------- host side -- */

/* Create a pool of num_blocks physical blocks of block_size tokens ([p2] "Direct
 * answer" and "Deep dive": one shared pool, a free queue with O(1) take-from-front
 * and return-to-back).  init_free_order: NULL for 0..N-1, else a host array that is
 * a permutation of 0..N-1 giving the initial queue order (copied).
 * Errors: BAD_ARG for num_blocks < 1, block_size < 1, N*block_size >= 2^31, a
 * non-permutation order or out == NULL. */
pa_status pa_pool_create(int32_t num_blocks, int32_t block_size,
                         const int32_t *init_free_order, pa_pool **out);

/* Release the pool's host memory.  NULL is ignored. */
void pa_pool_destroy(pa_pool *pool);

/* New empty sequence (length 0, empty table): the per-request block list that
 * draws from the shared pool ([p2] "Deep dive", the V1 structures: one block
 * list per request; the lifecycle starts at admission with none).  Ids are 0,
 * 1, 2, ... in creation order and are never reused. */
pa_status pa_seq_create(pa_pool *pool, int32_t *seq_out);

/* Make room for n_tokens new tokens of sequence seq ([p2] "Deep dive", lifecycle:
 * blocks are popped when the prompt is admitted and one more each time the last
 * block fills; [p3] "What does PagedAttention actually do differently?": blocks
 * are taken on demand, one each time a block_size boundary is crossed).
 * If the last block is partly filled and shared (ref_cnt > 1), it is first
 * replaced by a fresh copy ([p3] "How does copy-on-write eliminate duplicate
 * prompt KV cache?"): a block d is popped, table[last] = d, ref_cnt of the old
 * block drops by one, and cow_out = {old, d}; otherwise cow_out = {-1, -1}.  The
 * caller passes the pair to pa_write_kv, which copies the block's K/V on the device.
 * Then ceil((len + n)/bs) - ceil(len/bs) blocks are popped (front of the queue, in
 * logical order) and slots_out[i] = table[(len+i)/bs]*bs + (len+i)%bs.
 * slots_out: host int32[n_tokens] (may be NULL if n_tokens == 0).  cow_out: host
 * int32[2] or NULL (then a copy-on-write is refused with BAD_ARG).
 * Errors: BAD_SEQ, BAD_ARG (n_tokens < 0, null pointer), NO_BLOCKS (fewer free
 * blocks than needed, copy included); nothing changes on error. */
pa_status pa_alloc_append(pa_pool *pool, int32_t seq, int32_t n_tokens,
                          int32_t *slots_out, int32_t *cow_out);

/* One decode step's reservations in one call: pa_alloc_append (or, with
 * token_ids, pa_append_tokens) for seqs[0], seqs[1], ... in that order, with
 * n_tokens[i] tokens for seqs[i] (the pages' per-sequence lifecycle, [p2]
 * "Deep dive", batched so a step of B sequences costs one call).  All or
 * nothing: the status is that of the first call of the sequence that would
 * fail, and then the pool is unchanged.  slots_out: sum(n_tokens) entries in
 * batch order.  cow_out: 2 * n_seqs entries, {src, dst} or {-1, -1} per
 * sequence (a later sequence sharing the same partly filled block with an
 * earlier one may find it no longer shared, exactly as with single calls).
 * token_ids: NULL, or sum(n_tokens) ids back to back.  Each sequence may appear
 * once.  Errors: BAD_ARG (NULL arrays, negative count, a repeated or swapped-out
 * sequence), BAD_SEQ, NO_BLOCKS, CAPACITY. */
pa_status pa_alloc_append_batch(pa_pool *pool, const int32_t *seqs, int32_t n_seqs,
                                const int32_t *n_tokens, const int32_t *token_ids,
                                int32_t *slots_out, int32_t *cow_out);

/* pa_alloc_append that also records the new tokens' ids, so that the blocks
 * they fill can enter the prefix cache (pa_cache_commit).  A sequence's ids are
 * known only while every append supplied them: after a pa_alloc_append its later
 * blocks are never cached.  tokens: host int32[n_tokens].  Errors as
 * pa_alloc_append, and BAD_ARG for tokens == NULL with n_tokens > 0. */
pa_status pa_append_tokens(pa_pool *pool, int32_t seq, const int32_t *tokens, int32_t n_tokens,
                           int32_t *slots_out, int32_t *cow_out);

/* Admit a prompt into an empty sequence, reusing cached blocks ([p2] "Deep dive",
 * prefix-caching bullet: a block is keyed by its token ids and its parent's key,
 * identical prefixes find the existing blocks and only full blocks are cached;
 * [p1] "Automatic Prefix Caching (APC)", "APC Mechanics").
 * The prompt's full blocks are looked up in order and reused up to the first
 * miss, leaving at least the last token to compute (at most (n-1)/block_size
 * blocks).  A reused block's ref_cnt grows by one; one waiting in the free queue
 * is taken out of it.  Then new blocks are popped from the queue front (a popped
 * block that was cached loses its entry: an eviction).
 * tokens: host int32[n_tokens].  slots_out: host int32[n_tokens]; its first
 * n_tokens - *hit_tokens_out entries receive the slots of tokens *hit_tokens_out ..
 * n_tokens-1, the only ones whose K/V the caller must compute and write.
 * A block's key is SHA-256 over its parent block's key and its token ids, so it
 * names the whole prefix that ends with the block; a hit is a key match.
 * Errors: BAD_SEQ; BAD_ARG (sequence not empty, n_tokens < 0, NULL pointers);
 * NO_BLOCKS (reused blocks that wait in the queue count against it). */
pa_status pa_alloc_prompt(pa_pool *pool, int32_t seq, const int32_t *tokens, int32_t n_tokens,
                          int32_t *slots_out, int32_t *hit_tokens_out);

/* Enter the sequence's full blocks whose token ids are known into the prefix
 * cache; call it once their K/V is written (after the prefill of a prompt, or a
 * decode step that filled a block).  A prefix already cached under another block
 * is left as it is (one cached copy per prefix).  A cached block keeps its entry
 * after its sequences finish, while it waits in the free queue.
 * added_out: number of blocks entered (may be NULL).  Errors: BAD_SEQ. */
pa_status pa_cache_commit(pa_pool *pool, int32_t seq, int32_t *added_out);

/* Preemption by swapping ([p3] "What happens when the GPU runs out of KV
 * blocks?": copy a sequence's blocks to CPU RAM over PCIe and back when it is
 * rescheduled; the other strategy, recomputation, is pa_seq_free followed by a
 * new admission and prefill).  The pool keeps a host swap space of
 * num_host_blocks block ids with its own FIFO free queue (ids 0..n-1 at first);
 * the caller owns the host memory those ids index (pa_swap_blocks).
 * pa_swap_space sets its size; allowed only while no sequence is swapped out.
 * Errors: BAD_ARG (negative size, sequences swapped out). */
pa_status pa_swap_space(pa_pool *pool, int32_t num_host_blocks);

/* Swap a sequence out: for each block in logical order take a host block from
 * the front of the host queue, emit the pair {device, host}, and drop the
 * sequence's reference to the device block (which returns to the back of the
 * device free queue at ref_cnt 0, keeping any prefix-cache entry).  The
 * sequence keeps its length and token ids; until pa_swap_in it cannot be
 * appended to, forked, committed or exported (BAD_ARG).  pairs_out: host
 * int32[cap][2]; *n_out: number of pairs (= its blocks).  The caller must issue
 * the device-to-host copies (pa_swap_blocks, direction 0) on its stream before
 * any work that may write the released blocks.
 * Errors: BAD_SEQ; BAD_ARG (already swapped out, NULL); CAPACITY (cap too small);
 * NO_BLOCKS (host queue too short). */
pa_status pa_swap_out(pa_pool *pool, int32_t seq, int32_t *pairs_out, int32_t cap, int32_t *n_out);

/* Swap a sequence back in: for each host block in logical order pop a device
 * block from the free queue front (ref_cnt 1), emit {host, device}, and return
 * the host block to the back of the host queue.  The caller issues the
 * host-to-device copies (pa_swap_blocks, direction 1) before using the sequence.
 * Errors: BAD_SEQ; BAD_ARG (not swapped out, NULL); CAPACITY; NO_BLOCKS. */
pa_status pa_swap_in(pa_pool *pool, int32_t seq, int32_t *pairs_out, int32_t cap, int32_t *n_out);

/* Fork: a new sequence whose table and length equal the parent's; every shared
 * block's ref_cnt grows by one ([p1] "Virtual Memory Paging Analogy" on sharing;
 * [p3] copy-on-write section: one copy of the prompt KV, like fork()).
 * Errors: BAD_SEQ, BAD_ARG (child_out NULL). */
pa_status pa_fork_cow(pa_pool *pool, int32_t parent, int32_t *child_out);

/* Finish a sequence: for each block in logical order ref_cnt drops by one and a
 * block reaching zero is appended to the back of the free queue ([p2] "Deep dive").
 * Errors: BAD_SEQ. */
pa_status pa_seq_free(pa_pool *pool, int32_t seq);

/* Export block tables for n sequences as a host int32[n][max_blocks] array padded
 * with -1, and lens_out int32[n] (may be NULL).  Row i is sequence seqs[i]'s block
 * table: entry j is the physical block holding its logical block j ([p1] "Virtual
 * Memory Paging Analogy": each sequence keeps an array from logical to physical
 * block indices; [p1] "PagedAttention Mechanism": the kernel looks the blocks up
 * there).  The caller copies them to the device.
 * Errors: BAD_SEQ, BAD_ARG, CAPACITY (a table longer than max_blocks). */
pa_status pa_block_tables(const pa_pool *pool, const int32_t *seqs, int32_t n,
                          int32_t max_blocks, int32_t *tables_out, int32_t *lens_out);

/* Copy the table of one sequence (host int32[cap]); *n_out = its length in blocks.
 * Errors: BAD_SEQ, CAPACITY. */
pa_status pa_seq_table(const pa_pool *pool, int32_t seq, int32_t *table_out, int32_t cap,
                       int32_t *n_out, int32_t *len_out);

/* For each of n sequences, the number of leading table entries whose block is
 * shared (ref_cnt > 1), into host int32[n].  Forked sequences share a prefix of
 * their tables ([p3] copy-on-write section: one stored copy of a common prompt),
 * so these counts mark the blocks every sharer reads; pa_decode can read those
 * through the caches (cached_blocks_dev).  Errors: BAD_SEQ, BAD_ARG. */
pa_status pa_shared_prefix(const pa_pool *pool, const int32_t *seqs, int32_t n,
                           int32_t *blocks_out);

/* Snapshot of the pool ([p2] "Deep dive", the V1 structures: the free queue in
 * eviction order and a ref_cnt per block): counters, and optionally the free
 * queue from front to back (host int32[num_blocks], first free_blocks entries
 * valid) and ref_cnt (host int32[num_blocks]).  stats_out and either array may
 * be NULL.  Errors: BAD_ARG (pool NULL). */
pa_status pa_pool_state(const pa_pool *pool, pa_pool_stats *stats_out,
                        int32_t *free_order_out, int32_t *ref_cnt_out);

/* --------------------------------------------------------------- device side -- */

/* Write new tokens' K/V into their slots (the K/V of each processed chunk is
 * accumulated in paged blocks: [p1] "Mechanics of Chunked Prefill").
 * First, for each of the n_cow pairs {src, dst} (host int32[n_cow][2], as returned
 * by pa_alloc_append) the whole block src is copied to dst in both caches.  Then
 * token i (0 <= i < T) is scattered: cache[slot/bs][h][slot%bs][:] = new[i][h][:]
 * for every KV head h.  k_new, v_new: device fp16 [T][num_kv_heads][head_dim],
 * contiguous.  slots_dev: device int32[T]; negative slots are padding and skipped.
 * For e4m3 caches each value is stored as encode(clamp(x / scale, +-448)) with one
 * correctly rounded fp32 division and round-to-nearest-even.
 * All work is enqueued on hip_stream in that order.
 * Errors: BAD_ARG (null pointers with T > 0, bad pairs, bad descriptor),
 * UNSUPPORTED (dtype / block_size), HIP. */
pa_status pa_write_kv(const pa_kv_cache *cache, const void *k_new, const void *v_new,
                      const int32_t *slots_dev, int32_t T,
                      const int32_t *cow_pairs_host, int32_t n_cow, void *hip_stream);

/* Bytes of device workspace pa_decode needs for this shape (split-K partials). */
size_t pa_decode_workspace_bytes(int32_t B, int32_t num_heads, int32_t head_dim,
                                 int32_t max_context_len);

/* One continuous-batching step in one launch ([p1] "Chunked Prefill" and
 * "Mechanics of Chunked Prefill": prefill chunks of admitted requests are
 * scheduled in the same step as the decode of running ones; [p3] continuous
 * batching section).  Computes exactly what pa_prefill_chunk(prefill) and
 * pa_decode(decode) compute, over one cache (one layer), in one kernel whose
 * grid holds the prefill workgroups first and the decode workgroups after
 * them, so decode work fills the CUs the prefill's tail leaves idle.
 * prefill / decode: either may be NULL or empty (batch 0); fields as the
 * arguments of the two calls.  fp16 or e4m3 caches.
 * The one-launch form covers decode contexts up to 4 waves x 256 blocks of
 * units (8192 / 16384 / 32704 / 65344 tokens at block_size 8 / 16 / 32 / 64);
 * beyond that,
 * or with one part empty, the parts are launched one after the other on the
 * same stream (same results), which is when decode->workspace may be needed
 * (size as pa_decode_workspace_bytes).  Errors: as the two calls. */
typedef struct {
  const void *q;           /* device fp16 [total_q][num_heads][head_dim]            */
  int32_t total_q;
  const int32_t *cu_q;     /* device int32[batch + 1]                               */
  const int32_t *prior;    /* device int32[batch]                                   */
  const int32_t *tables;   /* device int32[batch][max_blocks]                       */
  int32_t batch, max_blocks, max_chunk;
  float *out;              /* device fp32 [total_q][num_heads][head_dim]            */
} pa_prefill_batch;

typedef struct {
  const void *q;           /* device fp16 [batch][num_heads][head_dim]              */
  const int32_t *tables;   /* device int32[batch][max_blocks]                       */
  const int32_t *lens;     /* device int32[batch]                                   */
  const int32_t *cached_blocks; /* NULL or device int32[batch] (pa_decode's hint)   */
  int32_t batch, max_blocks, max_context_len;
  float *out;              /* device fp32 [batch][num_heads][head_dim]              */
  void *workspace;         /* device, only for the two-launch fallback              */
  size_t workspace_bytes;
} pa_decode_batch;

pa_status pa_mixed_step(const pa_kv_cache *cache, int32_t num_heads, float scale,
                        const pa_prefill_batch *prefill, const pa_decode_batch *decode,
                        void *hip_stream);

/* Copy whole blocks between the device cache and caller-owned host memory, for
 * pa_swap_out / pa_swap_in.  host_k / host_v: host buffers of num_host_blocks
 * blocks each, in the cache's layout [block][num_kv_heads][block_size][head_dim]
 * (pinned memory from hipHostMalloc for asynchronous copies).  pairs_host:
 * host int32[n_pairs][2] as emitted: {device, host} for direction 0
 * (device -> host), {host, device} for direction 1 (host -> device).  Runs of
 * consecutive ids are merged into one copy per cache; copies are enqueued on
 * hip_stream with hipMemcpyAsync.  Errors: BAD_ARG (ids out of range, NULL,
 * bad direction), HIP. */
pa_status pa_swap_blocks(const pa_kv_cache *cache, void *host_k, void *host_v,
                         int32_t num_host_blocks, const int32_t *pairs_host, int32_t n_pairs,
                         int32_t direction, void *hip_stream);

/* Decode attention: one query per sequence over its paged context ([p1]
 * "PagedAttention Mechanism": look the physical blocks up in the block table,
 * gather K/V, run standard attention; [p2]/[p3]: the result equals attention over
 * the same tokens stored contiguously).
 * out[b][h] = softmax(scale * K_b q[b][h]) V_b over tokens 0..lens[b]-1 of KV head
 * h / (num_heads / num_kv_heads).  Sequences with lens[b] == 0 get zeros.
 * q: device fp16 [B][num_heads][head_dim].  tables_dev: device int32[B][max_blocks]
 * (as from pa_block_tables).  lens_dev: device int32[B].  cached_blocks_dev: NULL,
 * or device int32[B] (as from pa_shared_prefix): a read-pattern hint only, the
 * result does not depend on it.  K/V are streamed with non-temporal loads, since
 * each byte is read once per call, except the first cached_blocks[b] blocks of
 * sequence b, which other sequences of the batch also read and which are read
 * through the caches.  max_context_len: an upper bound on every lens[b] (sizes
 * the launch).  out_dev: device fp32 [B][num_heads][head_dim].  workspace: at
 * least pa_decode_workspace_bytes(...) (used only by batches too narrow to fill
 * the GPU with one workgroup per (sequence, head)).
 * Errors: BAD_ARG (shape, null pointers, num_heads % num_kv_heads, workspace too
 * small), UNSUPPORTED (block_size not 8/16/32/64, head_dim not 64/128, an e4m3 tile
 * under 1 KiB), HIP. */
pa_status pa_decode(const pa_kv_cache *cache, const void *q, int32_t num_heads,
                    const int32_t *tables_dev, const int32_t *lens_dev,
                    const int32_t *cached_blocks_dev, int32_t B, int32_t max_blocks,
                    int32_t max_context_len, float scale, float *out_dev, void *workspace_dev,
                    size_t workspace_bytes, void *hip_stream);

/* Bytes of the static per-GPU scratch that pa_decode_noalloc uses in place of
 * a workspace (16 MiB). */
#define PA_DECODE_SCRATCH_BYTES (16u << 20)

/* pa_decode for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels and the same result bits, with the split path's partials in a static
 * array of PA_DECODE_SCRATCH_BYTES that the library holds on each GPU until the
 * process ends, instead of a caller workspace.  It calls no allocating routine.
 * The caller still passes inputs and outputs, as for pa_decode.
 * Every call on one GPU shares that GPU's array, so calls that overlap on one GPU
 * (other streams, other threads) race; serialise them.  The array's earlier
 * contents do not matter (each call writes every partial it reads).
 * Errors: as pa_decode (no workspace errors), plus CAPACITY when
 * pa_decode_workspace_bytes(B, num_heads, head_dim, max_context_len) exceeds
 * PA_DECODE_SCRATCH_BYTES (nothing is launched; use pa_decode with a workspace),
 * and HIP if the array's device address cannot be looked up. */
pa_status pa_decode_noalloc(const pa_kv_cache *cache, const void *q, int32_t num_heads,
                            const int32_t *tables_dev, const int32_t *lens_dev,
                            const int32_t *cached_blocks_dev, int32_t B, int32_t max_blocks,
                            int32_t max_context_len, float scale, float *out_dev,
                            void *hip_stream);

/* One decode step in one launch: append each sequence's new token to the
 * cache and attend over the context that ends with it ([p1] "PagedAttention
 * Mechanism" and [p2] "Deep dive": each generated token's K/V goes into the
 * sequence's last block, then attention reads the blocks through the table).
 * Same result, bit for bit, as pa_write_kv of the new tokens followed by
 * pa_decode, with one launch instead of two: the kernel writes the new rows
 * and takes them from registers for the attention.
 * The new token of sequence b is its token lens[b] - 1 (lens clamped as in
 * pa_decode); the caller has already reserved its slot (pa_alloc_append with
 * n_tokens = 1, then pa_block_tables), so its row goes to physical block
 * tables[b][(lens[b]-1) / block_size], row (lens[b]-1) % block_size.  A sequence
 * with lens[b] == 0 appends nothing.  k_new, v_new: device fp16
 * [B][num_kv_heads][head_dim] (e4m3 caches store them with the cache's scales,
 * encoded as by pa_write_kv).  cow_pairs_host / n_cow: the copy-on-write pairs
 * of the reservation, copied on the stream before the launch (the last block
 * must not be shared when it is written).  Other arguments as for pa_decode.
 * Errors: as pa_decode, plus BAD_ARG for NULL or unaligned k_new / v_new and
 * for bad cow pairs. */
pa_status pa_decode_append(const pa_kv_cache *cache, const void *q, int32_t num_heads,
                           const void *k_new, const void *v_new, const int32_t *tables_dev,
                           const int32_t *lens_dev, const int32_t *cached_blocks_dev, int32_t B,
                           int32_t max_blocks, int32_t max_context_len, float scale,
                           float *out_dev, void *workspace_dev, size_t workspace_bytes,
                           const int32_t *cow_pairs_host, int32_t n_cow, void *hip_stream);

/* Chunked-prefill attention over the paged cache ([p1] "Chunked Prefill" and
 * "Mechanics of Chunked Prefill"): the chunk's K/V must already be written (by
 * pa_write_kv).  Sequence b owns query rows cu_q[b] .. cu_q[b+1]-1; row i of it sits
 * at absolute position prior[b] + i and attends to tokens 0 .. prior[b] + i (causal
 * inside the chunk, everything before it).
 * q: device fp16 [total_q_rows][num_heads][head_dim] (total_q_rows = cu_q[B]; rows at
 * or beyond it are never read or written).  cu_q_dev: device int32[B+1],
 * non-decreasing, cu_q[0] = 0.  prior_dev: device int32[B].  tables_dev: device
 * int32[B][max_blocks].  max_chunk: upper bound on cu_q[b+1] - cu_q[b].  out_dev:
 * device fp32 [total_q_rows][num_heads][head_dim].  An e4m3 cache is widened to
 * fp16 on the way to the matrix cores (exact) and its scales are applied to the
 * scores (k_scale) and the output (v_scale).
 * Errors: BAD_ARG, UNSUPPORTED (block_size not 8/16/32/64, head_dim not 64/128, an
 * e4m3 tile under 1 KiB), HIP. */
pa_status pa_prefill_chunk(const pa_kv_cache *cache, const void *q, int32_t num_heads,
                           int32_t total_q_rows, const int32_t *cu_q_dev, const int32_t *prior_dev,
                           const int32_t *tables_dev, int32_t B, int32_t max_blocks,
                           int32_t max_chunk, float scale, float *out_dev, void *hip_stream);

/* Measurement support, not part of the method: a read-only kernel with the
 * decode's access pattern, for the achievable read bandwidth of that pattern.
 * Wave w reads the 4 KiB tiles tile_ids[w * tiles_per_wave .. + tiles_per_wave)
 * of base (tile i = bytes 4096 i .. 4096 i + 4095), 64 lanes x 16 bytes x 4 loads
 * per tile, eight tiles in flight, non-temporal loads; ids are clamped into
 * 0 .. base_bytes / 4096 - 1.  Nothing is written except, with negligible
 * probability, 1 KiB of sink (a store that keeps the loads alive).
 * base_dev: device, 16-byte aligned, base_bytes >= 4096.  tile_ids_dev: device
 * int32[n_tiles].  tiles_per_wave: a positive multiple of 8 dividing n_tiles.
 * sink_dev: device, 16-byte aligned, 1024 bytes.  Enqueued on hip_stream.
 * Errors: BAD_ARG, HIP. */
pa_status pa_probe_tile_gather(const void *base_dev, int64_t base_bytes, const int32_t *tile_ids_dev,
                               int32_t n_tiles, int32_t tiles_per_wave, void *sink_dev,
                               void *hip_stream);

/* Measurement support, not part of the method: a kernel that only runs the
 * matrix cores with the chunked prefill's instruction (fp16 16x16x32 MFMA), for
 * the fp16 matrix throughput the device sustains.  n_workgroups workgroups of 4
 * waves; each wave issues iters * 8 MFMAs (8 independent accumulations) on
 * random-bit operands held in registers, like real data:
 * 16384 * 8 * iters * 4 * n_workgroups FLOP in all.
 * iters: a multiple of 4.  Nothing is written (sink_dev: device, 64 floats,
 * kept for a store the compiler cannot remove and no run takes).  Enqueued on
 * hip_stream.  Errors: BAD_ARG (NULL sink, negative sizes, iters not a
 * multiple of 4), HIP. */
pa_status pa_probe_mfma(int32_t n_workgroups, int32_t iters, float *sink_dev, void *hip_stream);

/* Message describing the last non-OK status on the calling thread ("" if none). */
const char *pa_last_error(void);

/* Library version string. */
const char *pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
