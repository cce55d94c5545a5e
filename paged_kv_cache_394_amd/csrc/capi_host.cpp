// C ABI: host-side entry points (block manager).  Declared in include/pa.h.
#include <string>

#include "pa.h"
#include "pool.hpp"
#include "status.hpp"

struct pa_pool {
  pa::BlockPool* impl;
};

namespace pa {
namespace {
thread_local std::string g_last_error;
}  // namespace

pa_status fail(pa_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

pa_status ok() {
  g_last_error.clear();
  return PA_OK;
}
}  // namespace pa

using pa::fail;

extern "C" {

const char* pa_last_error(void) { return pa::g_last_error.c_str(); }

const char* pa_version(void) { return "pa 0.1 (gfx950)"; }

pa_status pa_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* init_free_order,
                         pa_pool** out) {
  if (out == nullptr) return fail(PA_ERR_BAD_ARG, "pa_pool_create: out is NULL");
  std::string err;
  pa::BlockPool* impl = nullptr;
  const pa::Status st = pa::BlockPool::create(num_blocks, block_size, init_free_order, &impl, &err);
  if (st != pa::kOk) return fail(st, err);
  pa_pool* p = new (std::nothrow) pa_pool{impl};
  if (p == nullptr) {
    delete impl;
    return fail(PA_ERR_BAD_ARG, "pa_pool_create: out of host memory");
  }
  *out = p;
  return pa::ok();
}

void pa_pool_destroy(pa_pool* pool) {
  if (pool == nullptr) return;
  delete pool->impl;
  delete pool;
}

pa_status pa_seq_create(pa_pool* pool, int32_t* seq_out) {
  if (pool == nullptr || seq_out == nullptr) return fail(PA_ERR_BAD_ARG, "pa_seq_create: NULL argument");
  const pa::Status st = pool->impl->seq_create(seq_out);
  if (st != pa::kOk) return fail(st, "pa_seq_create: sequence id space or host memory exhausted");
  return pa::ok();
}

pa_status pa_alloc_append(pa_pool* pool, int32_t seq, int32_t n_tokens, int32_t* slots_out,
                          int32_t* cow_out) {
  if (pool == nullptr) return fail(PA_ERR_BAD_ARG, "pa_alloc_append: pool is NULL");
  std::string err;
  const pa::Status st = pool->impl->alloc_append(seq, n_tokens, nullptr, slots_out, cow_out, &err);
  if (st != pa::kOk) return fail(st, err);
  return pa::ok();
}

pa_status pa_append_tokens(pa_pool* pool, int32_t seq, const int32_t* tokens, int32_t n_tokens,
                           int32_t* slots_out, int32_t* cow_out) {
  if (pool == nullptr) return fail(PA_ERR_BAD_ARG, "pa_append_tokens: pool is NULL");
  if (n_tokens > 0 && tokens == nullptr) return fail(PA_ERR_BAD_ARG, "pa_append_tokens: tokens is NULL");
  std::string err;
  const pa::Status st = pool->impl->alloc_append(seq, n_tokens, tokens, slots_out, cow_out, &err);
  if (st != pa::kOk) return fail(st, err);
  return pa::ok();
}

pa_status pa_alloc_append_batch(pa_pool* pool, const int32_t* seqs, int32_t n_seqs,
                                const int32_t* n_tokens, const int32_t* token_ids, int32_t* slots_out,
                                int32_t* cow_out) {
  if (pool == nullptr) return fail(PA_ERR_BAD_ARG, "pa_alloc_append_batch: pool is NULL");
  std::string err;
  const pa::Status st =
      pool->impl->alloc_append_batch(seqs, n_seqs, n_tokens, token_ids, slots_out, cow_out, &err);
  if (st != pa::kOk) return fail(st, err);
  return pa::ok();
}

pa_status pa_alloc_prompt(pa_pool* pool, int32_t seq, const int32_t* tokens, int32_t n_tokens,
                          int32_t* slots_out, int32_t* hit_tokens_out) {
  if (pool == nullptr) return fail(PA_ERR_BAD_ARG, "pa_alloc_prompt: pool is NULL");
  std::string err;
  const pa::Status st = pool->impl->alloc_prompt(seq, tokens, n_tokens, slots_out, hit_tokens_out, &err);
  if (st != pa::kOk) return fail(st, err);
  return pa::ok();
}

pa_status pa_swap_space(pa_pool* pool, int32_t num_host_blocks) {
  if (pool == nullptr) return fail(PA_ERR_BAD_ARG, "pa_swap_space: pool is NULL");
  std::string err;
  const pa::Status st = pool->impl->set_swap_space(num_host_blocks, &err);
  if (st != pa::kOk) return fail(st, err);
  return pa::ok();
}

pa_status pa_swap_out(pa_pool* pool, int32_t seq, int32_t* pairs_out, int32_t cap, int32_t* n_out) {
  if (pool == nullptr) return fail(PA_ERR_BAD_ARG, "pa_swap_out: pool is NULL");
  std::string err;
  const pa::Status st = pool->impl->swap_out(seq, pairs_out, cap, n_out, &err);
  if (st != pa::kOk) return fail(st, err);
  return pa::ok();
}

pa_status pa_swap_in(pa_pool* pool, int32_t seq, int32_t* pairs_out, int32_t cap, int32_t* n_out) {
  if (pool == nullptr) return fail(PA_ERR_BAD_ARG, "pa_swap_in: pool is NULL");
  std::string err;
  const pa::Status st = pool->impl->swap_in(seq, pairs_out, cap, n_out, &err);
  if (st != pa::kOk) return fail(st, err);
  return pa::ok();
}

pa_status pa_cache_commit(pa_pool* pool, int32_t seq, int32_t* added_out) {
  if (pool == nullptr) return fail(PA_ERR_BAD_ARG, "pa_cache_commit: pool is NULL");
  std::string err;
  const pa::Status st = pool->impl->cache_commit(seq, added_out, &err);
  if (st != pa::kOk) return fail(st, err);
  return pa::ok();
}

pa_status pa_fork_cow(pa_pool* pool, int32_t parent, int32_t* child_out) {
  if (pool == nullptr) return fail(PA_ERR_BAD_ARG, "pa_fork_cow: pool is NULL");
  const pa::Status st = pool->impl->fork(parent, child_out);
  if (st == pa::kBadSeq) return fail(st, "pa_fork_cow: unknown parent sequence");
  if (st != pa::kOk) return fail(st, "pa_fork_cow: bad argument or out of host memory");
  return pa::ok();
}

pa_status pa_seq_free(pa_pool* pool, int32_t seq) {
  if (pool == nullptr) return fail(PA_ERR_BAD_ARG, "pa_seq_free: pool is NULL");
  const pa::Status st = pool->impl->seq_free(seq);
  if (st != pa::kOk) return fail(st, "pa_seq_free: unknown sequence");
  return pa::ok();
}

pa_status pa_block_tables(const pa_pool* pool, const int32_t* seqs, int32_t n, int32_t max_blocks,
                          int32_t* tables_out, int32_t* lens_out) {
  if (pool == nullptr) return fail(PA_ERR_BAD_ARG, "pa_block_tables: pool is NULL");
  std::string err;
  const pa::Status st = pool->impl->block_tables(seqs, n, max_blocks, tables_out, lens_out, &err);
  if (st != pa::kOk) return fail(st, err);
  return pa::ok();
}

pa_status pa_seq_table(const pa_pool* pool, int32_t seq, int32_t* table_out, int32_t cap,
                       int32_t* n_out, int32_t* len_out) {
  if (pool == nullptr) return fail(PA_ERR_BAD_ARG, "pa_seq_table: pool is NULL");
  const pa::Status st = pool->impl->seq_table(seq, table_out, cap, n_out, len_out);
  if (st == pa::kBadSeq) return fail(st, "pa_seq_table: unknown sequence");
  if (st != pa::kOk) return fail(st, "pa_seq_table: table longer than cap");
  return pa::ok();
}

pa_status pa_shared_prefix(const pa_pool* pool, const int32_t* seqs, int32_t n,
                           int32_t* blocks_out) {
  if (pool == nullptr) return fail(PA_ERR_BAD_ARG, "pa_shared_prefix: pool is NULL");
  std::string err;
  const pa::Status st = pool->impl->shared_prefix(seqs, n, blocks_out, &err);
  if (st != pa::kOk) return fail(st, err);
  return pa::ok();
}

pa_status pa_pool_state(const pa_pool* pool, pa_pool_stats* stats_out, int32_t* free_order_out,
                        int32_t* ref_cnt_out) {
  if (pool == nullptr) return fail(PA_ERR_BAD_ARG, "pa_pool_state: pool is NULL");
  pa::PoolStats st{};
  pool->impl->state(&st, free_order_out, ref_cnt_out);
  if (stats_out) {
    stats_out->num_blocks = st.num_blocks;
    stats_out->free_blocks = st.free_blocks;
    stats_out->used_blocks = st.used_blocks;
    stats_out->shared_blocks = st.shared_blocks;
    stats_out->total_refs = st.total_refs;
    stats_out->cow_copies = st.cow_copies;
    stats_out->live_seqs = st.live_seqs;
    stats_out->tokens = st.tokens;
    stats_out->waste_tokens = st.waste_tokens;
    stats_out->cached_blocks = st.cached_blocks;
    stats_out->prompt_tokens = st.prompt_tokens;
    stats_out->hit_tokens = st.hit_tokens;
    stats_out->evictions = st.evictions;
    stats_out->host_blocks = st.host_blocks;
    stats_out->host_free_blocks = st.host_free_blocks;
    stats_out->swapped_seqs = st.swapped_seqs;
  }
  return pa::ok();
}

}  // extern "C"
