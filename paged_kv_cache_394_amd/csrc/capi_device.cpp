// C ABI: device-side entry points.  Each call checks its arguments on the host,
// then enqueues the kernels on the caller's stream.  Declared in include/pa.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <string>

#include "launch.hpp"
#include "pa.h"
#include "status.hpp"

using pa::fail;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validates a cache descriptor; fills *d.  Returns PA_OK or an error status.
pa_status check_cache(const pa_kv_cache* c, const char* fn, pa::KvDesc* d) {
  const std::string f(fn);
  if (c == nullptr) return fail(PA_ERR_BAD_ARG, f + ": cache is NULL");
  if (c->k_cache == nullptr || c->v_cache == nullptr)
    return fail(PA_ERR_BAD_ARG, f + ": k_cache / v_cache is NULL");
  if (!aligned16(c->k_cache) || !aligned16(c->v_cache))
    return fail(PA_ERR_BAD_ARG, f + ": caches must be 16-byte aligned");
  if (c->num_blocks < 1 || c->num_kv_heads < 1)
    return fail(PA_ERR_BAD_ARG, f + ": num_blocks and num_kv_heads must be >= 1");
  if (c->block_size != 8 && c->block_size != 16 && c->block_size != 32 && c->block_size != 64)
    return fail(PA_ERR_UNSUPPORTED, f + ": kernels are built for block_size 8, 16, 32 and 64");
  if (static_cast<int64_t>(c->num_blocks) * c->block_size >= (int64_t(1) << 31))
    return fail(PA_ERR_BAD_ARG, f + ": num_blocks * block_size must be < 2^31");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, f + ": head_dim must be 64 or 128");
  // kernels form a block's byte offset from a 32-bit block size
  if (static_cast<int64_t>(c->num_kv_heads) * c->block_size * c->head_dim * 2 >= (int64_t(1) << 31))
    return fail(PA_ERR_BAD_ARG, f + ": one cache block (num_kv_heads * block_size * head_dim "
                                    "elements) must be < 2 GiB");
  if (c->dtype == PA_KV_FP8_E4M3 && c->block_size * c->head_dim < 1024)
    return fail(PA_ERR_UNSUPPORTED, f + ": an e4m3 (block, head) tile must be at least 1 KiB "
                                        "(block_size 8 needs head_dim 128)");
  if (c->dtype != PA_KV_F16 && c->dtype != PA_KV_FP8_E4M3)
    return fail(PA_ERR_BAD_ARG, f + ": unknown cache dtype");
  const bool fp8 = c->dtype == PA_KV_FP8_E4M3;
  if (fp8 && !(std::isfinite(c->k_scale) && c->k_scale > 0.f && std::isfinite(c->v_scale) &&
               c->v_scale > 0.f))
    return fail(PA_ERR_BAD_ARG, f + ": e4m3 scales must be finite and > 0");
  *d = pa::KvDesc{c->k_cache, c->v_cache, c->num_blocks, c->block_size, c->num_kv_heads,
                  c->head_dim, fp8, fp8 ? c->k_scale : 1.f, fp8 ? c->v_scale : 1.f};
  return PA_OK;
}

pa_status hip_status(hipError_t e, const char* fn) {
  if (e != hipSuccess) return fail(PA_ERR_HIP, std::string(fn) + ": " + hipGetErrorString(e));
  return pa::ok();
}

// Argument checks shared by pa_decode and pa_mixed_step (PA_OK when valid).
pa_status check_decode(const pa::KvDesc& d, const std::string& fn, int32_t num_heads, const void* q,
                       const int32_t* tables_dev, const int32_t* lens_dev, int32_t B,
                       int32_t max_blocks, int32_t max_context_len, float scale,
                       const float* out_dev) {
  if (num_heads < 1 || num_heads % d.num_kv_heads != 0)
    return fail(PA_ERR_BAD_ARG, fn + ": num_heads must be a positive multiple of num_kv_heads");
  if (B < 0 || max_blocks < 1 || max_context_len < 0)
    return fail(PA_ERR_BAD_ARG, fn + ": bad B / max_blocks / max_context_len");
  if (B == 0) return PA_OK;
  if (q == nullptr || tables_dev == nullptr || lens_dev == nullptr || out_dev == nullptr)
    return fail(PA_ERR_BAD_ARG, fn + ": NULL device pointer");
  if (!aligned16(q) || !aligned16(out_dev)) return fail(PA_ERR_BAD_ARG, fn + ": q / out must be 16-byte aligned");
  if (num_heads > 65535 || B > 65535) return fail(PA_ERR_BAD_ARG, fn + ": num_heads and B must be <= 65535");
  if (!std::isfinite(scale)) return fail(PA_ERR_BAD_ARG, fn + ": scale must be finite");
  if (pa::decode_units(B, num_heads, max_context_len) > (int64_t(1) << 31) - 64)
    return fail(PA_ERR_BAD_ARG, fn + ": B * num_heads * ceil(max_context_len / 256) too large for one launch");
  return PA_OK;
}

// The caller's workspace for pa_decode and its relatives (PA_OK when large enough).
pa_status check_workspace(const pa::KvDesc& d, const std::string& fn, int32_t num_heads, int32_t B,
                          int32_t max_context_len, const void* workspace_dev, size_t workspace_bytes) {
  const size_t need = pa::decode_workspace_bytes(B, num_heads, d.head_dim, max_context_len);
  if (workspace_bytes < need || (need > 0 && workspace_dev == nullptr))
    return fail(PA_ERR_BAD_ARG, fn + ": workspace smaller than pa_decode_workspace_bytes()");
  if (need > 0 && !aligned16(workspace_dev))
    return fail(PA_ERR_BAD_ARG, fn + ": workspace must be 16-byte aligned");
  return PA_OK;
}

// Argument checks shared by pa_prefill_chunk and pa_mixed_step.
pa_status check_prefill(const pa::KvDesc& d, const std::string& fn, int32_t num_heads, const void* q,
                        int32_t total_q_rows, const int32_t* cu_q_dev, const int32_t* prior_dev,
                        const int32_t* tables_dev, int32_t B, int32_t max_blocks, int32_t max_chunk,
                        float scale, const float* out_dev) {
  if (num_heads < 1 || num_heads % d.num_kv_heads != 0)
    return fail(PA_ERR_BAD_ARG, fn + ": num_heads must be a positive multiple of num_kv_heads");
  if (B < 0 || max_blocks < 1 || max_chunk < 0 || total_q_rows < 0)
    return fail(PA_ERR_BAD_ARG, fn + ": bad B / max_blocks / max_chunk / total_q_rows");
  if (B == 0 || total_q_rows == 0 || max_chunk == 0) return PA_OK;
  if (q == nullptr || cu_q_dev == nullptr || prior_dev == nullptr || tables_dev == nullptr ||
      out_dev == nullptr)
    return fail(PA_ERR_BAD_ARG, fn + ": NULL device pointer");
  if (!aligned16(q) || !aligned16(out_dev))
    return fail(PA_ERR_BAD_ARG, fn + ": q / out must be 16-byte aligned");
  if (num_heads > 65535 || B > 65535)
    return fail(PA_ERR_BAD_ARG, fn + ": num_heads and B must be <= 65535");
  if (!std::isfinite(scale)) return fail(PA_ERR_BAD_ARG, fn + ": scale must be finite");
  return PA_OK;
}

// Copy-on-write pairs: host int32[n][2], distinct in-pool ids.
pa_status check_cow(const pa::KvDesc& d, const std::string& fn, const int32_t* pairs, int32_t n) {
  if (n < 0) return fail(PA_ERR_BAD_ARG, fn + ": negative count");
  if (n == 0) return PA_OK;
  if (pairs == nullptr) return fail(PA_ERR_BAD_ARG, fn + ": NULL cow pairs");
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = pairs[2 * i], t = pairs[2 * i + 1];
    if (s < 0 || s >= d.num_blocks || t < 0 || t >= d.num_blocks || s == t)
      return fail(PA_ERR_BAD_ARG, fn + ": cow pair out of range");
  }
  return PA_OK;
}

}  // namespace

extern "C" {


pa_status pa_write_kv(const pa_kv_cache* cache, const void* k_new, const void* v_new,
                      const int32_t* slots_dev, int32_t T, const int32_t* cow_pairs_host,
                      int32_t n_cow, void* hip_stream) {
  const char* fn = "pa_write_kv";
  pa::KvDesc d;
  if (pa_status st = check_cache(cache, fn, &d); st != PA_OK) return st;
  if (T < 0 || n_cow < 0) return fail(PA_ERR_BAD_ARG, "pa_write_kv: negative count");
  if (T > 0 && (k_new == nullptr || v_new == nullptr || slots_dev == nullptr))
    return fail(PA_ERR_BAD_ARG, "pa_write_kv: NULL k_new / v_new / slots");
  if (T > 0 && (!aligned16(k_new) || !aligned16(v_new)))
    return fail(PA_ERR_BAD_ARG, "pa_write_kv: k_new / v_new must be 16-byte aligned");
  if (static_cast<int64_t>(T) * d.num_kv_heads * (d.head_dim / 8) >= (int64_t(1) << 31) * 256)
    return fail(PA_ERR_BAD_ARG, "pa_write_kv: too many tokens for one launch");
  if (pa_status st = check_cow(d, fn, cow_pairs_host, n_cow); st != PA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (n_cow > 0) {
    const hipError_t e = pa::launch_copy_blocks(d, cow_pairs_host, n_cow, s);
    if (e != hipSuccess) return hip_status(e, fn);
  }
  return hip_status(pa::launch_write_kv(d, k_new, v_new, slots_dev, T, s), fn);
}

size_t pa_decode_workspace_bytes(int32_t B, int32_t num_heads, int32_t head_dim,
                                 int32_t max_context_len) {
  return pa::decode_workspace_bytes(B, num_heads, head_dim, max_context_len);
}

pa_status pa_decode(const pa_kv_cache* cache, const void* q, int32_t num_heads,
                    const int32_t* tables_dev, const int32_t* lens_dev,
                    const int32_t* cached_blocks_dev, int32_t B, int32_t max_blocks,
                    int32_t max_context_len, float scale, float* out_dev, void* workspace_dev,
                    size_t workspace_bytes, void* hip_stream) {
  const char* fn = "pa_decode";
  pa::KvDesc d;
  if (pa_status st = check_cache(cache, fn, &d); st != PA_OK) return st;
  if (pa_status st = check_decode(d, fn, num_heads, q, tables_dev, lens_dev, B, max_blocks,
                                  max_context_len, scale, out_dev);
      st != PA_OK)
    return st;
  if (pa_status st = check_workspace(d, fn, num_heads, B, max_context_len, workspace_dev,
                                     workspace_bytes);
      st != PA_OK)
    return st;
  if (B == 0) return pa::ok();
  return hip_status(pa::launch_decode(d, q, num_heads, tables_dev, lens_dev, cached_blocks_dev, B,
                                      max_blocks, max_context_len, scale, out_dev, workspace_dev,
                                      static_cast<hipStream_t>(hip_stream)),
                    fn);
}

pa_status pa_decode_noalloc(const pa_kv_cache* cache, const void* q, int32_t num_heads,
                            const int32_t* tables_dev, const int32_t* lens_dev,
                            const int32_t* cached_blocks_dev, int32_t B, int32_t max_blocks,
                            int32_t max_context_len, float scale, float* out_dev, void* hip_stream) {
  const char* fn = "pa_decode_noalloc";
  pa::KvDesc d;
  if (pa_status st = check_cache(cache, fn, &d); st != PA_OK) return st;
  const size_t need = pa::decode_workspace_bytes(B, num_heads, d.head_dim, max_context_len);
  if (need > pa::decode_scratch_capacity())
    return fail(PA_ERR_CAPACITY, std::string(fn) + ": this batch needs " + std::to_string(need) +
                                     " bytes of split partials, over the library's static " +
                                     std::to_string(pa::decode_scratch_capacity()) +
                                     "-byte scratch; use pa_decode with a workspace");
  if (pa_status st = check_decode(d, fn, num_heads, q, tables_dev, lens_dev, B, max_blocks,
                                  max_context_len, scale, out_dev);
      st != PA_OK)
    return st;
  if (B == 0) return pa::ok();
  void* ws = nullptr;
  if (const hipError_t e = pa::decode_scratch(&ws); e != hipSuccess) return hip_status(e, fn);
  return hip_status(pa::launch_decode(d, q, num_heads, tables_dev, lens_dev, cached_blocks_dev, B,
                                      max_blocks, max_context_len, scale, out_dev, ws,
                                      static_cast<hipStream_t>(hip_stream)),
                    fn);
}

pa_status pa_decode_append(const pa_kv_cache* cache, const void* q, int32_t num_heads,
                           const void* k_new, const void* v_new, const int32_t* tables_dev,
                           const int32_t* lens_dev, const int32_t* cached_blocks_dev, int32_t B,
                           int32_t max_blocks, int32_t max_context_len, float scale, float* out_dev,
                           void* workspace_dev, size_t workspace_bytes,
                           const int32_t* cow_pairs_host, int32_t n_cow, void* hip_stream) {
  const char* fn = "pa_decode_append";
  pa::KvDesc d;
  if (pa_status st = check_cache(cache, fn, &d); st != PA_OK) return st;
  if (pa_status st = check_decode(d, fn, num_heads, q, tables_dev, lens_dev, B, max_blocks,
                                  max_context_len, scale, out_dev);
      st != PA_OK)
    return st;
  if (pa_status st = check_workspace(d, fn, num_heads, B, max_context_len, workspace_dev,
                                     workspace_bytes);
      st != PA_OK)
    return st;
  if (B > 0 && (k_new == nullptr || v_new == nullptr))
    return fail(PA_ERR_BAD_ARG, std::string(fn) + ": NULL k_new / v_new");
  if (B > 0 && (!aligned16(k_new) || !aligned16(v_new)))
    return fail(PA_ERR_BAD_ARG, std::string(fn) + ": k_new / v_new must be 16-byte aligned");
  if (pa_status st = check_cow(d, fn, cow_pairs_host, n_cow); st != PA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (n_cow > 0) {
    const hipError_t e = pa::launch_copy_blocks(d, cow_pairs_host, n_cow, s);
    if (e != hipSuccess) return hip_status(e, fn);
  }
  if (B == 0) return pa::ok();
  const pa::DecodeAppend append{k_new, v_new};
  return hip_status(pa::launch_decode(d, q, num_heads, tables_dev, lens_dev, cached_blocks_dev, B,
                                      max_blocks, max_context_len, scale, out_dev, workspace_dev, s,
                                      &append),
                    fn);
}

pa_status pa_prefill_chunk(const pa_kv_cache* cache, const void* q, int32_t num_heads,
                           int32_t total_q_rows, const int32_t* cu_q_dev, const int32_t* prior_dev,
                           const int32_t* tables_dev, int32_t B, int32_t max_blocks,
                           int32_t max_chunk, float scale, float* out_dev, void* hip_stream) {
  const char* fn = "pa_prefill_chunk";
  pa::KvDesc d;
  if (pa_status st = check_cache(cache, fn, &d); st != PA_OK) return st;
  if (pa_status st = check_prefill(d, fn, num_heads, q, total_q_rows, cu_q_dev, prior_dev, tables_dev,
                                   B, max_blocks, max_chunk, scale, out_dev);
      st != PA_OK)
    return st;
  if (B == 0 || total_q_rows == 0 || max_chunk == 0) return pa::ok();
  return hip_status(pa::launch_prefill(d, q, num_heads, total_q_rows, cu_q_dev, prior_dev,
                                       tables_dev, B, max_blocks, max_chunk, scale, out_dev,
                                       static_cast<hipStream_t>(hip_stream)),
                    fn);
}

pa_status pa_mixed_step(const pa_kv_cache* cache, int32_t num_heads, float scale,
                        const pa_prefill_batch* prefill, const pa_decode_batch* decode,
                        void* hip_stream) {
  const char* fn = "pa_mixed_step";
  pa::KvDesc d;
  if (pa_status st = check_cache(cache, fn, &d); st != PA_OK) return st;
  const bool has_p = prefill != nullptr && prefill->batch > 0 && prefill->total_q > 0 &&
                     prefill->max_chunk > 0;
  const bool has_d = decode != nullptr && decode->batch > 0;
  if (prefill != nullptr) {
    const pa_prefill_batch& p = *prefill;
    if (pa_status st = check_prefill(d, fn, num_heads, p.q, p.total_q, p.cu_q, p.prior, p.tables,
                                     p.batch, p.max_blocks, p.max_chunk, scale, p.out);
        st != PA_OK)
      return st;
  }
  if (decode != nullptr) {
    const pa_decode_batch& q = *decode;
    if (pa_status st = check_decode(d, fn, num_heads, q.q, q.tables, q.lens, q.batch, q.max_blocks,
                                    q.max_context_len, scale, q.out);
        st != PA_OK)
      return st;
    if (pa_status st = check_workspace(d, fn, num_heads, q.batch, q.max_context_len, q.workspace,
                                       q.workspace_bytes);
        st != PA_OK)
      return st;
  }
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (has_p && has_d && decode->max_context_len <= pa::mixed_max_context(d.block_size)) {
    const pa::MixedPrefill mp{prefill->q, prefill->total_q, prefill->cu_q, prefill->prior,
                              prefill->tables, prefill->batch, prefill->max_blocks,
                              prefill->max_chunk, prefill->out};
    const pa::MixedDecode md{decode->q, decode->tables, decode->lens, decode->cached_blocks,
                             decode->batch, decode->max_blocks, decode->max_context_len, decode->out};
    return hip_status(pa::launch_mixed(d, num_heads, scale, mp, md, s), fn);
  }
  // one part only, or decode contexts beyond the mixed launch: separate launches
  if (has_p) {
    const hipError_t e = pa::launch_prefill(d, prefill->q, num_heads, prefill->total_q, prefill->cu_q,
                                            prefill->prior, prefill->tables, prefill->batch,
                                            prefill->max_blocks, prefill->max_chunk, scale,
                                            prefill->out, s);
    if (e != hipSuccess) return hip_status(e, fn);
  }
  if (has_d)
    return hip_status(pa::launch_decode(d, decode->q, num_heads, decode->tables, decode->lens,
                                        decode->cached_blocks, decode->batch, decode->max_blocks,
                                        decode->max_context_len, scale, decode->out,
                                        decode->workspace, s),
                      fn);
  return pa::ok();
}

pa_status pa_swap_blocks(const pa_kv_cache* cache, void* host_k, void* host_v,
                         int32_t num_host_blocks, const int32_t* pairs_host, int32_t n_pairs,
                         int32_t direction, void* hip_stream) {
  const char* fn = "pa_swap_blocks";
  pa::KvDesc d;
  if (pa_status st = check_cache(cache, fn, &d); st != PA_OK) return st;
  if (n_pairs < 0 || num_host_blocks < 0 || (direction != 0 && direction != 1))
    return fail(PA_ERR_BAD_ARG, "pa_swap_blocks: bad count or direction");
  if (n_pairs == 0) return pa::ok();
  if (pairs_host == nullptr || host_k == nullptr || host_v == nullptr)
    return fail(PA_ERR_BAD_ARG, "pa_swap_blocks: NULL pointer");
  for (int32_t i = 0; i < n_pairs; ++i) {
    const int32_t dev = pairs_host[2 * i + (direction == 0 ? 0 : 1)];
    const int32_t host = pairs_host[2 * i + (direction == 0 ? 1 : 0)];
    if (dev < 0 || dev >= d.num_blocks || host < 0 || host >= num_host_blocks)
      return fail(PA_ERR_BAD_ARG, "pa_swap_blocks: block id out of range");
  }
  const size_t block_bytes =
      static_cast<size_t>(d.num_kv_heads) * d.block_size * d.head_dim * (d.fp8 ? 1 : 2);
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  // runs of consecutive device and host ids go in one copy per cache
  int32_t i = 0;
  while (i < n_pairs) {
    const int32_t dev0 = pairs_host[2 * i + (direction == 0 ? 0 : 1)];
    const int32_t host0 = pairs_host[2 * i + (direction == 0 ? 1 : 0)];
    int32_t run = 1;
    while (i + run < n_pairs &&
           pairs_host[2 * (i + run) + (direction == 0 ? 0 : 1)] == dev0 + run &&
           pairs_host[2 * (i + run) + (direction == 0 ? 1 : 0)] == host0 + run)
      ++run;
    const size_t bytes = block_bytes * run;
    for (int which = 0; which < 2; ++which) {
      char* dev_base = static_cast<char*>(which == 0 ? d.k : d.v) + block_bytes * dev0;
      char* host_base = static_cast<char*>(which == 0 ? host_k : host_v) + block_bytes * host0;
      const hipError_t e =
          direction == 0 ? hipMemcpyAsync(host_base, dev_base, bytes, hipMemcpyDeviceToHost, s)
                         : hipMemcpyAsync(dev_base, host_base, bytes, hipMemcpyHostToDevice, s);
      if (e != hipSuccess) return hip_status(e, fn);
    }
    i += run;
  }
  return pa::ok();
}

}  // extern "C"
