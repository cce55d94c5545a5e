// Host-side launchers of the gfx950 kernels (one translation unit per kernel
// family).  Arguments are validated by the C ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "pa.h"

namespace pa {

struct KvDesc {
  void* k;
  void* v;
  int32_t num_blocks, block_size, num_kv_heads, head_dim;
  bool fp8;
  float k_scale, v_scale;
};

// Copy whole blocks src -> dst in both caches; pairs: host int32[n][2].
hipError_t launch_copy_blocks(const KvDesc& c, const int32_t* pairs, int32_t n, hipStream_t s);

// Scatter T tokens' K/V rows to their slots.
hipError_t launch_write_kv(const KvDesc& c, const void* k_new, const void* v_new,
                           const int32_t* slots, int32_t T, hipStream_t s);

// Split-K decode: split kernel + split reduce.
int32_t decode_partition_tokens();
size_t decode_workspace_bytes(int32_t B, int32_t Hq, int32_t D, int32_t max_context_len);
// The split path's partials in a static per-GPU array instead of a caller
// workspace: its size, and this GPU's copy (looked up once per device).
size_t decode_scratch_capacity();
hipError_t decode_scratch(void** ptr);
// Work units (one wave each) of one decode launch; must stay below 2^31.
int64_t decode_units(int32_t B, int32_t Hq, int32_t max_context_len);
// The new token of every sequence for an appending decode: k_new / v_new are
// fp16 [B][Hkv][D]; sequence b's row goes to its token lens[b] - 1.
struct DecodeAppend {
  const void* k_new;
  const void* v_new;
};
// cached: NULL or int32[B], leading blocks per sequence read through the caches.
// append: NULL, or the new tokens written into the cache by the same launch.
hipError_t launch_decode(const KvDesc& c, const void* q, int32_t Hq, const int32_t* tables,
                         const int32_t* lens, const int32_t* cached, int32_t B, int32_t max_blocks,
                         int32_t max_context_len, float scale, float* out, void* workspace,
                         hipStream_t s, const DecodeAppend* append = nullptr);

// Chunked prefill (MFMA).
hipError_t launch_prefill(const KvDesc& c, const void* q, int32_t Hq, int32_t total_q,
                          const int32_t* cu_q, const int32_t* prior, const int32_t* tables,
                          int32_t B, int32_t max_blocks, int32_t max_chunk, float scale, float* out,
                          hipStream_t s);

// Mixed step: chunked prefill of some sequences and decode of others in one
// launch (fp16 or e4m3 caches).  The decode half supports contexts up to
// mixed_max_context(block_size) tokens; the caller falls back to two launches
// beyond.
struct MixedPrefill {
  const void* q;
  int32_t total_q;
  const int32_t *cu_q, *prior, *tables;
  int32_t B, max_blocks, max_chunk;
  float* out;
};
struct MixedDecode {
  const void* q;
  const int32_t *tables, *lens, *cached;
  int32_t B, max_blocks, max_ctx;
  float* out;
};
int32_t mixed_max_context(int32_t block_size);
hipError_t launch_mixed(const KvDesc& c, int32_t Hq, float scale, const MixedPrefill& p,
                        const MixedDecode& d, hipStream_t s);

}  // namespace pa
