// KV writes into the paged cache: the scatter of new tokens into their slots
// (the chunk's K/V accumulate in paged blocks: [p1] "vLLM PagedAttention Deep
// Dive", section "Mechanics of Chunked Prefill") and the whole-block copy that
// copy-on-write needs ([p3] "PagedAttention: Why Static Batching Wastes Your KV
// Cache", section "How does copy-on-write eliminate duplicate prompt KV cache?").
//
// Both are pure data movement, bound by HBM bandwidth: each lane moves 16 bytes
// per load and per store, and a (token, head) row of head_dim fp16 values is
// written by head_dim/8 adjacent lanes, so stores are full contiguous rows.
#include "device_common.hpp"
#include "launch.hpp"

namespace pa {
namespace {

using namespace dev;

// One thread per 8 consecutive values of one (token, head) row.
template <bool FP8>
__global__ __launch_bounds__(256) void write_kv_kernel(
    const half_t* __restrict__ k_new, const half_t* __restrict__ v_new,
    const int32_t* __restrict__ slots, void* __restrict__ k_cache, void* __restrict__ v_cache,
    int32_t T, int32_t Hkv, int32_t D, int32_t bs_log2, int64_t n_slots, float k_scale,
    float v_scale) {
  const int32_t chunks = D >> 3;  // 8-value chunks per row
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(T) * Hkv * chunks;
  if (gid >= total) return;
  const int32_t c = static_cast<int32_t>(gid % chunks);
  const int64_t row = gid / chunks;  // token * Hkv + head
  const int32_t h = static_cast<int32_t>(row % Hkv);
  const int64_t t = row / Hkv;
  const int32_t slot = slots[t];
  if (slot < 0 || slot >= n_slots) return;  // padding or out of range: skipped
  const int64_t blk = slot >> bs_log2;
  const int32_t off = slot & ((1 << bs_log2) - 1);
  const int64_t dst = (((blk * Hkv + h) << bs_log2) + off) * D + static_cast<int64_t>(c) * 8;
  const int64_t src = row * D + static_cast<int64_t>(c) * 8;
  const u32x4_t kb = *reinterpret_cast<const u32x4_t*>(k_new + src);
  const u32x4_t vb = *reinterpret_cast<const u32x4_t*>(v_new + src);
  if constexpr (!FP8) {
    *reinterpret_cast<u32x4_t*>(static_cast<half_t*>(k_cache) + dst) = kb;
    *reinterpret_cast<u32x4_t*>(static_cast<half_t*>(v_cache) + dst) = vb;
  } else {
    half8_t kh = __builtin_bit_cast(half8_t, kb);
    half8_t vh = __builtin_bit_cast(half8_t, vb);
    u32x2_t ko, vo;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      uint32_t kw = 0, vw = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kw |= e4m3_quant(static_cast<float>(kh[4 * w + j]), k_scale) << (8 * j);
        vw |= e4m3_quant(static_cast<float>(vh[4 * w + j]), v_scale) << (8 * j);
      }
      ko[w] = kw;
      vo[w] = vw;
    }
    *reinterpret_cast<u32x2_t*>(static_cast<uint8_t*>(k_cache) + dst) = ko;
    *reinterpret_cast<u32x2_t*>(static_cast<uint8_t*>(v_cache) + dst) = vo;
  }
}

constexpr int kMaxPairsPerLaunch = 64;
struct CopyPairs {
  int32_t src[kMaxPairsPerLaunch];
  int32_t dst[kMaxPairsPerLaunch];
};

// grid (n_pairs, 2): one workgroup copies one block of one cache (K or V) with
// 16-byte loads and stores.
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyPairs pairs, void* __restrict__ k_cache,
                                                          void* __restrict__ v_cache,
                                                          int64_t block_bytes) {
  uint8_t* base = static_cast<uint8_t*>(blockIdx.y == 0 ? k_cache : v_cache);
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(base + pairs.src[blockIdx.x] * block_bytes);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(base + pairs.dst[blockIdx.x] * block_bytes);
  const int64_t n16 = block_bytes >> 4;
  for (int64_t i = threadIdx.x; i < n16; i += blockDim.x) dst[i] = src[i];
}

}  // namespace

hipError_t launch_write_kv(const KvDesc& c, const void* k_new, const void* v_new,
                           const int32_t* slots, int32_t T, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int64_t total = static_cast<int64_t>(T) * c.num_kv_heads * (c.head_dim / 8);
  const int64_t grid = (total + 255) / 256;
  const int64_t n_slots = static_cast<int64_t>(c.num_blocks) * c.block_size;
  const int32_t lb = __builtin_ctz(static_cast<unsigned>(c.block_size));  // a power of two
  if (c.fp8) {
    write_kv_kernel<true><<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, s>>>(
        static_cast<const half_t*>(k_new), static_cast<const half_t*>(v_new), slots, c.k, c.v, T,
        c.num_kv_heads, c.head_dim, lb, n_slots, c.k_scale, c.v_scale);
  } else {
    write_kv_kernel<false><<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, s>>>(
        static_cast<const half_t*>(k_new), static_cast<const half_t*>(v_new), slots, c.k, c.v, T,
        c.num_kv_heads, c.head_dim, lb, n_slots, c.k_scale, c.v_scale);
  }
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const KvDesc& c, const int32_t* pairs, int32_t n, hipStream_t s) {
  const int64_t block_bytes =
      static_cast<int64_t>(c.num_kv_heads) * c.block_size * c.head_dim * (c.fp8 ? 1 : 2);
  for (int32_t first = 0; first < n; first += kMaxPairsPerLaunch) {
    const int32_t cnt = (n - first < kMaxPairsPerLaunch) ? (n - first) : kMaxPairsPerLaunch;
    CopyPairs p{};
    for (int32_t i = 0; i < cnt; ++i) {
      p.src[i] = pairs[2 * (first + i)];
      p.dst[i] = pairs[2 * (first + i) + 1];
    }
    copy_blocks_kernel<<<dim3(cnt, 2), dim3(256), 0, s>>>(p, c.k, c.v, block_bytes);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pa
