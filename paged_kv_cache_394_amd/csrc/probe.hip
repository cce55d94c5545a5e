// Measurement support, not part of the attention path.
//
// tile_gather_kernel only reads, with the decode's access pattern -- whole
// 4 KiB (block, head) tiles (16 tokens x 128 dims of fp16) picked by id from a
// large buffer, 64 lanes x 16 bytes x 4 loads per tile, eight tiles in flight
// per wave, non-temporal loads.  Its rate is the read bandwidth that pattern
// can reach on the device, the practical ceiling against which the decode's
// bandwidth is compared.
//
// mfma_loop_kernel only runs the matrix cores, with the prefill's instruction
// (v_mfma_f32_16x16x32_f16): each wave keeps kMfmaChains independent
// accumulations going on random-bit operands held in registers.  Its rate is the fp16
// matrix throughput the device sustains, clock under matrix load included:
// the practical ceiling for the chunked prefill.
#include <hip/hip_runtime.h>

#include <string>

#include "device_common.hpp"
#include "pa.h"
#include "status.hpp"

namespace pa {
namespace {

using namespace dev;

constexpr int kProbeTile = 4096;
constexpr int kProbeInFlight = 8;

// grid: ceil(n_tiles / per_wave / 4) workgroups of 4 waves; wave w reads tiles
// ids[w * per_wave .. + per_wave).  Ids are clamped into the buffer.
__global__ __launch_bounds__(256) void tile_gather_kernel(const uint8_t* __restrict__ base,
                                                          int32_t n_base_tiles,
                                                          const int32_t* __restrict__ ids,
                                                          int32_t n_tiles, int32_t per_wave,
                                                          u32x4_t* __restrict__ sink) {
  const int64_t wave = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t first = wave * per_wave;
  if (first >= n_tiles) return;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (int k = 0; k < per_wave; k += kProbeInFlight) {
    u32x4_t d[kProbeInFlight][4];
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u) {
      const int32_t id = min(max(ids[first + k + u], 0), n_base_tiles - 1);
      const u32x4_t* p = reinterpret_cast<const u32x4_t*>(base + static_cast<int64_t>(id) * kProbeTile) + lane;
#pragma unroll
      for (int i = 0; i < 4; ++i) d[u][i] = __builtin_nontemporal_load(p + 64 * i);
    }
#pragma unroll
    for (int u = 0; u < kProbeInFlight; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc ^= d[u][i];
  }
  // a data-dependent store the compiler cannot remove; taken only if the XOR of
  // everything read matches an arbitrary constant
  if (acc[0] == 0x9e3779b9u && acc[1] == 0x7f4a7c15u) sink[lane] = acc;
}

constexpr int kMfmaChains = 8;
constexpr int kMfmaOperands = 4;   // operand sets cycled through, iters is a multiple of this

// A small fp16 value with random sign and mantissa bits (magnitude in
// [2^-12, 2^-11)): operands with the bit patterns of real data.  (The same
// loop on constant operands measured 25% slower; which rate real operands get
// is what the probe is for.)
__device__ __forceinline__ half_t probe_value(uint32_t h) {
  h ^= h >> 16;
  h *= 0x7feb352du;
  h ^= h >> 15;
  const uint16_t bits = static_cast<uint16_t>((h & 0x83FFu) | (3u << 10));
  return __builtin_bit_cast(half_t, bits);
}

// grid: n_workgroups of 4 waves, `iters` rounds of kMfmaChains MFMAs a wave.
// The accumulators take a random walk of tiny steps (no overflow); they are
// folded into one value that is stored only if it equals a constant no run
// produces, so the work cannot be removed and nothing is written.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int32_t iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const uint32_t seed = (blockIdx.x * 256u + threadIdx.x) * 0x9e3779b1u;
  half8_t a[kMfmaOperands], b[kMfmaOperands];
#pragma unroll
  for (int r = 0; r < kMfmaOperands; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[r][e] = probe_value(seed + 0x632be5abu * (16 * r + e));
      b[r][e] = probe_value(~seed + 0x85ebca77u * (16 * r + e));
    }
  float4_t acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) acc[c] = float4_t{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; i += kMfmaOperands) {
#pragma unroll
    for (int r = 0; r < kMfmaOperands; ++r)
#pragma unroll
      for (int c = 0; c < kMfmaChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[r], b[(r + c) % kMfmaOperands], acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (s == -1234.5f) sink[lane] = s;
}

}  // namespace
}  // namespace pa

extern "C" pa_status pa_probe_mfma(int32_t n_workgroups, int32_t iters, float* sink_dev, void* hip_stream) {
  using pa::fail;
  const std::string f = "pa_probe_mfma";
  if (sink_dev == nullptr) return fail(PA_ERR_BAD_ARG, f + ": sink must not be NULL");
  if (n_workgroups < 0 || iters < 0 || iters % pa::kMfmaOperands != 0)
    return fail(PA_ERR_BAD_ARG, f + ": need n_workgroups >= 0 and iters a non-negative multiple of 4");
  if (n_workgroups == 0 || iters == 0) return pa::ok();
  pa::mfma_loop_kernel<<<dim3(static_cast<uint32_t>(n_workgroups)), dim3(256), 0,
                         static_cast<hipStream_t>(hip_stream)>>>(iters, sink_dev);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, f + ": " + hipGetErrorString(e));
  return pa::ok();
}

extern "C" pa_status pa_probe_tile_gather(const void* base_dev, int64_t base_bytes,
                                          const int32_t* tile_ids_dev, int32_t n_tiles,
                                          int32_t tiles_per_wave, void* sink_dev, void* hip_stream) {
  using pa::fail;
  const std::string f = "pa_probe_tile_gather";
  if (base_dev == nullptr || sink_dev == nullptr)
    return fail(PA_ERR_BAD_ARG, f + ": base and sink must not be NULL");
  if ((reinterpret_cast<uintptr_t>(base_dev) & 15u) != 0 || (reinterpret_cast<uintptr_t>(sink_dev) & 15u) != 0)
    return fail(PA_ERR_BAD_ARG, f + ": base and sink must be 16-byte aligned");
  if (base_bytes < pa::kProbeTile || base_bytes / pa::kProbeTile > INT32_MAX)
    return fail(PA_ERR_BAD_ARG, f + ": base_bytes must hold 1 .. 2^31-1 tiles of 4 KiB");
  if (n_tiles < 0 || tiles_per_wave <= 0 || tiles_per_wave % pa::kProbeInFlight != 0 ||
      n_tiles % tiles_per_wave != 0)
    return fail(PA_ERR_BAD_ARG, f + ": need n_tiles >= 0, tiles_per_wave a positive multiple of 8 "
                                    "dividing n_tiles");
  if (n_tiles > 0 && tile_ids_dev == nullptr) return fail(PA_ERR_BAD_ARG, f + ": tile_ids is NULL");
  if (n_tiles == 0) return pa::ok();
  const int64_t waves = n_tiles / tiles_per_wave;
  const int64_t grid = (waves + 3) / 4;
  pa::tile_gather_kernel<<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0,
                           static_cast<hipStream_t>(hip_stream)>>>(
      static_cast<const uint8_t*>(base_dev), static_cast<int32_t>(base_bytes / pa::kProbeTile),
      tile_ids_dev, n_tiles, tiles_per_wave, static_cast<pa::dev::u32x4_t*>(sink_dev));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, f + ": " + hipGetErrorString(e));
  return pa::ok();
}
