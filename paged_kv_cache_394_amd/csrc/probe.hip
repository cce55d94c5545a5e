// Measurement support, not part of the attention path: a kernel that only
// reads, with the decode's access pattern -- whole 4 KiB (block, head) tiles
// (16 tokens x 128 dims of fp16) picked by id from a large buffer, 64 lanes x
// 16 bytes x 4 loads per tile, eight tiles in flight per wave, non-temporal
// loads.  Its rate is the read bandwidth that pattern can reach on the device,
// the practical ceiling against which the decode's bandwidth is compared.
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

}  // namespace
}  // namespace pa

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
