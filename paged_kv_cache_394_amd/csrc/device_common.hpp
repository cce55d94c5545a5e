// Device-side helpers shared by the gfx950 kernels: vector types, the e4m3
// encoder, wave64 lane reductions.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa {
namespace dev {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

// fp32 -> OCP e4m3 code, round to nearest even.  |x| <= 448 and x not NaN
// (the caller clamps).  Normal range: round the 23-bit mantissa to 3 bits with
// the usual add-half-minus-one-plus-lsb trick, then rebias the exponent from
// 127 to 7; a mantissa carry rolls into the exponent as it should.  Below 2^-6
// the format is a fixed grid of 2^-9 steps, so scale by 2^9 (exact) and round
// to an integer with ties to even.
__device__ __forceinline__ uint32_t e4m3_from_f32(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  uint32_t abits = bits & 0x7fffffffu;
  const float a = __uint_as_float(abits);
  uint32_t code;
  if (a < 0.015625f) {
    code = static_cast<uint32_t>(__builtin_rintf(a * 512.0f));
  } else {
    abits += 0x7ffffu + ((abits >> 20) & 1u);
    code = (abits >> 20) - (120u << 3);
  }
  return sign | code;
}

// Quantise with a per-tensor scale: encode(clamp(x / scale, -448, 448)).  The
// division is IEEE (hipcc's default for fp32 '/').
__device__ __forceinline__ uint32_t e4m3_quant(float x, float scale) {
  float q = x / scale;
  q = fminf(fmaxf(q, -448.0f), 448.0f);
  return e4m3_from_f32(q);
}

// DPP lane moves within a 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Sum over aligned groups of N lanes (N in {1,2,4,8,16}) inside each 16-lane row;
// every lane of a group receives the group's sum.  After the two quad swaps a
// lane holds its quad's sum; the half-row mirror pairs each lane with one of the
// other quad of its 8-lane half; the row mirror pairs it with the other half.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp_mov<kDppQuadXor1>(v);
  if constexpr (N >= 4) v += dpp_mov<kDppQuadXor2>(v);
  if constexpr (N >= 8) v += dpp_mov<kDppRowHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_mov<kDppRowMirror>(v);
  return v;
}

// Butterfly over lanes l, l^M, l^2M, ... up to l^32 (M a power of two >= 1).
template <int M>
__device__ __forceinline__ float xor_max_from(float v) {
#pragma unroll
  for (int s = M; s < 64; s <<= 1) v = fmaxf(v, __shfl_xor(v, s, 64));
  return v;
}

template <int M>
__device__ __forceinline__ float xor_sum_from(float v) {
#pragma unroll
  for (int s = M; s < 64; s <<= 1) v += __shfl_xor(v, s, 64);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace dev
}  // namespace pa
