// Device code of the paged decode shared by decode.hip (its launches) and
// mixed.hip (decode workgroups inside the mixed prefill + decode launch).
// The design notes are at the top of decode.hip.
#pragma once
#include <algorithm>
#include <cmath>

#include "device_common.hpp"
#include "launch.hpp"

namespace pa {
namespace {

using namespace dev;

// Layout of one (block, head) tile of BS tokens for the wave's loads.  The
// tile is streamed in units of kUnit tokens (the whole tile for BS <= 16,
// else 16-token slices: rows 16 j .. 16 j + 15 of a tile are contiguous), so
// the registers a step holds do not grow with the block size.
template <int D, bool FP8, int BS = 16>
struct Geom {
  static constexpr int kBytes = FP8 ? 1 : 2;
  static constexpr int kEpl = 16 / kBytes;      // values per lane per 16-byte load
  static constexpr int kLpr = D / kEpl;         // lanes per token row
  static constexpr int kRpi = 64 / kLpr;        // token rows per 1 KiB load
  static constexpr int kUnit = BS < 16 ? BS : 16;  // tokens per streamed unit
  static constexpr int kSub = BS / kUnit;          // units per block
  static constexpr int kIpb = kUnit / kRpi;        // loads per unit
  static constexpr int kTile = BS * D * kBytes;    // one (block, head) tile
  static constexpr int kUnitBytes = kUnit * D * kBytes;
  static_assert(kLpr >= 4 && kLpr <= 16, "row group must fit a DPP row");
  static_assert(kIpb >= 1 && kUnit % kRpi == 0, "unit smaller than one load");
  static_assert((kSub & (kSub - 1)) == 0, "units per block must be a power of two");
};

// Most blocks a run of u >= 1 consecutive units can touch, sub units a block
// (a run may start on any unit of its first block).
__host__ __device__ constexpr int64_t run_blocks(int64_t u, int sub) { return 1 + (u + sub - 2) / sub; }

// q . k for the lane's kEpl values.
template <bool FP8>
struct QReg;

template <>
struct QReg<false> {
  half2_t v[4];
  __device__ void load(const half_t* p) {
    const half8_t x = *reinterpret_cast<const half8_t*>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = half2_t{x[2 * j], x[2 * j + 1]};
  }
  __device__ float dot(const u32x4_t& k) const {
    // bit-cast the whole vector: a bit_cast of one element expression (k[j])
    // is compiled as a read of element 0
    const half8_t kh = __builtin_bit_cast(half8_t, k);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      s = __builtin_amdgcn_fdot2(half2_t{kh[2 * j], kh[2 * j + 1]}, v[j], s, false);
    return s;
  }
};

template <>
struct QReg<true> {
  half2_t v[8];
  __device__ void load(const half_t* p) {
    const half8_t a = *reinterpret_cast<const half8_t*>(p);
    const half8_t b = *reinterpret_cast<const half8_t*>(p + 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = half2_t{a[2 * j], a[2 * j + 1]};
      v[4 + j] = half2_t{b[2 * j], b[2 * j + 1]};
    }
  }
  // Every e4m3 value is exactly representable in f16, so widening the codes to
  // f16 pairs and using the f16 dot product loses nothing.
  __device__ float dot(const u32x4_t& k) const {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const half2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k[w], 1.0f, false);
      const half2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k[w], 1.0f, true);
      s = __builtin_amdgcn_fdot2(lo, v[2 * w], s, false);
      s = __builtin_amdgcn_fdot2(hi, v[2 * w + 1], s, false);
    }
    return s;
  }
};

// acc += p * v for the lane's kEpl values.
template <bool FP8>
__device__ __forceinline__ void axpy(float* acc, float p, const u32x4_t& v);

template <>
__device__ __forceinline__ void axpy<false>(float* acc, float p, const u32x4_t& v) {
  const half8_t h = __builtin_bit_cast(half8_t, v);
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = fmaf(p, static_cast<float>(h[e]), acc[e]);
}

template <>
__device__ __forceinline__ void axpy<true>(float* acc, float p, const u32x4_t& v) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(v[w]), false);
    const float2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(v[w]), true);
    acc[4 * w + 0] = fmaf(p, lo[0], acc[4 * w + 0]);
    acc[4 * w + 1] = fmaf(p, lo[1], acc[4 * w + 1]);
    acc[4 * w + 2] = fmaf(p, hi[0], acc[4 * w + 2]);
    acc[4 * w + 3] = fmaf(p, hi[1], acc[4 * w + 3]);
  }
}

// One lane's 16-byte chunk of a new token's K and V row, in the cache's
// format.
struct NewRow {
  u32x4_t k, v;
};

// The lane's chunk (kEpl values from src, fp16) of a new token's row in the
// cache's format: the fp16 bytes, or e4m3 codes with the same encoding as the
// KV write.
template <bool FP8>
__device__ __forceinline__ u32x4_t new_row_chunk(const half_t* src, float scale) {
  if constexpr (!FP8) {
    return *reinterpret_cast<const u32x4_t*>(src);
  } else {
    const half8_t lo = *reinterpret_cast<const half8_t*>(src);
    const half8_t hi = *reinterpret_cast<const half8_t*>(src + 8);
    u32x4_t r;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = 4 * w + j;  // value e of the chunk is byte e
        word |= e4m3_quant(static_cast<float>(e < 8 ? lo[e] : hi[e - 8]), scale) << (8 * j);
      }
      r[w] = word;
    }
    return r;
  }
}

// The new tokens of an appending decode: k_new / v_new fp16 [B][Hkv][D]
// (sequence b's row is its token lens[b] - 1), the cache bases to write them
// to, and the e4m3 scales used to encode them for an fp8 cache.
struct AppendRows {
  const half_t* k_new;
  const half_t* v_new;
  uint8_t* k_dst;
  uint8_t* v_dst;
  float k_scale, v_scale;
};

// The lane's chunk of sequence b's new row for kv head kvh.
template <int D, bool FP8>
__device__ __forceinline__ NewRow load_new_row(const AppendRows& ap, int b, int kvh, int Hkv, int col) {
  const int64_t src = (static_cast<int64_t>(b) * Hkv + kvh) * D + col * Geom<D, FP8>::kEpl;
  return NewRow{new_row_chunk<FP8>(ap.k_new + src, ap.k_scale),
                new_row_chunk<FP8>(ap.v_new + src, ap.v_scale)};
}

// The lanes of token row 0 store the new row at token L - 1 (L >= 1) of
// physical block blk (the table's entry, unclamped: ids outside the pool are
// skipped, like out-of-range slots in the KV write).
template <int D, bool FP8, int BS>
__device__ __forceinline__ void store_new_row(const AppendRows& ap, const NewRow& nr, int blk, int kvh,
                                              int Hkv, int L, int num_blocks, int col, int row) {
  using G = Geom<D, FP8, BS>;
  if (row != 0 || static_cast<uint32_t>(blk) >= static_cast<uint32_t>(num_blocks)) return;
  const int64_t dst = (static_cast<int64_t>(blk) * Hkv + kvh) * G::kTile +
                      static_cast<int64_t>((L - 1) % BS) * D * G::kBytes + col * 16;
  *reinterpret_cast<u32x4_t*>(ap.k_dst + dst) = nr.k;
  *reinterpret_cast<u32x4_t*>(ap.v_dst + dst) = nr.v;
}

// K and V of kU units held in registers.
template <int D, bool FP8, int kU, int BS>
struct Tiles {
  u32x4_t k[kU][Geom<D, FP8, BS>::kIpb];
  u32x4_t v[kU][Geom<D, FP8, BS>::kIpb];
};

// Running state of one wave's online softmax.
template <int D, bool FP8>
struct Softmax {
  float m = -INFINITY;  // running max of the log2-domain scores
  float l = 0.f;        // running sum of exp2(s - m), per lane (rows summed at the end)
  float acc[Geom<D, FP8>::kEpl] = {};
};

// Block ids blk0 .. blk0 + n - 1 of one table row, lane j of register r holding
// entry blk0 + 64 r + j (0 past n).
template <int kTR>
__device__ __forceinline__ void load_block_ids(int (&tb)[kTR], const int32_t* __restrict__ trow,
                                               int blk0, int n, int lane) {
#pragma unroll
  for (int r = 0; r < kTR; ++r) {
    const int jj = r * 64 + lane;
    tb[r] = jj < n ? trow[blk0 + jj] : 0;
  }
}

// Entry bi of the block ids a wave loaded (load_block_ids), wave-uniform.
template <int kTR>
__device__ __forceinline__ int block_id_at(const int (&tb)[kTR], int bi) {
  int src = tb[0];
#pragma unroll
  for (int r = 1; r < kTR; ++r) src = (bi >= r * 64) ? tb[r] : src;
  return __builtin_amdgcn_readlane(src, bi & 63);
}

// Ids outside the pool read as block 0.
template <int kTR>
__device__ __forceinline__ void clamp_block_ids(int (&tb)[kTR], int num_blocks) {
#pragma unroll
  for (int r = 0; r < kTR; ++r)
    tb[r] = (static_cast<uint32_t>(tb[r]) < static_cast<uint32_t>(num_blocks)) ? tb[r] : 0;
}

// One 16-byte K/V load.  Each K/V byte of a call is read once, except blocks
// that several sequences share, so the loads default to non-temporal (they do
// not displace other lines from the caches; 233 -> 207 us on the 64-sequence
// 13B-shape decode); kNT = false reads through the caches, for shared blocks.
template <bool kNT>
__device__ __forceinline__ u32x4_t load_kv(const uint8_t* p) {
  if constexpr (kNT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  else return *reinterpret_cast<const u32x4_t*>(p);
}

// One wave's pass over nb >= 1 units of one (sequence, head): logical units
// u0 .. u0 + nb - 1 (unit u is slice u % kSub of logical block u / kSub);
// lane j of tb holds the physical id of logical block u0 / kSub + j (64 per
// register); context length L (tokens at or past L are masked).  kbase /
// vbase point at the (block 0, kv head) tile plus the lane's 16-byte offset.
// Leaves the online-softmax state in sm.  kNT picks the load flavour
// (load_kv).  With kAppend, token L - 1 is a new token whose row is taken
// from nr instead of the cache (its cache row is being written by the same
// launch).
template <int D, bool FP8, int kU, bool kPipe, int kTR, bool kNT, int BS, bool kAppend = false>
__device__ __forceinline__ void stream_blocks(const QReg<FP8>& qr, const int (&tb)[kTR], int nb,
                                              int u0, int L, const uint8_t* kbase,
                                              const uint8_t* vbase, int64_t blk_stride,
                                              float qk_scale, int row, Softmax<D, FP8>& sm,
                                              const NewRow& nr = NewRow{}) {
  using G = Geom<D, FP8, BS>;

  // Issue the loads of units j .. j+kU-1 of the run (past-the-end slots
  // reload the last unit and are masked when consumed).
  auto issue = [&](Tiles<D, FP8, kU, BS>& t, int j) {
    int64_t off[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int lu = u0 + min(j + u, nb - 1);              // wave-uniform
      const int bi = lu / G::kSub - u0 / G::kSub;          // block slot in tb
      int src = tb[0];
#pragma unroll
      for (int r = 1; r < kTR; ++r) src = (bi >= r * 64) ? tb[r] : src;
      const int phys = __builtin_amdgcn_readlane(src, bi & 63);
      off[u] = static_cast<int64_t>(phys) * blk_stride + (lu % G::kSub) * G::kUnitBytes;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int i = 0; i < G::kIpb; ++i)
        t.k[u][i] = load_kv<kNT>(kbase + off[u] + i * 1024);
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int i = 0; i < G::kIpb; ++i)
        t.v[u][i] = load_kv<kNT>(vbase + off[u] + i * 1024);
  };

  auto consume = [&](Tiles<D, FP8, kU, BS>& t, int j) {
    if constexpr (kAppend) {
      // the step holding token L - 1 (a uniform branch)
      if ((u0 + j) * G::kUnit < L && L <= (u0 + j + kU) * G::kUnit) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
#pragma unroll
          for (int i = 0; i < G::kIpb; ++i) {
            if ((u0 + j + u) * G::kUnit + i * G::kRpi + row == L - 1) {
              t.k[u][i] = nr.k;
              t.v[u][i] = nr.v;
            }
          }
        }
      }
    }
    float s[kU][G::kIpb];
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int i = 0; i < G::kIpb; ++i) s[u][i] = group_sum<G::kLpr>(qr.dot(t.k[u][i])) * qk_scale;
    // Only the step holding the end of the run or of the context has rows to
    // mask (tokens at or past L, past-the-end block slots): a uniform branch.
    if (j + kU > nb || (u0 + j + kU) * G::kUnit > L) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
#pragma unroll
        for (int i = 0; i < G::kIpb; ++i) {
          const int tok = (u0 + j + u) * G::kUnit + i * G::kRpi + row;
          if (!((j + u < nb) && (tok < L))) {
            s[u][i] = -INFINITY;
            t.v[u][i] = u32x4_t{0u, 0u, 0u, 0u};  // stale rows may hold non-finite bits
          }
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int i = 0; i < G::kIpb; ++i) mx = fmaxf(mx, s[u][i]);
    mx = xor_max_from<G::kLpr>(mx);
    if (mx > sm.m) {
      const float corr = fast_exp2(sm.m - mx);
      sm.l *= corr;
#pragma unroll
      for (int e = 0; e < G::kEpl; ++e) sm.acc[e] *= corr;
      sm.m = mx;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
#pragma unroll
      for (int i = 0; i < G::kIpb; ++i) {
        const float pr = fast_exp2(s[u][i] - sm.m);
        sm.l += pr;
        axpy<FP8>(sm.acc, pr, t.v[u][i]);
      }
    }
  };

  if constexpr (kPipe) {
    // two register buffers: the loads of one step are in flight while the
    // other is consumed
    Tiles<D, FP8, kU, BS> ta, tb2;
    issue(ta, 0);
    for (int j = 0;; j += 2 * kU) {
      const bool more1 = j + kU < nb;
      if (more1) issue(tb2, j + kU);
      consume(ta, j);
      if (!more1) break;
      const bool more2 = j + 2 * kU < nb;
      if (more2) issue(ta, j + 2 * kU);
      consume(tb2, j + kU);
      if (!more2) break;
    }
  } else {
    for (int j = 0; j < nb; j += kU) {
      Tiles<D, FP8, kU, BS> t;
      issue(t, j);
      consume(t, j);
    }
  }
}

// Sum the per-lane softmax state over the token rows of the wave: afterwards
// every lane holds the wave's sum l (returned) and its column group's acc.
template <int D, bool FP8>
__device__ __forceinline__ float sum_rows(Softmax<D, FP8>& sm) {
  using G = Geom<D, FP8>;
  const float l = xor_sum_from<G::kLpr>(sm.l);
#pragma unroll
  for (int e = 0; e < G::kEpl; ++e) sm.acc[e] = xor_sum_from<G::kLpr>(sm.acc[e]);
  return l;
}

// Rank of lane b's sequence (b < B <= 64) when sequences are sorted by
// clamped length, longest first, ties by index; lanes >= B get rank 64.
__device__ __forceinline__ int length_rank(int Lb, int lane, int B) {
  int rank = 0;
  for (int k = 0; k < B; ++k) {
    const int Lk = __builtin_amdgcn_readlane(Lb, k);
    rank += (Lk > Lb || (Lk == Lb && k < lane)) ? 1 : 0;
  }
  return lane < B ? rank : 64;
}

// ---------------------------------------------------------------------------
// Wide batches: one workgroup of kW waves per (sequence, head).
//
// grid (B * Hq), block kW * 64.  Workgroup g serves head h = g % Hq of the
// sequence of rank g / Hq in the longest-first order (B <= 64; beyond that the
// sequences keep their index order).  Wave w streams blocks
// units [w n / kW, (w + 1) n / kW) of the context's n units; at most 64 * kTR
// blocks per wave (checked by the host).
template <int D, bool FP8, int kU, bool kPipe, int kW, int kTR, int BS, bool kAppend = false>
__device__ __forceinline__ void decode_seq_body(
    int g, const half_t* __restrict__ q, const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ cached, float* __restrict__ out, int32_t B, int32_t Hq, int32_t Hkv,
    int32_t max_blocks, int32_t ctx_cap, int32_t num_blocks, float qk_scale, float v_scale,
    const AppendRows& ap = AppendRows{}) {
  using G = Geom<D, FP8, BS>;
  static_assert(kW >= 2 && kW <= 8, "2 to 8 waves per workgroup");
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = g % Hq;
  const int r = g / Hq;
  int b, L;
  if (B <= 64) {
    int Lb = 0;
    if (lane < B) Lb = min(max(lens[lane], 0), ctx_cap);
    const uint64_t hit = __ballot(length_rank(Lb, lane, B) == r);
    b = __ffsll(static_cast<unsigned long long>(hit)) - 1;
    L = __shfl(Lb, b, 64);
  } else {
    b = r;
    L = min(max(lens[b], 0), ctx_cap);
  }
  const int64_t bh = static_cast<int64_t>(b) * Hq + h;
  const int kvh = h / (Hq / Hkv);
  const int col = lane % G::kLpr;
  const int row = lane / G::kLpr;
  const int nunit = (L + G::kUnit - 1) / G::kUnit;
  const int u0 = static_cast<int>(static_cast<int64_t>(w) * nunit / kW);
  const int nb = static_cast<int>(static_cast<int64_t>(w + 1) * nunit / kW) - u0;

  Softmax<D, FP8> sm;
  // only the wave whose run ends with the context's last unit (it holds
  // token L - 1) reads the new row; it also writes it, once per kv head
  const bool last_wave = kAppend && nb > 0 && u0 + nb == nunit;
  NewRow nr{};
  if constexpr (kAppend) {
    if (last_wave) nr = load_new_row<D, FP8>(ap, b, kvh, Hkv, col);
  }
  if (nb > 0) {
    const int b0 = u0 / G::kSub;
    int tb[kTR];
    load_block_ids<kTR>(tb, tables + static_cast<int64_t>(b) * max_blocks, b0,
                        (u0 + nb - 1) / G::kSub - b0 + 1, lane);
    QReg<FP8> qr;
    qr.load(q + bh * D + col * G::kEpl);
    int new_blk = -1;  // the new token's block, before ids are clamped
    if constexpr (kAppend) {
      if (last_wave) new_blk = block_id_at<kTR>(tb, (L - 1) / BS - b0);
    }
    clamp_block_ids<kTR>(tb, num_blocks);
    const uint8_t* kb = kc + static_cast<int64_t>(kvh) * G::kTile + lane * 16;
    const uint8_t* vb = vc + static_cast<int64_t>(kvh) * G::kTile + lane * 16;
    const int64_t stride = static_cast<int64_t>(Hkv) * G::kTile;
    // a run that starts inside the sequence's shared prefix reads through the caches
    if (cached != nullptr && b0 < cached[b])
      stream_blocks<D, FP8, kU, kPipe, kTR, false, BS, kAppend>(qr, tb, nb, u0, L, kb, vb, stride, qk_scale,
                                                                row, sm, nr);
    else
      stream_blocks<D, FP8, kU, kPipe, kTR, true, BS, kAppend>(qr, tb, nb, u0, L, kb, vb, stride, qk_scale,
                                                               row, sm, nr);
    if constexpr (kAppend) {
      if (last_wave && h % (Hq / Hkv) == 0)
        store_new_row<D, FP8, BS>(ap, nr, new_blk, kvh, Hkv, L, num_blocks, col, row);
    }
  }
  const float l = sum_rows<D, FP8>(sm);

  __shared__ float s_o[kW][D];
  __shared__ float s_m[kW];
  __shared__ float s_l[kW];
  if (row == 0) {
#pragma unroll
    for (int e = 0; e < G::kEpl; ++e) s_o[w][col * G::kEpl + e] = sm.acc[e];
  }
  if (lane == 0) {
    s_m[w] = sm.m;
    s_l[w] = l;
  }
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += kW * 64) {
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < kW; ++u) M = fmaxf(M, s_m[u]);
    float o = 0.f, ls = 0.f;
#pragma unroll
    for (int u = 0; u < kW; ++u) {
      const float f = (s_m[u] == -INFINITY) ? 0.f : fast_exp2(s_m[u] - M);
      o = fmaf(f, s_o[u][d], o);
      ls = fmaf(f, s_l[u], ls);
    }
    out[bh * D + d] = ls > 0.f ? o * v_scale / ls : 0.f;  // empty context: zeros
  }
}

// One workgroup per (sequence, head); see decode_seq_body.
template <int D, bool FP8, int kU, bool kPipe, int kW, int kTR, int BS, bool kAppend>
__global__ __launch_bounds__(kW * 64) void decode_seq_kernel(
    const half_t* __restrict__ q, const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ cached, float* __restrict__ out, int32_t B, int32_t Hq, int32_t Hkv,
    int32_t max_blocks, int32_t ctx_cap, int32_t num_blocks, float qk_scale, float v_scale,
    AppendRows ap) {
  decode_seq_body<D, FP8, kU, kPipe, kW, kTR, BS, kAppend>(blockIdx.x, q, kc, vc, tables, lens, cached, out,
                                                         B, Hq, Hkv, max_blocks, ctx_cap, num_blocks,
                                                         qk_scale, v_scale, ap);
}

}  // namespace
}  // namespace pa
