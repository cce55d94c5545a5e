// Paged decode attention for gfx950: one query per (sequence, head) over a KV
// cache scattered across 16-token physical blocks found through a block table
// ([p1] "vLLM PagedAttention Deep Dive", section "PagedAttention Mechanism":
// look up the physical blocks, gather their K/V, run standard attention).
//
// Decode reads every cached K/V byte once and does ~1 FLOP per byte, so the
// kernels are bound by HBM bandwidth ([p3] "PagedAttention: Why Static Batching
// Wastes Your KV Cache": the constraint is memory, not FLOPs).  The design
// follows from that.
//
// Per wave (stream_blocks): one wave64 streams a run of blocks of one
// (sequence, head) with an online softmax.
// * The block-table entries of the run are read once, one per lane, and each
//   block id is then taken with a lane read into a scalar register, so no
//   dependent memory access sits inside the block loop.
// * Coalesced tiles.  One (block, head) tile is 16 x head_dim contiguous values.
//   Load instruction i of a wave reads bytes [1024 i, 1024 i + 1024) of the tile,
//   16 bytes per lane, so each load is one fully used 1 KiB run.  A lane then
//   holds 16 bytes of one token row; the lanes of one row (head_dim*bytes/16 of
//   them) sit in one DPP row group, where the q.k partial sums are reduced with
//   DPP moves, no LDS.
// * kU blocks of K and V are loaded per step; with kPipe the loads of the next
//   step are issued before the current one is consumed (two register buffers).
//   The K/V loads are non-temporal: each byte is read once per step, so they
//   are kept from displacing the caches' other lines (measured: 233 -> 207 us
//   on the 13B-shaped batch).
// * Online softmax in the log2 domain (scores pre-scaled by log2 e, so exp is
//   the hardware exp2); the running max is wave-uniform, so the rescale of the
//   accumulators is a uniform branch taken only when the max grows.  V is
//   accumulated per lane for the lane's own rows; rows are summed once at the
//   end.  Only the step holding the end of the context masks rows.
// * e4m3 caches are widened in registers with the gfx950 packed fp8
//   conversions (to f16 pairs for q.k, to f32 pairs for p.V); the K scale is
//   folded into the score scale and the V scale is applied once to the output.
//
// Two launch shapes, picked per call from the batch shape:
// * Wide batches (many (sequence, head) pairs): decode_seq_kernel, one
//   workgroup of W waves per (sequence, head); wave w takes the w-th of W equal
//   runs of the context and the W partial results are merged through LDS.
//   Workgroups are dispatched longest sequence first, so the kernel ends on the
//   shortest ones.  One kernel, no workspace.
// * Narrow batches with long contexts: decode_split_kernel, one wave per
//   split of kSplit blocks, and decode_reduce_kernel merging the splits'
//   (max, sum, weighted V) partials.  Units are ordered longest first as well
//   (full splits, then partial splits by decreasing size).
#include <algorithm>
#include <cmath>

#include "device_common.hpp"
#include "launch.hpp"

namespace pa {
namespace {

using namespace dev;

template <int D, bool FP8>
struct Geom {
  static constexpr int kBytes = FP8 ? 1 : 2;
  static constexpr int kEpl = 16 / kBytes;      // values per lane per 16-byte load
  static constexpr int kLpr = D / kEpl;         // lanes per token row
  static constexpr int kRpi = 64 / kLpr;        // token rows per 1 KiB load
  static constexpr int kIpb = kBlock / kRpi;    // loads per block tile
  static constexpr int kTile = kBlock * D * kBytes;
  static_assert(kLpr >= 4 && kLpr <= 16, "row group must fit a DPP row");
  static_assert(kIpb >= 1, "tile smaller than one load");
};

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

// K and V tiles of kU blocks held in registers.
template <int D, bool FP8, int kU>
struct Tiles {
  u32x4_t k[kU][Geom<D, FP8>::kIpb];
  u32x4_t v[kU][Geom<D, FP8>::kIpb];
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

// One wave's pass over nb >= 1 blocks of one (sequence, head): logical blocks
// blk0 .. blk0 + nb - 1, physical ids in tb, context length L (tokens at or
// past L are masked).  kbase / vbase point at the (block 0, kv head) tile plus
// the lane's 16-byte offset.  Leaves the online-softmax state in sm.  kNT
// picks the load flavour (load_kv).
template <int D, bool FP8, int kU, bool kPipe, int kTR, bool kNT>
__device__ __forceinline__ void stream_blocks(const QReg<FP8>& qr, const int (&tb)[kTR], int nb,
                                              int blk0, int L, const uint8_t* kbase,
                                              const uint8_t* vbase, int64_t blk_stride,
                                              float qk_scale, int row, Softmax<D, FP8>& sm) {
  using G = Geom<D, FP8>;

  // Issue the loads of blocks j .. j+kU-1 of the run (past-the-end slots
  // reload the last block and are masked when consumed).
  auto issue = [&](Tiles<D, FP8, kU>& t, int j) {
    int64_t off[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int jj = min(j + u, nb - 1);  // wave-uniform
      int src = tb[0];
#pragma unroll
      for (int r = 1; r < kTR; ++r) src = (jj >= r * 64) ? tb[r] : src;
      const int phys = __builtin_amdgcn_readlane(src, jj & 63);
      off[u] = static_cast<int64_t>(phys) * blk_stride;
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

  auto consume = [&](Tiles<D, FP8, kU>& t, int j) {
    float s[kU][G::kIpb];
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int i = 0; i < G::kIpb; ++i) s[u][i] = group_sum<G::kLpr>(qr.dot(t.k[u][i])) * qk_scale;
    // Only the step holding the end of the run or of the context has rows to
    // mask (tokens at or past L, past-the-end block slots): a uniform branch.
    if (j + kU > nb || (blk0 + j + kU) * kBlock > L) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
#pragma unroll
        for (int i = 0; i < G::kIpb; ++i) {
          const int tok = (blk0 + j + u) * kBlock + i * G::kRpi + row;
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
    Tiles<D, FP8, kU> ta, tb2;
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
      Tiles<D, FP8, kU> t;
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
// [w nblk / kW, (w + 1) nblk / kW) of the context; at most 64 * kTR blocks per
// wave (checked by the host).
template <int D, bool FP8, int kU, bool kPipe, int kW, int kTR>
__global__ __launch_bounds__(kW * 64) void decode_seq_kernel(
    const half_t* __restrict__ q, const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ cached, float* __restrict__ out, int32_t B, int32_t Hq, int32_t Hkv,
    int32_t max_blocks, int32_t ctx_cap, int32_t num_blocks, float qk_scale, float v_scale) {
  using G = Geom<D, FP8>;
  static_assert(kW >= 2 && kW <= 8, "2 to 8 waves per workgroup");
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = blockIdx.x;
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
  const int nblk = (L + kBlock - 1) / kBlock;
  const int blk0 = static_cast<int>(static_cast<int64_t>(w) * nblk / kW);
  const int nb = static_cast<int>(static_cast<int64_t>(w + 1) * nblk / kW) - blk0;

  Softmax<D, FP8> sm;
  if (nb > 0) {
    int tb[kTR];
    load_block_ids<kTR>(tb, tables + static_cast<int64_t>(b) * max_blocks, blk0, nb, lane);
    QReg<FP8> qr;
    qr.load(q + bh * D + col * G::kEpl);
    clamp_block_ids<kTR>(tb, num_blocks);
    const uint8_t* kb = kc + static_cast<int64_t>(kvh) * G::kTile + lane * 16;
    const uint8_t* vb = vc + static_cast<int64_t>(kvh) * G::kTile + lane * 16;
    const int64_t stride = static_cast<int64_t>(Hkv) * G::kTile;
    // a run that starts inside the sequence's shared prefix reads through the caches
    if (cached != nullptr && blk0 < cached[b])
      stream_blocks<D, FP8, kU, kPipe, kTR, false>(qr, tb, nb, blk0, L, kb, vb, stride, qk_scale, row, sm);
    else
      stream_blocks<D, FP8, kU, kPipe, kTR, true>(qr, tb, nb, blk0, L, kb, vb, stride, qk_scale, row, sm);
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

// ---------------------------------------------------------------------------
// Narrow batches: split-K over waves, then a merge kernel.

// Position of one split unit: sequence, split, clamped context length.
struct UnitPos {
  int b, split, L;
  bool valid;
};

// Longest-first order of the split units of a batch of at most 64 sequences,
// computed by every wave from the lengths (lane b reads lens[b]), so no
// ordering pass is launched.  Units are numbered f = unit / Hq (heads are the
// fastest index).  First come every sequence's full splits of kSplit blocks,
// then the one partly filled split of each sequence sorted by size, largest
// first (ties by sequence index), and last a zero-size unit for each empty
// context, which writes its zero output.
template <int kSplit>
__device__ __forceinline__ UnitPos longest_first_unit(int f, const int32_t* __restrict__ lens,
                                                      int B, int ctx_cap, int lane) {
  int Lb = 0;
  if (lane < B) Lb = min(max(lens[lane], 0), ctx_cap);
  const int nblk = (Lb + kBlock - 1) / kBlock;
  const int F = nblk / kSplit;      // full splits
  const int psz = nblk % kSplit;    // blocks in the partly filled split (0: none)
  const bool has_tail = lane < B && (psz != 0 || nblk == 0);
  int pre = F;  // inclusive prefix sum of F over the lanes
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(pre, o, 64);
    if (lane >= o) pre += t;
  }
  const int total_full = __shfl(pre, 63, 64);
  UnitPos r;
  if (f < total_full) {
    const int b = __popcll(__ballot(pre <= f));  // sequences whose full splits all precede f
    r.b = b;
    r.split = f - __shfl(pre - F, b, 64);
    r.L = __shfl(Lb, b, 64);
    r.valid = true;
    return r;
  }
  const int p = f - total_full;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int rank = 0;
  for (int sz = kSplit - 1; sz >= 0; --sz) {
    const uint64_t m = __ballot(has_tail && psz == sz);
    if (psz < sz) rank += __popcll(m);
    if (psz == sz) rank += __popcll(m & below);
  }
  const uint64_t hit = __ballot(has_tail && rank == p);
  if (hit == 0) {
    r.valid = false;
    return r;
  }
  const int b = __ffsll(static_cast<unsigned long long>(hit)) - 1;
  r.b = b;
  r.split = __shfl(F, b, 64);
  r.L = __shfl(Lb, b, 64);
  r.valid = true;
  return r;
}

// grid (ceil(units / kWPG)), block kWPG * 64.  With kLongestFirst (B <= 64) the
// units follow longest_first_unit; otherwise unit u = (split * B + b) * Hq + h.
//   qk_scale = softmax scale * log2(e) * k_scale;  v_scale = 1 for fp16.
//   ctx_cap = min(max_blocks * 16, max_context_len): lengths are clamped to it.
//   ws_o [B][Hq][nsplit][D], ws_ml [B][Hq][nsplit][2] (max, sum), log2 domain.
template <int D, bool FP8, int kSplit, int kU, bool kPipe, int kWPG, bool kLongestFirst>
__global__ __launch_bounds__(kWPG * 64) void decode_split_kernel(
    const half_t* __restrict__ q, const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ cached, float* __restrict__ out, float* __restrict__ ws_o,
    float* __restrict__ ws_ml, int32_t B, int32_t Hq, int32_t Hkv,
    int32_t max_blocks, int32_t ctx_cap, int32_t nsplit, int32_t num_blocks, float qk_scale,
    float v_scale) {
  using G = Geom<D, FP8>;
  static_assert(kSplit % kU == 0, "a split is a whole number of steps");
  constexpr int kTR = (kSplit + 63) / 64;  // block-id registers per lane
  const int lane = threadIdx.x & 63;
  const int unit = __builtin_amdgcn_readfirstlane(blockIdx.x * kWPG + (threadIdx.x >> 6));
  const int h = unit % Hq;
  int b, split, L;
  if constexpr (kLongestFirst) {
    const UnitPos pos = longest_first_unit<kSplit>(unit / Hq, lens, B, ctx_cap, lane);
    if (!pos.valid) return;
    b = pos.b;
    split = pos.split;
    L = pos.L;
  } else {
    const int bsplit = unit / Hq;
    b = bsplit % B;
    split = bsplit / B;
    if (split >= nsplit) return;
    L = lens[b];
  }
  const int64_t bh = static_cast<int64_t>(b) * Hq + h;
  const int blk0 = split * kSplit;
  const int kvh = h / (Hq / Hkv);
  const int col = lane % G::kLpr;
  const int row = lane / G::kLpr;

  // The split's block ids (entries past the table's end are not read) and q
  // are loaded together, before either is used.
  int tb[kTR];
  load_block_ids<kTR>(tb, tables + static_cast<int64_t>(b) * max_blocks, blk0,
                      min(kSplit, max_blocks - blk0), lane);
  QReg<FP8> qr;
  qr.load(q + bh * D + col * G::kEpl);

  L = min(max(L, 0), ctx_cap);
  const int nblk = (L + kBlock - 1) / kBlock;
  if (blk0 >= nblk) {
    if (split == 0) {  // empty context: zero output
      for (int d = lane; d < D; d += 64) out[bh * D + d] = 0.f;
    }
    return;
  }
  const int nb = min(kSplit, nblk - blk0);
  const int nsplit_b = (nblk + kSplit - 1) / kSplit;
  clamp_block_ids<kTR>(tb, num_blocks);
  Softmax<D, FP8> sm;
  const uint8_t* kb = kc + static_cast<int64_t>(kvh) * G::kTile + lane * 16;
  const uint8_t* vb = vc + static_cast<int64_t>(kvh) * G::kTile + lane * 16;
  const int64_t stride = static_cast<int64_t>(Hkv) * G::kTile;
  if (cached != nullptr && blk0 < cached[b])
    stream_blocks<D, FP8, kU, kPipe, kTR, false>(qr, tb, nb, blk0, L, kb, vb, stride, qk_scale, row, sm);
  else
    stream_blocks<D, FP8, kU, kPipe, kTR, true>(qr, tb, nb, blk0, L, kb, vb, stride, qk_scale, row, sm);
  const float l = sum_rows<D, FP8>(sm);
  if (row != 0) return;
  float* dst;
  float mul;
  if (nsplit_b == 1) {
    dst = out + bh * D;
    mul = v_scale / l;
  } else {
    const int64_t slot = bh * nsplit + split;
    dst = ws_o + slot * D;
    mul = v_scale;
    if (lane == 0) {
      ws_ml[slot * 2 + 0] = sm.m;
      ws_ml[slot * 2 + 1] = l;
    }
  }
#pragma unroll
  for (int e = 0; e < G::kEpl; e += 4) {
    *reinterpret_cast<float4_t*>(dst + col * G::kEpl + e) =
        float4_t{sm.acc[e] * mul, sm.acc[e + 1] * mul, sm.acc[e + 2] * mul, sm.acc[e + 3] * mul};
  }
}

// grid (ceil(B * Hq / 4)), block 256: one wave merges the splits of one
// (b, h).  The length, every split's (max, sum) and the lane's D/64 output
// columns of every split are loaded at once (up to kMaxP splits; slots past
// the sequence's own split count are loaded but not used, and any further
// splits are merged in a second, looped pass), so the merge costs about one
// memory round trip.
template <int D, int kMaxP>
__global__ __launch_bounds__(256) void decode_reduce_kernel(const float* __restrict__ ws_o,
                                                            const float* __restrict__ ws_ml,
                                                            const int32_t* __restrict__ lens,
                                                            float* __restrict__ out, int32_t B,
                                                            int32_t Hq, int32_t ctx_cap,
                                                            int32_t nsplit, int32_t split_blocks) {
  constexpr int kCols = D / 64;
  const int lane = threadIdx.x & 63;
  const int unit = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (unit >= B * Hq) return;
  const int b = unit / Hq;
  const int64_t base = static_cast<int64_t>(unit) * nsplit;
  const int pre = min(nsplit, kMaxP);
  int L = lens[b];
  float mp[kMaxP], lp[kMaxP], op[kMaxP][kCols];
#pragma unroll
  for (int p = 0; p < kMaxP; ++p) {
    if (p < pre) {
      const float2_t ml = *reinterpret_cast<const float2_t*>(ws_ml + (base + p) * 2);
      mp[p] = ml[0];
      lp[p] = ml[1];
#pragma unroll
      for (int c = 0; c < kCols; ++c) op[p][c] = ws_o[(base + p) * D + c * 64 + lane];
    }
  }
  L = min(max(L, 0), ctx_cap);
  const int nblk = (L + kBlock - 1) / kBlock;
  const int np = (nblk + split_blocks - 1) / split_blocks;
  if (np <= 1) return;
  float M = -INFINITY;
#pragma unroll
  for (int p = 0; p < kMaxP; ++p)
    if (p < np) M = fmaxf(M, mp[p]);
  for (int p = kMaxP; p < np; ++p) M = fmaxf(M, ws_ml[(base + p) * 2]);
  float l = 0.f, acc[kCols] = {};
#pragma unroll
  for (int p = 0; p < kMaxP; ++p) {
    if (p < np) {
      const float f = fast_exp2(mp[p] - M);
      l = fmaf(f, lp[p], l);
#pragma unroll
      for (int c = 0; c < kCols; ++c) acc[c] = fmaf(f, op[p][c], acc[c]);
    }
  }
  for (int p = kMaxP; p < np; ++p) {
    const float f = fast_exp2(ws_ml[(base + p) * 2] - M);
    l = fmaf(f, ws_ml[(base + p) * 2 + 1], l);
#pragma unroll
    for (int c = 0; c < kCols; ++c) acc[c] = fmaf(f, ws_o[(base + p) * D + c * 64 + lane], acc[c]);
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int c = 0; c < kCols; ++c) out[static_cast<int64_t>(unit) * D + c * 64 + lane] = acc[c] * inv;
}

// Zero fill for the degenerate launch where every context is empty (a kernel,
// not a memset, so the call stays safe to capture in a graph).
__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ out, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) out[i] = 0.f;
}

int64_t ctx_blocks_of(int32_t max_ctx) { return (static_cast<int64_t>(max_ctx) + kBlock - 1) / kBlock; }

int32_t ctx_cap_of(int32_t max_blocks, int32_t max_ctx) {
  return static_cast<int32_t>(std::min<int64_t>(static_cast<int64_t>(max_blocks) * kBlock, max_ctx));
}

template <int D, bool FP8, int kSplit, int kU, bool kPipe, int kWPG, bool kLongestFirst>
hipError_t run_split(const KvDesc& c, const void* q, int32_t Hq, const int32_t* tables,
                     const int32_t* lens, const int32_t* cached, int32_t B, int32_t max_blocks,
                     int32_t max_ctx, float scale, float* out, void* workspace, hipStream_t s) {
  const int64_t nsplit64 = (ctx_blocks_of(max_ctx) + kSplit - 1) / kSplit;
  const int32_t nsplit = static_cast<int32_t>(nsplit64);
  const int64_t units = nsplit64 * B * Hq;
  const int32_t ctx_cap = ctx_cap_of(max_blocks, max_ctx);
  float* ws_o = static_cast<float*>(workspace);
  float* ws_ml = ws_o + static_cast<size_t>(B) * Hq * nsplit * D;
  const float qk_scale = scale * kLog2e * (FP8 ? c.k_scale : 1.0f);
  const float v_scale = FP8 ? c.v_scale : 1.0f;
  const uint32_t groups = static_cast<uint32_t>((units + kWPG - 1) / kWPG);
  decode_split_kernel<D, FP8, kSplit, kU, kPipe, kWPG, kLongestFirst>
      <<<dim3(groups), dim3(kWPG * 64), 0, s>>>(
          static_cast<const half_t*>(q), static_cast<const uint8_t*>(c.k),
          static_cast<const uint8_t*>(c.v), tables, lens, cached, out, ws_o, ws_ml, B, Hq,
          c.num_kv_heads,
          max_blocks, ctx_cap, nsplit, c.num_blocks, qk_scale, v_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nsplit > 1) {
    const uint32_t rgroups = static_cast<uint32_t>((static_cast<int64_t>(B) * Hq + 3) / 4);
    decode_reduce_kernel<D, 8><<<dim3(rgroups), dim3(256), 0, s>>>(ws_o, ws_ml, lens, out, B, Hq,
                                                                   ctx_cap, nsplit, kSplit);
    e = hipGetLastError();
  }
  return e;
}

template <int D, bool FP8, int kU, bool kPipe, int kW, int kTR>
hipError_t run_seq(const KvDesc& c, const void* q, int32_t Hq, const int32_t* tables,
                   const int32_t* lens, const int32_t* cached, int32_t B, int32_t max_blocks,
                   int32_t max_ctx, float scale, float* out, hipStream_t s) {
  const float qk_scale = scale * kLog2e * (FP8 ? c.k_scale : 1.0f);
  const float v_scale = FP8 ? c.v_scale : 1.0f;
  decode_seq_kernel<D, FP8, kU, kPipe, kW, kTR>
      <<<dim3(static_cast<uint32_t>(static_cast<int64_t>(B) * Hq)), dim3(kW * 64), 0, s>>>(
          static_cast<const half_t*>(q), static_cast<const uint8_t*>(c.k),
          static_cast<const uint8_t*>(c.v), tables, lens, cached, out, B, Hq, c.num_kv_heads,
          max_blocks, ctx_cap_of(max_blocks, max_ctx), c.num_blocks, qk_scale, v_scale);
  return hipGetLastError();
}

// Launch configurations.  Split path: blocks per split, blocks per step,
// pipelined, waves per workgroup.  Per-sequence path: blocks per step,
// pipelined, waves per workgroup (4, or 8 for batches too small to fill the
// chip with 4), block-id registers per wave (a wave takes at most 64 * kSeqTR
// blocks).
constexpr int kSplitF16 = 32, kUF16 = 2, kWpgF16 = 2;
constexpr bool kPipeF16 = true;
constexpr int kSplitF8 = 32, kUF8 = 4, kWpgF8 = 1;
constexpr bool kPipeF8 = false;
static_assert(kSplitF16 == kSplitF8, "one split size: the workspace size does not depend on dtype");
constexpr int kSeqUF16 = 2, kSeqUF8 = 4;
constexpr bool kSeqPipeF16 = false, kSeqPipeF8 = false;
constexpr int kSeqTR = 1;
// The per-sequence path is taken when the batch alone fills the chip, at least
// kSeqMinWaves waves (about three per wave slot of the 256 CUs at these
// kernels' occupancy), and no wave holds more than 64 * kSeqTR blocks.
constexpr int64_t kSeqMinWaves = 8192;

// Waves per workgroup of the per-sequence path for this batch, or 0 for the
// split path.
int seq_waves(int32_t B, int32_t Hq, int32_t max_ctx) {
  const int64_t pairs = static_cast<int64_t>(B) * Hq;
  const int64_t blocks = ctx_blocks_of(max_ctx);
  for (int w : {4, 8}) {
    if (pairs * w >= kSeqMinWaves && (blocks + w - 1) / w <= 64 * kSeqTR) return w;
  }
  return 0;
}

}  // namespace

int32_t decode_partition_tokens() { return kSplitF16 * kBlock; }

size_t decode_workspace_bytes(int32_t B, int32_t Hq, int32_t D, int32_t max_context_len) {
  if (B <= 0 || Hq <= 0 || D <= 0 || max_context_len <= 0) return 0;
  const int64_t nsplit = (ctx_blocks_of(max_context_len) + kSplitF16 - 1) / kSplitF16;
  return static_cast<size_t>(B) * Hq * nsplit * (D + 2) * sizeof(float);
}

int64_t decode_units(int32_t B, int32_t Hq, int32_t max_context_len) {
  const int64_t nsplit = (ctx_blocks_of(max_context_len) + kSplitF16 - 1) / kSplitF16;
  return nsplit * B * Hq;
}

hipError_t launch_decode(const KvDesc& c, const void* q, int32_t Hq, const int32_t* tables,
                         const int32_t* lens, const int32_t* cached, int32_t B, int32_t max_blocks,
                         int32_t max_ctx, float scale, float* out, void* workspace, hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (max_ctx <= 0) {
    // every length is 0: zero output
    const int64_t n = static_cast<int64_t>(B) * Hq * c.head_dim;
    zero_kernel<<<dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, s>>>(out, n);
    return hipGetLastError();
  }
#define PA_SEQ_ARGS c, q, Hq, tables, lens, cached, B, max_blocks, max_ctx, scale, out, s
#define PA_SPLIT_ARGS c, q, Hq, tables, lens, cached, B, max_blocks, max_ctx, scale, out, workspace, s
  const int sw = seq_waves(B, Hq, max_ctx);
  if (sw == 4) {
    if (c.head_dim == 128)
      return c.fp8 ? run_seq<128, true, kSeqUF8, kSeqPipeF8, 4, kSeqTR>(PA_SEQ_ARGS)
                   : run_seq<128, false, kSeqUF16, kSeqPipeF16, 4, kSeqTR>(PA_SEQ_ARGS);
    return c.fp8 ? run_seq<64, true, kSeqUF8, kSeqPipeF8, 4, kSeqTR>(PA_SEQ_ARGS)
                 : run_seq<64, false, kSeqUF16, kSeqPipeF16, 4, kSeqTR>(PA_SEQ_ARGS);
  }
  if (sw == 8) {
    if (c.head_dim == 128)
      return c.fp8 ? run_seq<128, true, kSeqUF8, kSeqPipeF8, 8, kSeqTR>(PA_SEQ_ARGS)
                   : run_seq<128, false, kSeqUF16, kSeqPipeF16, 8, kSeqTR>(PA_SEQ_ARGS);
    return c.fp8 ? run_seq<64, true, kSeqUF8, kSeqPipeF8, 8, kSeqTR>(PA_SEQ_ARGS)
                 : run_seq<64, false, kSeqUF16, kSeqPipeF16, 8, kSeqTR>(PA_SEQ_ARGS);
  }
  // longest-first unit order needs every length in one wave: B <= 64
  const bool lf = B <= 64;
  if (c.head_dim == 128) {
    if (c.fp8)
      return lf ? run_split<128, true, kSplitF8, kUF8, kPipeF8, kWpgF8, true>(PA_SPLIT_ARGS)
                : run_split<128, true, kSplitF8, kUF8, kPipeF8, kWpgF8, false>(PA_SPLIT_ARGS);
    return lf ? run_split<128, false, kSplitF16, kUF16, kPipeF16, kWpgF16, true>(PA_SPLIT_ARGS)
              : run_split<128, false, kSplitF16, kUF16, kPipeF16, kWpgF16, false>(PA_SPLIT_ARGS);
  }
  if (c.fp8)
    return lf ? run_split<64, true, kSplitF8, kUF8, kPipeF8, kWpgF8, true>(PA_SPLIT_ARGS)
              : run_split<64, true, kSplitF8, kUF8, kPipeF8, kWpgF8, false>(PA_SPLIT_ARGS);
  return lf ? run_split<64, false, kSplitF16, kUF16, kPipeF16, kWpgF16, true>(PA_SPLIT_ARGS)
            : run_split<64, false, kSplitF16, kUF16, kPipeF16, kWpgF16, false>(PA_SPLIT_ARGS);
#undef PA_SPLIT_ARGS
#undef PA_SEQ_ARGS
}

}  // namespace pa
