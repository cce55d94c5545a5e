// Paged decode attention for gfx950: one query per (sequence, head) over a KV
// cache scattered across 16-token physical blocks found through a block table
// ([p1] "vLLM PagedAttention Deep Dive", section "PagedAttention Mechanism":
// look up the physical blocks, gather their K/V, run standard attention).
//
// Decode reads every cached K/V byte once and does ~1 FLOP per byte, so the
// kernel is bound by HBM bandwidth ([p3] "PagedAttention: Why Static Batching
// Wastes Your KV Cache": the constraint is memory, not FLOPs).  The design
// follows from that:
//
// * Split-K.  The context of a (sequence, head) is cut into partitions of
//   kPartBlocks blocks; one workgroup of kWaves wave64s owns one partition and
//   each wave a contiguous run of its blocks.  A second small kernel merges the
//   partitions' (max, sum, weighted V) partials.  Sequences that fit in one
//   partition are finished by the first kernel directly.
// * Coalesced tiles.  One (block, head) tile is 16 x head_dim contiguous values.
//   Load instruction i of a wave reads bytes [1024 i, 1024 i + 1024) of the tile,
//   16 bytes per lane, so each load is one fully used 1 KiB run.  A lane then
//   holds 16 bytes of one token row; the lanes of one row (head_dim*bytes/16 of
//   them) sit in one DPP row group, where the q.k partial sums are reduced with
//   DPP moves, no LDS.
// * Online softmax per wave in the log2 domain (scores pre-scaled by log2 e, so
//   exp is the hardware exp2); the running max is wave-uniform, so the rescale
//   of the accumulators is a uniform branch taken only when the max grows.
//   V is accumulated per lane for the lane's own rows; rows are summed once per
//   wave at the end, then waves are merged through LDS.
// * e4m3 caches are widened in registers with the gfx950 packed fp8->f32
//   conversion; the K scale is folded into the score scale and the V scale is
//   applied once to the output.
#include <cmath>

#include "device_common.hpp"
#include "launch.hpp"

namespace pa {
namespace {

using namespace dev;

constexpr int kWaves = 4;
constexpr int kPartBlocks = 32;  // 512 tokens per partition
constexpr int kBlocksPerWave = kPartBlocks / kWaves;

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
  float v[16];
  __device__ void load(const half_t* p) {
    const half8_t a = *reinterpret_cast<const half8_t*>(p);
    const half8_t b = *reinterpret_cast<const half8_t*>(p + 8);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[j] = static_cast<float>(a[j]);
      v[8 + j] = static_cast<float>(b[j]);
    }
  }
  __device__ float dot(const u32x4_t& k) const {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(k[w]), false);
      const float2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(k[w]), true);
      s = fmaf(lo[0], v[4 * w + 0], s);
      s = fmaf(lo[1], v[4 * w + 1], s);
      s = fmaf(hi[0], v[4 * w + 2], s);
      s = fmaf(hi[1], v[4 * w + 3], s);
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

// grid (nparts, Hq, B), block kWaves*64.
//   qk_scale = softmax scale * log2(e) * k_scale;  v_scale = 1 for fp16.
//   ws_o [B][Hq][nparts][D], ws_ml [B][Hq][nparts][2] (max, sum), log2 domain.
template <int D, bool FP8>
__global__ __launch_bounds__(kWaves * 64) void decode_partition_kernel(
    const half_t* __restrict__ q, const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ lens, float* __restrict__ out,
    float* __restrict__ ws_o, float* __restrict__ ws_ml, int32_t Hq, int32_t Hkv,
    int32_t max_blocks, int32_t max_ctx, int32_t nparts, int32_t num_blocks, float qk_scale,
    float v_scale) {
  using G = Geom<D, FP8>;
  const int p = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t bh = static_cast<int64_t>(b) * Hq + h;

  int L = lens[b];
  L = min(max(L, 0), min(max_blocks * kBlock, max_ctx));
  const int nblk = (L + kBlock - 1) / kBlock;
  const int blk_begin = p * kPartBlocks;
  if (blk_begin >= nblk) {
    if (p == 0) {
      for (int d = threadIdx.x; d < D; d += kWaves * 64) out[bh * D + d] = 0.f;
    }
    return;
  }
  const int nparts_b = (nblk + kPartBlocks - 1) / kPartBlocks;
  const int blk_end = min(nblk, blk_begin + kPartBlocks);
  const int my_begin = blk_begin + w * kBlocksPerWave;
  const int my_end = min(blk_end, my_begin + kBlocksPerWave);
  const int kvh = h / (Hq / Hkv);
  const int col = lane % G::kLpr;
  const int row = lane / G::kLpr;

  QReg<FP8> qr;
  qr.load(q + bh * D + col * G::kEpl);

  float m_run = -INFINITY;
  float l_run = 0.f;
  float acc[G::kEpl];
#pragma unroll
  for (int e = 0; e < G::kEpl; ++e) acc[e] = 0.f;

  const int32_t* trow = tables + static_cast<int64_t>(b) * max_blocks;
  const int64_t head_off = static_cast<int64_t>(kvh) * G::kTile + lane * 16;

  // two blocks per step: one max reduction per 32 tokens, 2*kIpb loads in flight
  for (int j = my_begin; j < my_end; j += 2) {
    const bool has2 = (j + 1) < my_end;
    int phys0 = trow[j];
    phys0 = (static_cast<uint32_t>(phys0) < static_cast<uint32_t>(num_blocks)) ? phys0 : 0;
    int phys1 = has2 ? trow[j + 1] : phys0;
    phys1 = (static_cast<uint32_t>(phys1) < static_cast<uint32_t>(num_blocks)) ? phys1 : 0;
    const int64_t t0 = static_cast<int64_t>(phys0) * Hkv * G::kTile + head_off;
    const int64_t t1 = static_cast<int64_t>(phys1) * Hkv * G::kTile + head_off;
    u32x4_t kd[2][G::kIpb], vd[2][G::kIpb];
#pragma unroll
    for (int i = 0; i < G::kIpb; ++i) {
      kd[0][i] = *reinterpret_cast<const u32x4_t*>(kc + t0 + i * 1024);
      kd[1][i] = *reinterpret_cast<const u32x4_t*>(kc + t1 + i * 1024);
    }
#pragma unroll
    for (int i = 0; i < G::kIpb; ++i) {
      vd[0][i] = *reinterpret_cast<const u32x4_t*>(vc + t0 + i * 1024);
      vd[1][i] = *reinterpret_cast<const u32x4_t*>(vc + t1 + i * 1024);
    }
    float s[2][G::kIpb];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int i = 0; i < G::kIpb; ++i) {
        const int tok = (j + u) * kBlock + i * G::kRpi + row;
        const bool valid = (tok < L) && (u == 0 || has2);
        const float sc = group_sum<G::kLpr>(qr.dot(kd[u][i])) * qk_scale;
        s[u][i] = valid ? sc : -INFINITY;
        if (!valid) vd[u][i] = u32x4_t{0u, 0u, 0u, 0u};  // stale rows may hold non-finite bits
        mx = fmaxf(mx, s[u][i]);
      }
    }
    mx = xor_max_from<G::kLpr>(mx);
    if (mx > m_run) {
      const float corr = fast_exp2(m_run - mx);
      l_run *= corr;
#pragma unroll
      for (int e = 0; e < G::kEpl; ++e) acc[e] *= corr;
      m_run = mx;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int i = 0; i < G::kIpb; ++i) {
        const float pr = fast_exp2(s[u][i] - m_run);
        l_run += pr;
        axpy<FP8>(acc, pr, vd[u][i]);
      }
    }
  }

  // rows -> wave: lanes of one row hold equal l_run; sum across rows only
  l_run = xor_sum_from<G::kLpr>(l_run);
#pragma unroll
  for (int e = 0; e < G::kEpl; ++e) acc[e] = xor_sum_from<G::kLpr>(acc[e]);

  __shared__ float s_o[kWaves][D];
  __shared__ float s_m[kWaves];
  __shared__ float s_l[kWaves];
  if (row == 0) {
#pragma unroll
    for (int e = 0; e < G::kEpl; ++e) s_o[w][col * G::kEpl + e] = acc[e];
  }
  if (lane == 0) {
    s_m[w] = m_run;
    s_l[w] = l_run;
  }
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += kWaves * 64) {
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < kWaves; ++u) M = fmaxf(M, s_m[u]);
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int u = 0; u < kWaves; ++u) {
      const float f = (s_m[u] == -INFINITY) ? 0.f : fast_exp2(s_m[u] - M);
      o = fmaf(f, s_o[u][d], o);
      l = fmaf(f, s_l[u], l);
    }
    if (nparts_b == 1) {
      out[bh * D + d] = o * v_scale / l;
    } else {
      const int64_t slot = bh * nparts + p;
      ws_o[slot * D + d] = o * v_scale;
      if (d == 0) {
        ws_ml[slot * 2 + 0] = M;
        ws_ml[slot * 2 + 1] = l;
      }
    }
  }
}

// grid (Hq, B), block D: merge the partitions of (b, h).
template <int D>
__global__ __launch_bounds__(D) void decode_reduce_kernel(const float* __restrict__ ws_o,
                                                          const float* __restrict__ ws_ml,
                                                          const int32_t* __restrict__ lens,
                                                          float* __restrict__ out, int32_t Hq,
                                                          int32_t max_blocks, int32_t max_ctx,
                                                          int32_t nparts) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  int L = lens[b];
  L = min(max(L, 0), min(max_blocks * kBlock, max_ctx));
  const int nblk = (L + kBlock - 1) / kBlock;
  const int np = (nblk + kPartBlocks - 1) / kPartBlocks;
  if (np <= 1) return;
  const int64_t base = (static_cast<int64_t>(b) * Hq + h) * nparts;
  float M = -INFINITY;
  for (int p = 0; p < np; ++p) M = fmaxf(M, ws_ml[(base + p) * 2]);
  float o = 0.f, l = 0.f;
  for (int p = 0; p < np; ++p) {
    const float f = fast_exp2(ws_ml[(base + p) * 2] - M);
    o = fmaf(f, ws_o[(base + p) * D + d], o);
    l = fmaf(f, ws_ml[(base + p) * 2 + 1], l);
  }
  out[(static_cast<int64_t>(b) * Hq + h) * D + d] = o / l;
}

// Zero fill for the degenerate launch where every context is empty (a kernel,
// not a memset, so the call stays safe to capture in a graph).
__global__ __launch_bounds__(256) void zero_kernel(float* __restrict__ out, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) out[i] = 0.f;
}

template <int D, bool FP8>
hipError_t run(const KvDesc& c, const void* q, int32_t Hq, const int32_t* tables,
               const int32_t* lens, int32_t B, int32_t max_blocks, int32_t max_ctx, float scale,
               float* out, void* workspace, hipStream_t s) {
  const int32_t ctx_blocks = (max_ctx + kBlock - 1) / kBlock;
  const int32_t nparts = (ctx_blocks + kPartBlocks - 1) / kPartBlocks;
  if (B == 0) return hipSuccess;
  if (nparts == 0) {
    // every length is 0: zero output
    const int64_t n = static_cast<int64_t>(B) * Hq * D;
    zero_kernel<<<dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, s>>>(out, n);
    return hipGetLastError();
  }
  float* ws_o = static_cast<float*>(workspace);
  float* ws_ml = ws_o + static_cast<size_t>(B) * Hq * nparts * D;
  const float qk_scale = scale * kLog2e * (FP8 ? c.k_scale : 1.0f);
  const float v_scale = FP8 ? c.v_scale : 1.0f;
  decode_partition_kernel<D, FP8><<<dim3(nparts, Hq, B), dim3(kWaves * 64), 0, s>>>(
      static_cast<const half_t*>(q), static_cast<const uint8_t*>(c.k),
      static_cast<const uint8_t*>(c.v), tables, lens, out, ws_o, ws_ml, Hq, c.num_kv_heads,
      max_blocks, max_ctx, nparts, c.num_blocks, qk_scale, v_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nparts > 1) {
    decode_reduce_kernel<D><<<dim3(Hq, B), dim3(D), 0, s>>>(ws_o, ws_ml, lens, out, Hq, max_blocks,
                                                            max_ctx, nparts);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

int32_t decode_partition_tokens() { return kPartBlocks * kBlock; }

size_t decode_workspace_bytes(int32_t B, int32_t Hq, int32_t D, int32_t max_context_len) {
  if (B <= 0 || Hq <= 0 || D <= 0 || max_context_len <= 0) return 0;
  const int64_t ctx_blocks = (static_cast<int64_t>(max_context_len) + kBlock - 1) / kBlock;
  const int64_t nparts = (ctx_blocks + kPartBlocks - 1) / kPartBlocks;
  return static_cast<size_t>(B) * Hq * nparts * (D + 2) * sizeof(float);
}

hipError_t launch_decode(const KvDesc& c, const void* q, int32_t Hq, const int32_t* tables,
                         const int32_t* lens, int32_t B, int32_t max_blocks, int32_t max_ctx,
                         float scale, float* out, void* workspace, hipStream_t s) {
  if (c.head_dim == 128) {
    return c.fp8 ? run<128, true>(c, q, Hq, tables, lens, B, max_blocks, max_ctx, scale, out, workspace, s)
                 : run<128, false>(c, q, Hq, tables, lens, B, max_blocks, max_ctx, scale, out, workspace, s);
  }
  return c.fp8 ? run<64, true>(c, q, Hq, tables, lens, B, max_blocks, max_ctx, scale, out, workspace, s)
               : run<64, false>(c, q, Hq, tables, lens, B, max_blocks, max_ctx, scale, out, workspace, s);
}

}  // namespace pa
