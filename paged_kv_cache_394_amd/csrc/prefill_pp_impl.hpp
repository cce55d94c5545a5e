// Chunked prefill over an fp16 cache with the two halves of an eight-wave
// workgroup taking turns on the matrix cores (the pa_prefill_chunk kernel for
// fp16 caches).  The design notes are at the top of prefill.hip; the helpers
// (block-id lookups, the K swizzle, the workgroup order) are shared with the
// four-wave body in prefill_impl.hpp, which e4m3 caches and the mixed prefill
// + decode launch use.
#pragma once
#include "prefill_impl.hpp"

namespace pa {
namespace {

using namespace dev;

constexpr int kQW = 8;                // waves per workgroup, 32 query rows each
constexpr int kQThreads = 64 * kQW;   // 512
constexpr int kQRows = 32 * kQW;      // 256 query rows per workgroup

// LDS layout of a staged tile: 64 key rows of head_dim halfs, row-major, with
// the 16-byte chunks XOR-swizzled by row.  K uses kswz (as prefill_body); V
// uses vswz, an even swizzle that keeps the two chunks of a 32-byte piece
// together and sends the 8 rows that one half-wave of transpose loads reads to
// 8 different bank groups.
template <int D>
__device__ __forceinline__ int vswz(int r) {
  if constexpr (D == 128) return (r & 7) << 1;
  else return ((r >> 1) & 3) << 1;
}

// Direct global -> LDS copy of 16 bytes a lane: lane l of the wave writes
// bytes [16 l, 16 l + 16) after `lds` (wave-uniform).  No register holds the
// data; completion is counted by vmcnt.
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// Wait until every global load of the wave, direct-to-LDS ones included, has
// landed (vmcnt 0; the other counters are not waited on).
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Zero rows [first, 64) of a staged V tile: keys past the end get weight 0,
// but stale cache rows may hold non-finite bits, and 0 * NaN is NaN.
template <int D>
__device__ __forceinline__ void zero_rows(half_t* buf, int first, int tid) {
  constexpr int CPR = D / 8;
  for (int s = first * CPR + tid; s < kBk * CPR; s += kQThreads)
    *reinterpret_cast<u32x4_t*>(buf + s * 8) = u32x4_t{0u, 0u, 0u, 0u};
}

// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

typedef __fp16 tr4_t __attribute__((__vector_size__(8)));

// Transpose load (gfx950 ds_read_b64_tr_b16): within each 16-lane group, lane
// r supplies the address of 4 consecutive halfs M[r]; lane t receives
// M[t / 4][t % 4], M[4 + t / 4][t % 4], M[8 + t / 4][t % 4], M[12 + t / 4][t % 4].
__device__ __forceinline__ u32x2_t lds_tr(const half_t* p) {
  return __builtin_bit_cast(
      u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4f16((__attribute__((address_space(3))) tr4_t*)(p)));
}

// grid (ceil(B * Hq / 8) * 8 * nqt) with nqt = ceil(max_chunk / kQRows),
// block kQThreads.  Same arguments as prefill_body for an fp16 cache; same
// result up to the rounding of the fp32 sums.
//
// Wave w owns query rows q0 + 32 w .. + 31.  Waves 0-3 (set 0) and 4-7 (set
// 1) sit on the same four SIMDs (wave w on SIMD w % 4), and the key tiles are
// processed in phases separated by workgroup barriers.  In phase 2 t set 0
// runs its matrix work (P.V of tile t - 1, then the scores of tile t) while
// set 1 runs the softmax of tile t - 1 on the vector ALUs; in phase 2 t + 1
// the roles swap.  So each SIMD always has one wave feeding its matrix core
// and one wave doing the exponentials, instead of both waves waiting on the
// same dependency chain.  K of tile t + 1 and V of tile t are copied to LDS at
// the start of phase 2 t (into the buffers of tiles t - 1 and t - 2, which no
// wave reads after phase 2 t - 1) and waited for at the end of phase 2 t + 1.
template <int D, int BS>
__device__ __forceinline__ void prefill_pp_body(
    int u, const half_t* __restrict__ q, const half_t* __restrict__ kc, const half_t* __restrict__ vc,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ prior,
    const int32_t* __restrict__ tables, float* __restrict__ out, int32_t B, int32_t Hq, int32_t Hkv,
    int32_t total_q, int32_t max_blocks, int32_t num_blocks, int32_t nqt, float qk_scale) {
  using G = PGeom<D>;
  // separate buffers, so that the compiler can tell the copies into one from
  // the reads of another
  __shared__ __attribute__((aligned(16))) half_t sK0[G::KBUF];
  __shared__ __attribute__((aligned(16))) half_t sK1[G::KBUF];
  __shared__ __attribute__((aligned(16))) half_t sV0[G::KBUF];
  __shared__ __attribute__((aligned(16))) half_t sV1[G::KBUF];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int set = w >> 2;
  const int g = lane >> 4;
  const int c16 = lane & 15;

  // workgroup -> (query tile, pair): ids 8 apart share a pair, so one XCD
  const int x = u % kXcds;
  const int rest = u / kXcds;
  const int qt = rest % nqt;
  const int pair = (rest / nqt) * kXcds + x;
  if (pair >= B * Hq) return;
  const int h = pair % Hq;
  const int rank = pair / Hq;
  int b;
  if (B <= 64) {
    int Wb = 0;
    if (lane < B) Wb = max(prior[lane], 0) + (cu_q[lane + 1] - cu_q[lane]);
    b = __ffsll(static_cast<unsigned long long>(__ballot(work_rank(Wb, lane, B) == rank))) - 1;
  } else {
    b = rank;
  }

  const int row0 = cu_q[b];
  const int C = cu_q[b + 1] - row0;
  const int P = max(prior[b], 0);
  const int q0 = qt * kQRows;
  if (q0 >= C || row0 < 0) return;
  const int L_total = min(P + C, max_blocks * BS);
  const int kvh = h / (Hq / Hkv);
  const int32_t* trow = tables + static_cast<int64_t>(b) * max_blocks;

  const bool neg = qk_scale < 0.f;
  const float c = fmaxf(neg ? -qk_scale : qk_scale, 1e-30f);

  // Q as the B operand of S^T = K Q^T: lane holds q[row c16][32 kk + 8 g .. + 8]
  half8_t qb[2][G::DK];
  int qrow[2];
  bool qvalid[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    qrow[st] = q0 + 32 * w + 16 * st + c16;
    qvalid[st] = qrow[st] < C && (row0 + qrow[st]) < total_q;
    const half_t* qp = q + (static_cast<int64_t>(row0 + qrow[st]) * Hq + h) * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < G::DK; ++kk) {
      half8_t v = qvalid[st] ? *reinterpret_cast<const half8_t*>(qp + 32 * kk) : half8_t{};
      qb[st][kk] = neg ? -v : v;
    }
  }

  float4_t o[2][G::DT];
  float m[2], l[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    m[st] = -INFINITY;
    l[st] = 0.f;
#pragma unroll
    for (int dt = 0; dt < G::DT; ++dt) o[st][dt] = float4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int wq_first = q0 + 32 * w;
  const int wq_last = min(q0 + 32 * w + 32, C) - 1;
  const int n_keys = min(P + min(q0 + kQRows, C), L_total);
  const int ntiles = (n_keys + kBk - 1) / kBk;
  // tiles holding keys some row of this wave sees: 0 .. wtiles - 1
  const int wtiles = wq_last < wq_first ? 0 : min(ntiles, (P + wq_last) / kBk + 1);

  // Staging copies.  Copy i of wave w fills 16-byte slots 64 (w + kQW i) ..
  // + 63 of a tile: 64 / CPR consecutive rows, which lie inside block slot
  // dslot[i] of the tile (wave-uniform).  Lane l copies the chunk that the
  // swizzle puts at slot 64 (w + kQW i) + l, found kbo[i] (K) or vbo[i] (V)
  // bytes into its block.  Both offsets are the same for every tile, so a copy
  // costs a block lookup and a 64-bit add; a tile's block offsets are formed
  // once, for its K copy, and reused for its V copy one step later.  Rows past
  // the context read whatever their block holds.
  constexpr int CPR = D / 8;
  constexpr int NI = kBk * CPR / 64 / kQW;
  static_assert(NI >= 1 && kBk * CPR == 64 * kQW * NI, "a tile is whole wave copies");
  int dslot[NI];
  uint32_t kbo[NI], vbo[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int s0 = 64 * (w + kQW * i);
    const int r = (s0 + lane) / CPR, ch = (s0 + lane) % CPR;
    dslot[i] = (s0 / CPR) / BS;
    const uint32_t row = static_cast<uint32_t>((kvh * BS + r % BS) * D);
    kbo[i] = 2u * (row + ((ch ^ kswz<D>(r)) << 3));
    vbo[i] = 2u * (row + ((ch ^ vswz<D>(r)) << 3));
  }
  // bytes per cache block: below 2^31 (checked when the cache is described)
  const uint32_t blk_bytes = 2u * static_cast<uint32_t>(Hkv * BS * D);
  // byte offsets of the blocks this wave copies, for the tile whose table
  // entries lanes 0 .. kBk / BS - 1 of ids hold
  auto block_offsets = [&](int ids, uint64_t (&bo)[NI]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int id = clamp_id(__builtin_amdgcn_readlane(ids, dslot[i]), num_blocks);
      bo[i] = static_cast<uint64_t>(static_cast<uint32_t>(id)) * blk_bytes;
    }
  };
  auto copy_tile = [&](half_t* buf, const half_t* cache, const uint64_t (&bo)[NI],
                       const uint32_t (&lo)[NI]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      dma16(reinterpret_cast<const char*>(cache) + bo[i] + lo[i], buf + 64 * (w + kQW * i) * 8);
  };

  // Per-lane byte offsets of the MFMA operand reads.  K: as in prefill_body.
  // V^T (the A operand of O^T = V^T P^T) by transpose loads: for 32-key pair
  // kp and dim tile dt, lane c16 of group g supplies halfs dt*16 + 4 (c16 % 4)
  // .. + 3 of key 32 kp + 4 g + c16 / 4 (+ 16 for the second load) and receives
  // keys 4 g .. 4 g + 3 of dim dt*16 + c16: the k slots 8 g .. 8 g + 7 that
  // match the P^T operand built from the score registers.
  int k_rd[G::DK][2], v_rd[G::DT];
#pragma unroll
  for (int kk = 0; kk < G::DK; ++kk)
#pragma unroll
    for (int par = 0; par < 2; ++par)
      k_rd[kk][par] = 2 * (c16 * D + (((4 * kk + g) ^ kswz<D>(16 * par + c16)) << 3));
  {
    const int key = 4 * g + (c16 >> 2);
#pragma unroll
    for (int dt = 0; dt < G::DT; ++dt)
      v_rd[dt] = 2 * (key * D + (((2 * dt + ((c16 >> 1) & 1)) ^ vswz<D>(key)) << 3) + 4 * (c16 & 1));
  }
  const char* sKb[2] = {reinterpret_cast<const char*>(sK0), reinterpret_cast<const char*>(sK1)};
  const char* sVb[2] = {reinterpret_cast<const char*>(sV0), reinterpret_cast<const char*>(sV1)};

  float4_t sacc[2][4];      // scores of one tile: [st][ks] keys 16 ks + 4 g + i, row 16 st + c16
  half2_t pk[2][4][2];      // its weights in fp16, kept for the next matrix phase

  // S^T = K Q^T for the tile in K buffer KB.
  auto scores = [&](auto kb) __attribute__((always_inline)) {
    constexpr int KB = decltype(kb)::value;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sacc[st][ks] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < G::DK; ++kk) {
      half8_t a[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        a[ks] = *reinterpret_cast<const half8_t*>(sKb[KB] + 2 * (ks * 16 * D) + k_rd[kk][ks & 1]);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int st = 0; st < 2; ++st)
          sacc[st][ks] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[ks], qb[st][kk], sacc[st][ks], 0, 0, 0);
    }
    // order: the operand reads of step kk + 1 are issued before the 8 MFMAs of
    // step kk (one step of reads in flight, 32 registers)
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
    for (int kk = 0; kk < G::DK; ++kk) {
      if (kk + 1 < G::DK) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 8, 0);
    }
  };

  // O^T += V^T P^T for the tile in V buffer VB.
  auto accumulate = [&](auto vb) __attribute__((always_inline)) {
    constexpr int VB = decltype(vb)::value;
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      half8_t bp[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const half2_t* a0 = pk[st][2 * kp];
        const half2_t* a1 = pk[st][2 * kp + 1];
        bp[st] = half8_t{a0[0][0], a0[0][1], a0[1][0], a0[1][1], a1[0][0], a1[0][1], a1[1][0], a1[1][1]};
      }
#pragma unroll
      for (int dt = 0; dt < G::DT; ++dt) {
        const half_t* p = reinterpret_cast<const half_t*>(sVb[VB] + 2 * (32 * kp * D) + v_rd[dt]);
        const u32x2_t lo = lds_tr(p);
        const u32x2_t hi = lds_tr(p + 16 * D);
        const half8_t a = __builtin_bit_cast(half8_t, u32x4_t{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
        for (int st = 0; st < 2; ++st)
          o[st][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bp[st], o[st][dt], 0, 0, 0);
      }
    }
    // order: the two transpose loads of dim tile n + 2 are issued before the
    // two MFMAs of dim tile n (two tiles of loads in flight)
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
    for (int n = 0; n < 2 * G::DT; ++n) {
      if (n + 2 < 2 * G::DT) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
    }
  };

  // Softmax of tile kt's scores into pk: causal mask on diagonal tiles, lazy
  // rescale (the running max moves, and the output is rescaled, only when a
  // lane's scores exceed it by more than 2^kLazyRescale), fp16 weights.
  auto softmax = [&](int kt) __attribute__((always_inline)) {
    const int key0 = kt * kBk;
    if (key0 + kBk - 1 > P + wq_first) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int lim = P + qrow[st];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (key0 + 16 * ks + 4 * g + i > lim) sacc[st][ks][i] = -INFINITY;
      }
    }
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      float mt = max4(sacc[st][0]);
#pragma unroll
      for (int ks = 1; ks < 4; ++ks) mt = maxf(mt, max4(sacc[st][ks]));
      const float grow = (mt - m[st]) * c;
      if (__ballot(grow > kLazyRescale) != 0) {
        mt = maxf(mt, __shfl_xor(mt, 16, 64));
        mt = maxf(mt, __shfl_xor(mt, 32, 64));
        const float m_new = maxf(m[st], mt);
        const float corr = (m[st] == -INFINITY) ? 0.f : fast_exp2((m[st] - m_new) * c);
        l[st] *= corr;
#pragma unroll
        for (int dt = 0; dt < G::DT; ++dt) o[st][dt] *= corr;
        m[st] = m_new;
      }
      const float mc = (m[st] == -INFINITY) ? 0.f : m[st] * c;
      float ps = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float p0 = fast_exp2(fmaf(sacc[st][ks][2 * j], c, -mc));
          const float p1 = fast_exp2(fmaf(sacc[st][ks][2 * j + 1], c, -mc));
          pk[st][ks][j] = half2_t{static_cast<half_t>(p0), static_cast<half_t>(p1)};
          ps = __builtin_amdgcn_fdot2(pk[st][ks][j], kOnes2, ps, false);
        }
      l[st] += ps;
    }
  };

  // Prologue: K of tile 0 into LDS.
  uint64_t bo_v[NI];  // blocks of tile t, for its V copy in step t
  {
    const int ids0 = tile_ids_lanes<BS>(trow, 0, max_blocks, lane);
    wait_loads();
    block_offsets(ids0, bo_v);
  }
  if (ntiles > 0) {
    copy_tile(sK0, kc, bo_v, kbo);
    wait_loads();
  }
  int ids_k = tile_ids_lanes<BS>(trow, 1, max_blocks, lane);  // tile t + 1, for K
  __syncthreads();

  // Step t = phases 2 t and 2 t + 1 (PAR = t % 2): tile t's K is in K buffer
  // PAR, tile t - 1's V in V buffer 1 - PAR.  Each set runs its own copy of
  // the loop (SET is a compile-time constant), with the same barriers.
  auto step = [&](auto setc, auto par, int t) __attribute__((always_inline)) {
    constexpr int SET = decltype(setc)::value;
    constexpr int PAR = decltype(par)::value;
    using CP = std::integral_constant<int, PAR>;
    using CQ = std::integral_constant<int, 1 - PAR>;
    // copies for the next step: K of tile t + 1, V of tile t
    uint64_t bo_k[NI];
    block_offsets(ids_k, bo_k);
    copy_tile(PAR ? sK0 : sK1, kc, bo_k, kbo);
    copy_tile(PAR ? sV1 : sV0, vc, bo_v, vbo);
#pragma unroll
    for (int i = 0; i < NI; ++i) bo_v[i] = bo_k[i];
    ids_k = tile_ids_lanes<BS>(trow, t + 2, max_blocks, lane);
    // the matrix phase of a set: P.V of tile t - 1, then the scores of tile t
    auto matrix = [&]() __attribute__((always_inline)) {
      if (t >= 1 && t - 1 < wtiles) accumulate(CQ{});
      if (t < wtiles) scores(CP{});
    };
    if constexpr (SET == 0) {
      matrix();
    } else {
      if (t >= 1 && t - 1 < wtiles) softmax(t - 1);
    }
    // keeps the sets in step; orders no memory (nothing a wave reads in this
    // step is written in it), so the copies issued above stay in flight
    __builtin_amdgcn_s_barrier();
    if constexpr (SET == 0) {
      if (t < wtiles) softmax(t);
    } else {
      matrix();
    }
    wait_loads();
    if (t < ntiles && (t + 1) * kBk > n_keys) {
      __syncthreads();  // every wave's copy of V tile t has landed before its tail is cleared
      zero_rows<D>(PAR ? sV1 : sV0, n_keys - t * kBk, tid);
    }
    __syncthreads();
  };
  auto run = [&](auto setc) __attribute__((always_inline)) {
    for (int t = 0; t <= ntiles; t += 2) {
      step(setc, std::integral_constant<int, 0>{}, t);
      if (t + 1 <= ntiles) step(setc, std::integral_constant<int, 1>{}, t + 1);
    }
  };
  if (set == 0) run(std::integral_constant<int, 0>{});
  else run(std::integral_constant<int, 1>{});

#pragma unroll
  for (int st = 0; st < 2; ++st) {
    float lt = l[st];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    if (!qvalid[st]) continue;
    const float inv = 1.0f / lt;
    float* orow = out + (static_cast<int64_t>(row0 + qrow[st]) * Hq + h) * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < G::DT; ++dt) *reinterpret_cast<float4_t*>(orow + dt * 16) = o[st][dt] * inv;
  }
}

template <int D, int BS>
__global__ __launch_bounds__(kQThreads) void prefill_pp_kernel(
    const half_t* __restrict__ q, const half_t* __restrict__ kc, const half_t* __restrict__ vc,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ prior,
    const int32_t* __restrict__ tables, float* __restrict__ out, int32_t B, int32_t Hq,
    int32_t Hkv, int32_t total_q, int32_t max_blocks, int32_t num_blocks, int32_t nqt, float qk_scale) {
  prefill_pp_body<D, BS>(blockIdx.x, q, kc, vc, cu_q, prior, tables, out, B, Hq, Hkv, total_q,
                         max_blocks, num_blocks, nqt, qk_scale);
}

}  // namespace
}  // namespace pa
