// Device code of the chunked prefill shared by prefill.hip (its launch) and
// mixed.hip (prefill workgroups inside the mixed prefill + decode launch).
// The design notes are at the top of prefill.hip.
#pragma once
#include <cmath>
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace pa {
namespace {

using namespace dev;

constexpr int kBq = 128;       // query rows per workgroup
constexpr int kBk = 64;        // keys per tile
constexpr int kThreads = 256;
constexpr int kXcds = 8;       // workgroup ids are dealt round robin over 8 XCDs
constexpr float kLazyRescale = 8.0f;  // log2 growth of a row max that forces a rescale

template <int D>
struct PGeom {
  // K is stored row-major without padding; the 16-byte chunk c of key row r
  // sits at chunk c ^ kswz(r).  V^T rows (one per head-dim column) hold the
  // tile's 64 keys as 8 granules of 8 keys: granule 4 p + g of a row holds
  // keys 32 p + 16 hb + 4 g + i (hb < 2, i < 4) at slot 4 hb + i, which is
  // exactly the 8 keys lane group g feeds to one P.V MFMA; granule q of row r
  // sits at q ^ vswz(r).  Both swizzles keep the MFMA operand reads and the
  // staging stores free of bank conflicts.
  static constexpr int DK = D / 32;         // MFMA steps over head_dim for S
  static constexpr int DT = D / 16;         // 16-wide output tiles over head_dim
  static constexpr int CPR = D / 8;         // 16-byte chunks per K row
  static constexpr int KLOADS = kBk * CPR / kThreads;  // K chunks per thread
  static constexpr int VTHREADS = 8 * (D / 4);         // threads staging V: granule x column quad
  static constexpr int KBUF = kBk * D;      // halfs per K buffer
  static constexpr int VBUF = D * kBk;      // halfs per V^T buffer
  static_assert(kBk * CPR % kThreads == 0, "K tile must split evenly");
  static_assert(16 * CPR % 64 == 0, "a wave's K chunks must stay in one block");
  static_assert(VTHREADS <= kThreads && VTHREADS % 64 == 0, "V staging must fill whole waves");
};

__device__ __forceinline__ int swz8(int r) { return (r ^ (r >> 2)) & 7; }

constexpr half2_t kOnes2 = {static_cast<half_t>(1.0f), static_cast<half_t>(1.0f)};

__device__ __forceinline__ float maxf(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max4(float4_t v) { return maxf(maxf(v[0], v[1]), maxf(v[2], v[3])); }

template <int D>
__device__ __forceinline__ int kswz(int r) {
  if constexpr (D == 128) return r & 15;
  else return swz8(r);
}

// Cache element: fp16, or an e4m3 code (widened to fp16 on the way to LDS).
template <bool FP8>
using elem_t = std::conditional_t<FP8, uint8_t, half_t>;

// Registers holding one K/V tile between its global loads and its LDS stores,
// in the cache's format: per K chunk 8 values, per V row quad 4 values.
template <int D, bool FP8>
struct Stage {
  using KReg = std::conditional_t<FP8, u32x2_t, u32x4_t>;
  using VReg = std::conditional_t<FP8, uint32_t, u32x2_t>;
  KReg k[PGeom<D>::KLOADS];
  VReg v[8];   // keys 4 g + i of block 2 p (v[i]) and of block 2 p + 1 (v[4 + i])
};

// 8 K values (one 16-byte LDS chunk) and 4 V values as fp16.  Every e4m3
// value is exact in fp16; the scales are applied to the scores and the output.
__device__ __forceinline__ u32x4_t widen_k(const u32x4_t& k) { return k; }
__device__ __forceinline__ u32x4_t widen_k(const u32x2_t& k) {
  return u32x4_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k[0], 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k[0], 1.0f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k[1], 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k[1], 1.0f, true))};
}
__device__ __forceinline__ u32x2_t widen_v(const u32x2_t& v) { return v; }
__device__ __forceinline__ u32x2_t widen_v(uint32_t v) {
  return u32x2_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, true))};
}

// Rank of lane b's sequence (b < B <= 64) by total length, longest first,
// ties by index; lanes >= B get rank 64.
__device__ __forceinline__ int work_rank(int Wb, int lane, int B) {
  int rank = 0;
  for (int k = 0; k < B; ++k) {
    const int Wk = __builtin_amdgcn_readlane(Wb, k);
    rank += (Wk > Wb || (Wk == Wb && k < lane)) ? 1 : 0;
  }
  return lane < B ? rank : 64;
}

// The block ids of a key tile (kBk / BS of them, at most 8; wave-uniform;
// ids past the table's end, or outside the pool, read as block 0), as scalars.
struct TileBlocks {
  int p0, p1, p2, p3, p4, p5, p6, p7;
};

// Block j (0..7) of a tile.  A free function on values: as a member reading
// this->pN the selects are folded into one indexed load and the struct is
// left in memory.
__device__ __forceinline__ int pick_block(int j, const TileBlocks& t) {
  const int a = (j & 1) ? t.p1 : t.p0, b = (j & 1) ? t.p3 : t.p2;
  const int c = (j & 1) ? t.p5 : t.p4, d = (j & 1) ? t.p7 : t.p6;
  const int lo = (j & 2) ? b : a, hi = (j & 2) ? d : c;
  return (j & 4) ? hi : lo;
}

__device__ __forceinline__ int table_id(const int32_t* __restrict__ trow, int idx, int max_blocks,
                                        int num_blocks) {
  int v = idx < max_blocks ? trow[idx] : 0;
  v = __builtin_amdgcn_readfirstlane(v);
  return (static_cast<uint32_t>(v) < static_cast<uint32_t>(num_blocks)) ? v : 0;
}

// Lanes 0 .. kBk/BS - 1 load the table entries of tile kt (a vector load,
// waited on in order with the tile loads, one tile ahead of use).
template <int BS>
__device__ __forceinline__ int tile_ids_lanes(const int32_t* __restrict__ trow, int kt, int max_blocks,
                                              int lane) {
  const int j = kt * (kBk / BS) + lane;
  return (lane < kBk / BS && j < max_blocks) ? trow[j] : 0;
}

__device__ __forceinline__ int clamp_id(int v, int num_blocks) {
  return (static_cast<uint32_t>(v) < static_cast<uint32_t>(num_blocks)) ? v : 0;
}

template <int BS>
__device__ __forceinline__ TileBlocks tile_blocks_from(int ids, int num_blocks) {
  constexpr int n = kBk / BS;
  auto at = [&](int j) { return j < n ? clamp_id(__builtin_amdgcn_readlane(ids, j), num_blocks) : 0; };
  return TileBlocks{at(0), at(1), at(2), at(3), at(4), at(5), at(6), at(7)};
}

template <int BS>
__device__ __forceinline__ TileBlocks tile_blocks(const int32_t* __restrict__ trow, int kt,
                                                  int max_blocks, int num_blocks) {
  constexpr int n = kBk / BS;
  const int j0 = kt * n;
  auto at = [&](int j) { return j < n ? table_id(trow, j0 + j, max_blocks, num_blocks) : 0; };
  return TileBlocks{at(0), at(1), at(2), at(3), at(4), at(5), at(6), at(7)};
}

// Per-thread staging geometry for BS-token blocks.  K load i of thread t is
// 16-byte chunk i * 256 + t of the tile: key (i * 256 + t) / CPR; the 64 / CPR
// keys a wave loads per instruction are consecutive and aligned, so they lie
// in one block (wave-uniform base).  V: thread (w, lane < D/2) stages granule
// q = 2 w + lane / (D/4) (pair p = q / 4, group g = q % 4) for columns
// 4 dq .. 4 dq + 3, dq = lane % (D/4): keys 32 p + 16 hb + 4 g + i (hb < 2,
// i < 4), rows of block (32 p + 16 hb + 4 g) / BS -- the same block for the
// whole wave at each hb, for every block size 8, 16, 32 and 64.
template <int D, int BS>
struct StageGeom {
  int k_row;    // the chunk's key within the tile, for i = 0 (adds 256 i / CPR)
  int k_col;    // its chunk index
  int k_head;   // halfs from a block's base to this kv head's rows
  bool v_on;    // thread stages V
  int vq, dq;   // granule (0..7) and column quad
  int v_off[2]; // halfs from a block's base to the thread's first V row, per hb

  __device__ void init(int tid, int kvh) {
    using G = PGeom<D>;
    const int w = tid >> 6, lane = tid & 63;
    k_row = tid / G::CPR;
    k_col = tid % G::CPR;
    k_head = kvh * BS * D;
    v_on = lane < D / 2;
    vq = (2 * w + lane / (D / 4)) & 7;
    dq = lane % (D / 4);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
      v_off[hb] = (kvh * BS + (32 * (vq >> 2) + 16 * hb + 4 * (vq & 3)) % BS) * D + 4 * dq;
  }
};

// Issue the global loads of a key tile.  Every load stays inside the pool;
// rows past the context are fixed up by store_tile.
template <int D, int BS, bool FP8>
__device__ __forceinline__ void load_tile(Stage<D, FP8>& st, const StageGeom<D, BS>& sg,
                                          const TileBlocks& tb, const elem_t<FP8>* __restrict__ kc,
                                          const elem_t<FP8>* __restrict__ vc, int64_t blk_stride,
                                          int w) {
  using G = PGeom<D>;
  using KReg = typename Stage<D, FP8>::KReg;
  using VReg = typename Stage<D, FP8>::VReg;
#pragma unroll
  for (int i = 0; i < G::KLOADS; ++i) {
    const int key = sg.k_row + i * (kThreads / G::CPR);
    const int blk = ((i * kThreads + 64 * w) / G::CPR) / BS;  // wave-uniform
    const elem_t<FP8>* base = kc + static_cast<int64_t>(pick_block(blk, tb)) * blk_stride;
    st.k[i] = *reinterpret_cast<const KReg*>(base + sg.k_head + (key % BS) * D + sg.k_col * 8);
  }
  if (sg.v_on) {
    // pair p = w / 2 and group pair g / 2 = w % 2 are wave-uniform
    const int kb = 32 * (w >> 1) + 8 * (w & 1);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const elem_t<FP8>* base = vc + static_cast<int64_t>(pick_block((kb + 16 * hb) / BS, tb)) * blk_stride;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st.v[4 * hb + i] = *reinterpret_cast<const VReg*>(base + sg.v_off[hb] + i * D);
    }
  }
}

// Write a staged tile to one LDS buffer: K row-major, V transposed.  On the
// tile holding the end of the keys (tail), V rows at or past n_keys are zeroed
// (their P is 0, but stale cache rows may hold non-finite bits); K rows there
// only produce scores that the causal mask removes.
template <int D, int BS, bool FP8>
__device__ __forceinline__ void store_tile(const Stage<D, FP8>& st, const StageGeom<D, BS>& sg,
                                           half_t* __restrict__ sK, half_t* __restrict__ sVt, bool tail,
                                           int key0, int n_keys) {
  using G = PGeom<D>;
#pragma unroll
  for (int i = 0; i < G::KLOADS; ++i) {
    const int r = sg.k_row + i * (kThreads / G::CPR);
    *reinterpret_cast<u32x4_t*>(&sK[r * D + ((sg.k_col ^ kswz<D>(r)) << 3)]) = widen_k(st.k[i]);
  }
  if (!sg.v_on) return;
  u32x2_t v[8];
#pragma unroll
  for (int s8 = 0; s8 < 8; ++s8) v[s8] = widen_v(st.v[s8]);
  if (tail) {
    const int kb = key0 + 32 * (sg.vq >> 2) + 4 * (sg.vq & 3);
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8)
      if (kb + 16 * (s8 >> 2) + (s8 & 3) >= n_keys) v[s8] = u32x2_t{0u, 0u};
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // column 4 dq + j of the granule's 8 keys, two keys a word: half j & 1 of word j / 2
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
    u32x4_t row;
#pragma unroll
    for (int wd = 0; wd < 4; ++wd)
      row[wd] = __builtin_amdgcn_perm(v[2 * wd + 1][j >> 1], v[2 * wd][j >> 1], sel);
    const int r = 4 * sg.dq + j;
    *reinterpret_cast<u32x4_t*>(&sVt[r * kBk + ((sg.vq ^ swz8(r)) << 3)]) = row;
  }
}

// grid (ceil(B * Hq / 8) * 8 * nqt), block 256.  qk_scale = softmax scale *
// log2 e (* k_scale for an e4m3 cache); v_scale multiplies the output (1 for
// fp16).
template <int D, int BS, bool FP8 = false>
__device__ __forceinline__ void prefill_body(
    int u, const half_t* __restrict__ q, const elem_t<FP8>* __restrict__ kc,
    const elem_t<FP8>* __restrict__ vc, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ prior, const int32_t* __restrict__ tables, float* __restrict__ out,
    int32_t B, int32_t Hq, int32_t Hkv, int32_t total_q, int32_t max_blocks, int32_t num_blocks,
    int32_t nqt, float qk_scale, float v_scale = 1.0f) {
  using G = PGeom<D>;
  __shared__ __attribute__((aligned(16))) half_t sK[2 * G::KBUF];
  __shared__ __attribute__((aligned(16))) half_t sVt[2 * G::VBUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int q0 = qt * kBq;
  if (q0 >= C || row0 < 0) return;
  const int L_total = min(P + C, max_blocks * BS);
  const int kvh = h / (Hq / Hkv);
  const int32_t* trow = tables + static_cast<int64_t>(b) * max_blocks;

  // Scores are kept in raw units and scaled inside the exponent by c > 0; a
  // negative scale flips the sign of q instead (exact).  A zero scale becomes
  // 1e-30, which leaves every exp2 of a finite score at 1 and keeps masked
  // scores at -inf (a zero factor would turn them into NaN).
  const bool neg = qk_scale < 0.f;
  const float c = fmaxf(neg ? -qk_scale : qk_scale, 1e-30f);

  // Q as the B operand of S^T = K Q^T: lane holds q[row = c16][d = 32 kk + 8 g .. +8]
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

  const int wq_first = q0 + 32 * w;                      // first query row of this wave
  const int wq_last = min(q0 + 32 * w + 32, C) - 1;      // last valid one (< first if none)
  const int n_keys = min(P + min(q0 + kBq, C), L_total);  // keys any row of the group needs
  const int ntiles = (n_keys + kBk - 1) / kBk;

  StageGeom<D, BS> sg;
  sg.init(tid, kvh);
  const int64_t blk_stride = static_cast<int64_t>(Hkv) * BS * D;
  Stage<D, FP8> stg;
  int ids_next = 0;
  if (ntiles > 0) {
    load_tile<D, BS, FP8>(stg, sg, tile_blocks<BS>(trow, 0, max_blocks, num_blocks), kc, vc, blk_stride, w);
    ids_next = tile_ids_lanes<BS>(trow, 1, max_blocks, lane);
    store_tile<D, BS>(stg, sg, sK, sVt, kBk > n_keys, 0, n_keys);
  }

  // Per-lane byte offsets of the MFMA operand reads.  The K swizzle of row
  // 16 ks + c16 depends on ks only through its parity, and the V^T swizzle of
  // row 16 dt + c16 on dt only through its parity, so four registers each
  // cover every read; the rest of each address is an immediate.
  int k_rd[G::DK][2], v_rd[2][2];
#pragma unroll
  for (int kk = 0; kk < G::DK; ++kk)
#pragma unroll
    for (int par = 0; par < 2; ++par)
      k_rd[kk][par] = 2 * (c16 * D + (((4 * kk + g) ^ kswz<D>(16 * par + c16)) << 3));
#pragma unroll
  for (int kp = 0; kp < 2; ++kp)
#pragma unroll
    for (int par = 0; par < 2; ++par)
      v_rd[kp][par] = 2 * (c16 * kBk + (((4 * kp + g) ^ swz8(16 * par + c16)) << 3));
  const char* sKb = reinterpret_cast<const char*>(sK);
  const char* sVb = reinterpret_cast<const char*>(sVt);

  // One key tile.  PAR (the LDS buffer holding tile kt) is a compile-time
  // constant: the loop below runs tiles in pairs, so every LDS address is a
  // per-lane register plus an immediate offset.
  auto step = [&](auto par, int kt) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par)::value;
    const int key0 = kt * kBk;
    const bool more = kt + 1 < ntiles;
    if (more) {
      const TileBlocks tb = tile_blocks_from<BS>(ids_next, num_blocks);
      ids_next = tile_ids_lanes<BS>(trow, kt + 2, max_blocks, lane);
      load_tile<D, BS, FP8>(stg, sg, tb, kc, vc, blk_stride, w);
    }
    __syncthreads();  // buffer PAR written; buffer 1 - PAR no longer read

    if (!(wq_last < wq_first || key0 > P + wq_last)) {  // keys of this tile visible to the wave
      // S^T tiles: [st][ks] holds keys key0 + 16 ks + 4 g + i for query row c16
      float4_t sacc[2][4];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) sacc[st][ks] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < G::DK; ++kk) {
        half8_t a[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          a[ks] = *reinterpret_cast<const half8_t*>(sKb + 2 * (PAR * G::KBUF + ks * 16 * D) +
                                                    k_rd[kk][ks & 1]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int st = 0; st < 2; ++st)
            sacc[st][ks] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[ks], qb[st][kk], sacc[st][ks], 0, 0, 0);
      }

      if (key0 + kBk - 1 > P + wq_first) {  // tile crosses the diagonal of some row
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int lim = P + qrow[st];  // last visible key of this lane's row
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (key0 + 16 * ks + 4 * g + i > lim) sacc[st][ks][i] = -INFINITY;
        }
      }

      // P in fp16, two keys a register: pk[st][ks][j] = keys 4 g + 2 j, + 1 of sub-tile ks
      half2_t pk[2][4][2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        // NaN-propagating maximum: gfx950 forms it into three-input max
        // instructions without the quieting step the IEEE maxNum needs
        float mt = max4(sacc[st][0]);
#pragma unroll
        for (int ks = 1; ks < 4; ++ks) mt = maxf(mt, max4(sacc[st][ks]));
        // move the running max (and rescale) only when some lane's scores grew
        // past it by more than 2^kLazyRescale: exp2 arguments stay <=
        // kLazyRescale.  The lane-local max decides; the row max over the 4
        // lane groups is only formed when a rescale happens.
        const float grow = (mt - m[st]) * c;  // +inf on the first visible tile
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
        // the row sum adds the fp16 values the P.V product uses (exact
        // products, fp32 accumulation): one dot2 per two keys
        float ps = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const float p0 = fast_exp2(fmaf(sacc[st][ks][2 * j], c, -mc));
            const float p1 = fast_exp2(fmaf(sacc[st][ks][2 * j + 1], c, -mc));
            pk[st][ks][j] = half2_t{static_cast<half_t>(p0), static_cast<half_t>(p1)};
            ps = __builtin_amdgcn_fdot2(pk[st][ks][j], kOnes2, ps, false);
          }
        }
        l[st] += ps;
      }

      // O^T += V^T P^T over two 32-key pairs of sub-tiles (0,1) and (2,3)
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
          const half8_t a = *reinterpret_cast<const half8_t*>(sVb + 2 * (PAR * G::VBUF + dt * 16 * kBk) +
                                                              v_rd[kp][dt & 1]);
#pragma unroll
          for (int st = 0; st < 2; ++st)
            o[st][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bp[st], o[st][dt], 0, 0, 0);
        }
      }
    }
    if (more)
      store_tile<D, BS>(stg, sg, sK + (1 - PAR) * G::KBUF, sVt + (1 - PAR) * G::VBUF,
                        key0 + 2 * kBk > n_keys, key0 + kBk, n_keys);
  };

  for (int kt = 0; kt < ntiles; kt += 2) {
    step(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 < ntiles) step(std::integral_constant<int, 1>{}, kt + 1);
  }

#pragma unroll
  for (int st = 0; st < 2; ++st) {
    float lt = l[st];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    if (!qvalid[st]) continue;
    const float inv = v_scale / lt;
    float* orow = out + (static_cast<int64_t>(row0 + qrow[st]) * Hq + h) * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < G::DT; ++dt) {
      *reinterpret_cast<float4_t*>(orow + dt * 16) = o[st][dt] * inv;
    }
  }
}


template <int D, int BS, bool FP8>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(
    const half_t* __restrict__ q, const elem_t<FP8>* __restrict__ kc, const elem_t<FP8>* __restrict__ vc,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ prior,
    const int32_t* __restrict__ tables, float* __restrict__ out, int32_t B, int32_t Hq,
    int32_t Hkv, int32_t total_q, int32_t max_blocks, int32_t num_blocks, int32_t nqt,
    float qk_scale, float v_scale) {
  prefill_body<D, BS, FP8>(blockIdx.x, q, kc, vc, cu_q, prior, tables, out, B, Hq, Hkv, total_q,
                           max_blocks, num_blocks, nqt, qk_scale, v_scale);
}

}  // namespace
}  // namespace pa
