// Paged decode attention for gfx950: one query per (sequence, head) over a KV
// cache scattered across physical blocks of 8, 16, 32 or 64 tokens found
// through a block table
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
// * Coalesced tiles.  One (block, head) tile is block_size x head_dim contiguous
//   values, streamed in units of up to 16 token rows (a 32- or 64-token tile
//   is 2 or 4 contiguous units of the same block), each at least 1 KiB.
//   Load instruction i of a wave reads bytes [1024 i, 1024 i + 1024) of a unit,
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
#include <mutex>

#include "decode_impl.hpp"

// Partials of the split path for pa_decode_noalloc, which takes no workspace
// from its caller: one array of kDecodeScratchBytes per GPU the library runs
// on, held until the process ends.  Every launch on a GPU shares that GPU's
// copy, so calls that overlap on one GPU race.  Nothing in it has to start at
// zero: the merge reads only the partials the same call's split kernel wrote.
static constexpr size_t kDecodeScratchBytes = PA_DECODE_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace pa {
namespace {

constexpr int kMaxScratchDevices = 64;

using namespace dev;

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
template <int kSplit, int kUnit>
__device__ __forceinline__ UnitPos longest_first_unit(int f, const int32_t* __restrict__ lens,
                                                      int B, int ctx_cap, int lane) {
  int Lb = 0;
  if (lane < B) Lb = min(max(lens[lane], 0), ctx_cap);
  const int nunit = (Lb + kUnit - 1) / kUnit;
  const int F = nunit / kSplit;     // full splits
  const int psz = nunit % kSplit;   // units in the partly filled split (0: none)
  const bool has_tail = lane < B && (psz != 0 || nunit == 0);
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
//   ctx_cap = min(max_blocks * BS, max_context_len): lengths are clamped to it.
//   ws_o [B][Hq][nsplit][D], ws_ml [B][Hq][nsplit][2] (max, sum), log2 domain.
//   With kAppend, ap carries each sequence's new token (see append_row).
template <int D, bool FP8, int kSplit, int kU, bool kPipe, int kWPG, bool kLongestFirst, int BS,
          bool kAppend>
__global__ __launch_bounds__(kWPG * 64) void decode_split_kernel(
    const half_t* __restrict__ q, const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ cached, float* __restrict__ out, float* __restrict__ ws_o,
    float* __restrict__ ws_ml, int32_t B, int32_t Hq, int32_t Hkv,
    int32_t max_blocks, int32_t ctx_cap, int32_t nsplit, int32_t num_blocks, float qk_scale,
    float v_scale, AppendRows ap) {
  using G = Geom<D, FP8, BS>;
  static_assert(kSplit % kU == 0, "a split is a whole number of steps");
  static_assert(kSplit % G::kSub == 0, "a split is a whole number of blocks");
  constexpr int kSplitBlocks = kSplit / G::kSub;
  constexpr int kTR = (kSplitBlocks + 63) / 64;  // block-id registers per lane
  const int lane = threadIdx.x & 63;
  const int unit = __builtin_amdgcn_readfirstlane(blockIdx.x * kWPG + (threadIdx.x >> 6));
  const int h = unit % Hq;
  int b, split, L;
  if constexpr (kLongestFirst) {
    const UnitPos pos = longest_first_unit<kSplit, G::kUnit>(unit / Hq, lens, B, ctx_cap, lane);
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
  const int u0 = split * kSplit;         // first unit of the split
  const int b0 = split * kSplitBlocks;   // and its block
  const int kvh = h / (Hq / Hkv);
  const int col = lane % G::kLpr;
  const int row = lane / G::kLpr;

  // The split's block ids (entries past the table's end are not read) and q
  // are loaded together, before either is used.
  int tb[kTR];
  load_block_ids<kTR>(tb, tables + static_cast<int64_t>(b) * max_blocks, b0,
                      min(kSplitBlocks, max_blocks - b0), lane);
  QReg<FP8> qr;
  qr.load(q + bh * D + col * G::kEpl);

  L = min(max(L, 0), ctx_cap);
  const int nunit = (L + G::kUnit - 1) / G::kUnit;
  if (u0 >= nunit) {
    if (split == 0) {  // empty context: zero output
      for (int d = lane; d < D; d += 64) out[bh * D + d] = 0.f;
    }
    return;
  }
  const int nb = min(kSplit, nunit - u0);
  const int nsplit_b = (nunit + kSplit - 1) / kSplit;
  // L >= 1 here; the last split holds token L - 1, reads its new row and
  // writes it (once per kv head)
  const bool last_split = kAppend && split == nsplit_b - 1;
  NewRow nr{};
  int new_blk = -1;
  if constexpr (kAppend) {
    if (last_split) {
      nr = load_new_row<D, FP8>(ap, b, kvh, Hkv, col);
      new_blk = block_id_at<kTR>(tb, (L - 1) / BS - b0);
    }
  }
  clamp_block_ids<kTR>(tb, num_blocks);
  Softmax<D, FP8> sm;
  const uint8_t* kb = kc + static_cast<int64_t>(kvh) * G::kTile + lane * 16;
  const uint8_t* vb = vc + static_cast<int64_t>(kvh) * G::kTile + lane * 16;
  const int64_t stride = static_cast<int64_t>(Hkv) * G::kTile;
  if (cached != nullptr && b0 < cached[b])
    stream_blocks<D, FP8, kU, kPipe, kTR, false, BS, kAppend>(qr, tb, nb, u0, L, kb, vb, stride, qk_scale,
                                                              row, sm, nr);
  else
    stream_blocks<D, FP8, kU, kPipe, kTR, true, BS, kAppend>(qr, tb, nb, u0, L, kb, vb, stride, qk_scale,
                                                             row, sm, nr);
  if constexpr (kAppend) {
    if (last_split && h % (Hq / Hkv) == 0)
      store_new_row<D, FP8, BS>(ap, nr, new_blk, kvh, Hkv, L, num_blocks, col, row);
  }
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
                                                            int32_t nsplit, int32_t split_tokens) {
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
  const int np = (L + split_tokens - 1) / split_tokens;
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

int64_t ctx_units_of(int32_t max_ctx, int unit) { return (static_cast<int64_t>(max_ctx) + unit - 1) / unit; }

int32_t ctx_cap_of(int32_t max_blocks, int32_t max_ctx, int bs) {
  return static_cast<int32_t>(std::min<int64_t>(static_cast<int64_t>(max_blocks) * bs, max_ctx));
}

// Splits cover kSplitTokens tokens whatever the block size, so the workspace
// (one partial per split) does not depend on it.
constexpr int kSplitTokens = 512;

// The device-side form of an append request (empty when there is none).
template <bool FP8>
AppendRows append_rows(const KvDesc& c, const DecodeAppend* a) {
  if (a == nullptr) return AppendRows{};
  return AppendRows{static_cast<const half_t*>(a->k_new), static_cast<const half_t*>(a->v_new),
                    static_cast<uint8_t*>(c.k), static_cast<uint8_t*>(c.v),
                    FP8 ? c.k_scale : 1.0f, FP8 ? c.v_scale : 1.0f};
}

template <int D, bool FP8, int kSplit, int kU, bool kPipe, int kWPG, bool kLongestFirst, int BS,
          bool kAppend>
hipError_t run_split(const KvDesc& c, const void* q, int32_t Hq, const int32_t* tables,
                     const int32_t* lens, const int32_t* cached, int32_t B, int32_t max_blocks,
                     int32_t max_ctx, float scale, float* out, void* workspace, hipStream_t s,
                     const DecodeAppend* append) {
  static_assert(kSplit * Geom<D, FP8, BS>::kUnit == kSplitTokens, "a split is kSplitTokens tokens");
  const int64_t nsplit64 = (ctx_units_of(max_ctx, Geom<D, FP8, BS>::kUnit) + kSplit - 1) / kSplit;
  const int32_t nsplit = static_cast<int32_t>(nsplit64);
  const int64_t units = nsplit64 * B * Hq;
  const int32_t ctx_cap = ctx_cap_of(max_blocks, max_ctx, BS);
  float* ws_o = static_cast<float*>(workspace);
  float* ws_ml = ws_o + static_cast<size_t>(B) * Hq * nsplit * D;
  const float qk_scale = scale * kLog2e * (FP8 ? c.k_scale : 1.0f);
  const float v_scale = FP8 ? c.v_scale : 1.0f;
  const uint32_t groups = static_cast<uint32_t>((units + kWPG - 1) / kWPG);
  decode_split_kernel<D, FP8, kSplit, kU, kPipe, kWPG, kLongestFirst, BS, kAppend>
      <<<dim3(groups), dim3(kWPG * 64), 0, s>>>(
          static_cast<const half_t*>(q), static_cast<const uint8_t*>(c.k),
          static_cast<const uint8_t*>(c.v), tables, lens, cached, out, ws_o, ws_ml, B, Hq,
          c.num_kv_heads, max_blocks, ctx_cap, nsplit, c.num_blocks, qk_scale, v_scale,
          append_rows<FP8>(c, append));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nsplit > 1) {
    const uint32_t rgroups = static_cast<uint32_t>((static_cast<int64_t>(B) * Hq + 3) / 4);
    decode_reduce_kernel<D, 8><<<dim3(rgroups), dim3(256), 0, s>>>(ws_o, ws_ml, lens, out, B, Hq,
                                                                   ctx_cap, nsplit, kSplitTokens);
    e = hipGetLastError();
  }
  return e;
}

template <int D, bool FP8, int kU, bool kPipe, int kW, int kTR, int BS, bool kAppend>
hipError_t run_seq(const KvDesc& c, const void* q, int32_t Hq, const int32_t* tables,
                   const int32_t* lens, const int32_t* cached, int32_t B, int32_t max_blocks,
                   int32_t max_ctx, float scale, float* out, hipStream_t s, const DecodeAppend* append) {
  const float qk_scale = scale * kLog2e * (FP8 ? c.k_scale : 1.0f);
  const float v_scale = FP8 ? c.v_scale : 1.0f;
  decode_seq_kernel<D, FP8, kU, kPipe, kW, kTR, BS, kAppend>
      <<<dim3(static_cast<uint32_t>(static_cast<int64_t>(B) * Hq)), dim3(kW * 64), 0, s>>>(
          static_cast<const half_t*>(q), static_cast<const uint8_t*>(c.k),
          static_cast<const uint8_t*>(c.v), tables, lens, cached, out, B, Hq, c.num_kv_heads,
          max_blocks, ctx_cap_of(max_blocks, max_ctx, BS), c.num_blocks, qk_scale, v_scale,
          append_rows<FP8>(c, append));
  return hipGetLastError();
}

// Launch configurations.  Split path: blocks per step, pipelined, waves per
// workgroup (a split is kSplitTokens tokens).  Per-sequence path: blocks per
// step, pipelined, waves per workgroup (4, or 8 for batches too small to fill
// the chip with 4), block-id registers per wave (a wave takes at most
// 64 * kSeqTR blocks).
constexpr int kUF16 = 2, kWpgF16 = 2;
constexpr bool kPipeF16 = true;
constexpr int kUF8 = 4, kWpgF8 = 1;
constexpr bool kPipeF8 = false;
constexpr int kSeqUF16 = 2, kSeqUF8 = 1;
constexpr bool kSeqPipeF16 = false, kSeqPipeF8 = false;
constexpr int kSeqTR = 1;
// The per-sequence path is taken when the batch alone fills the chip, at least
// kSeqMinWaves waves (about three per wave slot of the 256 CUs at these
// kernels' occupancy), and no wave holds more than 64 * kSeqTR blocks.
constexpr int64_t kSeqMinWaves = 8192;

// Waves per workgroup of the per-sequence path for this batch, or 0 for the
// split path (units of `unit` tokens, `sub` units a block).
int seq_waves(int32_t B, int32_t Hq, int32_t max_ctx, int unit, int sub) {
  const int64_t pairs = static_cast<int64_t>(B) * Hq;
  const int64_t units = ctx_units_of(max_ctx, unit);
  for (int w : {4, 8}) {
    if (pairs * w >= kSeqMinWaves && run_blocks((units + w - 1) / w, sub) <= 64 * kSeqTR) return w;
  }
  return 0;
}

// A streamed unit must cover at least one 1 KiB wave load.
template <int D, bool FP8, int BS>
constexpr bool kTileFits = (BS < 16 ? BS : 16) * D * (FP8 ? 1 : 2) >= 1024;

template <int D, bool FP8, int BS, bool kAppend>
hipError_t launch_decode_typed(const KvDesc& c, const void* q, int32_t Hq, const int32_t* tables,
                               const int32_t* lens, const int32_t* cached, int32_t B,
                               int32_t max_blocks, int32_t max_ctx, float scale, float* out,
                               void* workspace, hipStream_t s, const DecodeAppend* append) {
  if constexpr (!kTileFits<D, FP8, BS>) {
    return hipErrorInvalidValue;  // rejected by the caller's argument checks
  } else {
    constexpr int kU = FP8 ? kSeqUF8 : kSeqUF16;
    constexpr bool kPipe = FP8 ? kSeqPipeF8 : kSeqPipeF16;
    using G = Geom<D, FP8, BS>;
    const int sw = seq_waves(B, Hq, max_ctx, G::kUnit, G::kSub);
    if (sw == 4)
      return run_seq<D, FP8, kU, kPipe, 4, kSeqTR, BS, kAppend>(c, q, Hq, tables, lens, cached, B,
                                                                max_blocks, max_ctx, scale, out, s, append);
    if (sw == 8)
      return run_seq<D, FP8, kU, kPipe, 8, kSeqTR, BS, kAppend>(c, q, Hq, tables, lens, cached, B,
                                                                max_blocks, max_ctx, scale, out, s, append);
    constexpr int kSplit = kSplitTokens / G::kUnit;  // units per split
    constexpr int kSU = FP8 ? kUF8 : kUF16;
    constexpr bool kSPipe = FP8 ? kPipeF8 : kPipeF16;
    constexpr int kWpg = FP8 ? kWpgF8 : kWpgF16;
    // longest-first unit order needs every length in one wave: B <= 64
    if (B <= 64)
      return run_split<D, FP8, kSplit, kSU, kSPipe, kWpg, true, BS, kAppend>(
          c, q, Hq, tables, lens, cached, B, max_blocks, max_ctx, scale, out, workspace, s, append);
    return run_split<D, FP8, kSplit, kSU, kSPipe, kWpg, false, BS, kAppend>(
        c, q, Hq, tables, lens, cached, B, max_blocks, max_ctx, scale, out, workspace, s, append);
  }
}

template <int BS, bool kAppend>
hipError_t launch_decode_head(const KvDesc& c, const void* q, int32_t Hq, const int32_t* tables,
                              const int32_t* lens, const int32_t* cached, int32_t B,
                              int32_t max_blocks, int32_t max_ctx, float scale, float* out,
                              void* workspace, hipStream_t s, const DecodeAppend* append) {
#define PA_ARGS c, q, Hq, tables, lens, cached, B, max_blocks, max_ctx, scale, out, workspace, s, append
  if (c.head_dim == 128)
    return c.fp8 ? launch_decode_typed<128, true, BS, kAppend>(PA_ARGS)
                 : launch_decode_typed<128, false, BS, kAppend>(PA_ARGS);
  return c.fp8 ? launch_decode_typed<64, true, BS, kAppend>(PA_ARGS)
               : launch_decode_typed<64, false, BS, kAppend>(PA_ARGS);
#undef PA_ARGS
}

template <int BS>
hipError_t launch_decode_bs(const KvDesc& c, const void* q, int32_t Hq, const int32_t* tables,
                            const int32_t* lens, const int32_t* cached, int32_t B,
                            int32_t max_blocks, int32_t max_ctx, float scale, float* out,
                            void* workspace, hipStream_t s, const DecodeAppend* append) {
  if (append != nullptr)
    return launch_decode_head<BS, true>(c, q, Hq, tables, lens, cached, B, max_blocks, max_ctx, scale,
                                        out, workspace, s, append);
  return launch_decode_head<BS, false>(c, q, Hq, tables, lens, cached, B, max_blocks, max_ctx, scale,
                                       out, workspace, s, append);
}

}  // namespace

int32_t decode_partition_tokens() { return kSplitTokens; }

size_t decode_scratch_capacity() { return kDecodeScratchBytes; }

hipError_t decode_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  static std::mutex mu;
  static void* addr[kMaxScratchDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    // with dev current: the address of this GPU's copy of the array (the name
    // itself is a host-side stand-in and must never reach a kernel)
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

size_t decode_workspace_bytes(int32_t B, int32_t Hq, int32_t D, int32_t max_context_len) {
  if (B <= 0 || Hq <= 0 || D <= 0 || max_context_len <= 0) return 0;
  const int64_t nsplit = (static_cast<int64_t>(max_context_len) + kSplitTokens - 1) / kSplitTokens;
  return static_cast<size_t>(B) * Hq * nsplit * (D + 2) * sizeof(float);
}

int64_t decode_units(int32_t B, int32_t Hq, int32_t max_context_len) {
  const int64_t nsplit = (static_cast<int64_t>(max_context_len) + kSplitTokens - 1) / kSplitTokens;
  return nsplit * B * Hq;
}

hipError_t launch_decode(const KvDesc& c, const void* q, int32_t Hq, const int32_t* tables,
                         const int32_t* lens, const int32_t* cached, int32_t B, int32_t max_blocks,
                         int32_t max_ctx, float scale, float* out, void* workspace, hipStream_t s,
                         const DecodeAppend* append) {
  if (B == 0) return hipSuccess;
  if (max_ctx <= 0) {
    // every length is 0: zero output
    const int64_t n = static_cast<int64_t>(B) * Hq * c.head_dim;
    zero_kernel<<<dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, s>>>(out, n);
    return hipGetLastError();
  }
  switch (c.block_size) {
    case 8:
      return launch_decode_bs<8>(c, q, Hq, tables, lens, cached, B, max_blocks, max_ctx, scale, out,
                                 workspace, s, append);
    case 32:
      return launch_decode_bs<32>(c, q, Hq, tables, lens, cached, B, max_blocks, max_ctx, scale, out,
                                  workspace, s, append);
    case 64:
      return launch_decode_bs<64>(c, q, Hq, tables, lens, cached, B, max_blocks, max_ctx, scale, out,
                                  workspace, s, append);
    default:
      return launch_decode_bs<16>(c, q, Hq, tables, lens, cached, B, max_blocks, max_ctx, scale, out,
                                  workspace, s, append);
  }
}

}  // namespace pa
