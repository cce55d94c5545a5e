// Chunked-prefill attention over the paged KV cache for gfx950.
//
// [p1] "vLLM PagedAttention Deep Dive", sections "Chunked Prefill" and
// "Mechanics of Chunked Prefill": a long prompt is processed in chunks; each
// chunk's K/V is accumulated in paged blocks, and each chunk query attends to
// the whole cached context before the chunk plus the chunk tokens up to its own
// position.  Prefill is the compute-heavy phase ([p1], "Chunked Prefill"), and
// here Q.K^T and P.V really are dense tiles, so they run on the matrix cores
// (v_mfma_f32_16x16x32_f16).
//
// Two workgroup shapes share the tile arithmetic below.  e4m3 caches (and the
// prefill half of the mixed prefill + decode launch) use a four-wave body of
// 128 query rows (prefill_impl.hpp); fp16 caches use an eight-wave workgroup of
// 256 rows (prefill_pp_impl.hpp) whose two four-wave halves take turns on the
// matrix cores, so that on every SIMD one wave runs MFMAs while the other runs
// the softmax's exponentials.
//
// Tiling.  A wave owns 32 query rows (two 16-row sub-tiles) of one (sequence,
// head).  Keys are walked in tiles of 64 (8, 4, 2 or 1 blocks of 8, 16, 32 or
// 64 tokens looked up in the block table), staged through LDS.
// Each wave computes S^T = K Q^T (so a lane ends up holding the scores of one
// query row, which makes the row max / sum and the output rescale lane-local up
// to two cross-lane steps) and then O^T = V^T P^T with P taken straight from the
// S^T registers: the 32-key contraction of one MFMA is permuted so that lane
// group g's 8 slots are keys {4g..4g+3} and {16+4g..16+4g+3} of a 32-key pair,
// exactly the scores that lane already holds; the V^T operand is read in that
// key order.  Online softmax in the log2 domain with fp32 statistics; the running
// max is only moved (and the output rescaled) when some lane's scores exceed it
// by more than 2^8, so P <= 2^8 stays well inside fp16.  Each lane tests its
// own 16 scores; the cross-lane row max is formed only on the (rare) rescale.
// P is rounded to fp16 for the MFMA, fp32 accumulation.  The causal mask is
// applied only on tiles that cross the diagonal.
//
// Staging, four-wave body.  The K/V tiles are double-buffered in LDS: the
// global loads of tile t+1 are issued into registers before tile t is computed
// and written to the other buffer after it, so one barrier per tile separates
// the phases.  The block ids of tile t+1 come from a vector load issued one tile
// earlier, so no scalar-cache wait sits at the top of the loop; every load of a
// wave falls in one block, so each address is a block base plus a per-thread
// constant.  V is transposed in registers: a thread loads the 8 keys of one V^T
// granule x 4 columns (8-byte loads) and writes 4 granules of 16 bytes.
// Neither buffer is padded: 16-byte chunks are XOR-swizzled by row (K: chunk ^
// (row & 15) for head_dim 128; V^T: granule ^ ((row ^ row >> 2) & 7)), layouts
// that measure free of LDS bank conflicts for both the staging stores and the
// MFMA operand reads on gfx950.
//
// Staging, eight-wave kernel.  K and V go from the cache straight into LDS
// (global_load_lds, 16 bytes a lane, no register round trip), both row-major
// with swizzled 16-byte chunks; the V^T operand is formed at read time by the
// gfx950 transpose load (ds_read_b64_tr_b16).  K of tile t+1 and V of tile t
// are in flight while tile t is computed, and a barrier pair per tile separates
// the two halves' phases.
//
// Order.  Workgroups are dispatched longest sequence first (prior + chunk;
// every workgroup ranks the <= 64 sequences itself), and the query tiles of one
// (sequence, head) are given workgroup ids 8 apart, which the dispatcher sends
// to the same XCD: they read the same K/V tiles at about the same time and
// share that XCD's L2.
#include "prefill_pp_impl.hpp"

namespace pa {
namespace {
using namespace dev;
}  // namespace

template <int D, int BS, bool FP8>
void run_prefill(const KvDesc& c, const void* q, int32_t Hq, int32_t total_q, const int32_t* cu_q,
                 const int32_t* prior, const int32_t* tables, int32_t B, int32_t max_blocks,
                 int32_t max_chunk, float scale, float* out, hipStream_t s) {
  const int64_t pairs = static_cast<int64_t>(B) * Hq;
  const int64_t pairs8 = (pairs + kXcds - 1) / kXcds * kXcds;
  const float qk_scale = scale * kLog2e * (FP8 ? c.k_scale : 1.0f);
  if constexpr (FP8) {
    const int32_t nqt = (max_chunk + kBq - 1) / kBq;
    prefill_kernel<D, BS, true><<<dim3(static_cast<uint32_t>(pairs8 * nqt)), dim3(kThreads), 0, s>>>(
        static_cast<const half_t*>(q), static_cast<const uint8_t*>(c.k), static_cast<const uint8_t*>(c.v),
        cu_q, prior, tables, out, B, Hq, c.num_kv_heads, total_q, max_blocks, c.num_blocks, nqt, qk_scale,
        c.v_scale);
  } else {
    const int32_t nqt = (max_chunk + kQRows - 1) / kQRows;
    prefill_pp_kernel<D, BS><<<dim3(static_cast<uint32_t>(pairs8 * nqt)), dim3(kQThreads), 0, s>>>(
        static_cast<const half_t*>(q), static_cast<const half_t*>(c.k), static_cast<const half_t*>(c.v),
        cu_q, prior, tables, out, B, Hq, c.num_kv_heads, total_q, max_blocks, c.num_blocks, nqt, qk_scale);
  }
}

template <int BS>
hipError_t launch_prefill_bs(const KvDesc& c, const void* q, int32_t Hq, int32_t total_q,
                             const int32_t* cu_q, const int32_t* prior, const int32_t* tables,
                             int32_t B, int32_t max_blocks, int32_t max_chunk, float scale,
                             float* out, hipStream_t s) {
#define PA_ARGS c, q, Hq, total_q, cu_q, prior, tables, B, max_blocks, max_chunk, scale, out, s
  if (c.head_dim == 128) {
    if (c.fp8) run_prefill<128, BS, true>(PA_ARGS);
    else run_prefill<128, BS, false>(PA_ARGS);
  } else {
    if (c.fp8) run_prefill<64, BS, true>(PA_ARGS);
    else run_prefill<64, BS, false>(PA_ARGS);
  }
#undef PA_ARGS
  return hipGetLastError();
}

hipError_t launch_prefill(const KvDesc& c, const void* q, int32_t Hq, int32_t total_q,
                          const int32_t* cu_q, const int32_t* prior, const int32_t* tables,
                          int32_t B, int32_t max_blocks, int32_t max_chunk, float scale, float* out,
                          hipStream_t s) {
  if (B <= 0 || max_chunk <= 0 || total_q <= 0) return hipSuccess;
  switch (c.block_size) {
    case 8:
      return launch_prefill_bs<8>(c, q, Hq, total_q, cu_q, prior, tables, B, max_blocks, max_chunk,
                                  scale, out, s);
    case 32:
      return launch_prefill_bs<32>(c, q, Hq, total_q, cu_q, prior, tables, B, max_blocks, max_chunk,
                                   scale, out, s);
    case 64:
      return launch_prefill_bs<64>(c, q, Hq, total_q, cu_q, prior, tables, B, max_blocks, max_chunk,
                                   scale, out, s);
    default:
      return launch_prefill_bs<16>(c, q, Hq, total_q, cu_q, prior, tables, B, max_blocks, max_chunk,
                                   scale, out, s);
  }
}

}  // namespace pa
