// One launch for a whole continuous-batching step: the chunked-prefill
// workgroups of the sequences being admitted and the decode workgroups of the
// running ones ([p1] "Chunked Prefill": prefill chunks are scheduled together
// with decode requests in the same step; [p3] continuous batching section: the
// batch is refilled at every iteration).
//
// The grid holds every prefill workgroup first, then one decode workgroup per
// (sequence, head).  The dispatcher hands out workgroups in id order, so the
// decode workgroups start as soon as prefill workgroups retire: the
// HBM-bound decode fills the CUs that the MFMA-bound prefill leaves idle in its
// tail, instead of running after it.  Both halves are four-wave workgroup
// bodies: prefill_body (the standalone prefill's body for e4m3 caches; for
// fp16 caches the standalone launch uses an eight-wave kernel, equal within
// rounding) and decode_seq_body (the standalone decode's, bit-identical in
// result); the decode half runs at the prefill's occupancy (2 workgroups per CU).
#include "decode_impl.hpp"
#include "prefill_impl.hpp"

namespace pa {
namespace {

using namespace dev;

// per-sequence decode inside the mixed launch: 2 units per step (1 for
// e4m3), not pipelined, 4 waves (the standalone per-sequence configurations)
template <bool FP8>
constexpr int kMixU = FP8 ? 1 : 2;
constexpr int kMixW = 4;
static_assert(kMixW * 64 == kThreads, "decode and prefill workgroups have one shape");

// qk_scale = softmax scale * log2 e (* k_scale for e4m3); v_scale = 1 for fp16.
template <int D, int kTR, int BS, bool FP8>
__global__ __launch_bounds__(kThreads, 2) void mixed_step_kernel(
    const half_t* __restrict__ pq, const elem_t<FP8>* __restrict__ kc,
    const elem_t<FP8>* __restrict__ vc, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ prior, const int32_t* __restrict__ ptables, float* __restrict__ pout,
    int32_t Bp, int32_t Hq, int32_t Hkv, int32_t total_q, int32_t pmax_blocks, int32_t num_blocks,
    int32_t nqt, float qk_scale, float v_scale, int32_t n_prefill_wgs, const half_t* __restrict__ dq,
    const int32_t* __restrict__ dtables, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ cached, float* __restrict__ dout, int32_t Bd, int32_t dmax_blocks,
    int32_t ctx_cap) {
  const int wg = blockIdx.x;
  if (wg < n_prefill_wgs) {
    prefill_body<D, BS, FP8>(wg, pq, kc, vc, cu_q, prior, ptables, pout, Bp, Hq, Hkv, total_q,
                             pmax_blocks, num_blocks, nqt, qk_scale, v_scale);
  } else {
    decode_seq_body<D, FP8, kMixU<FP8>, false, kMixW, kTR, BS>(
        wg - n_prefill_wgs, dq, reinterpret_cast<const uint8_t*>(kc),
        reinterpret_cast<const uint8_t*>(vc), dtables, lens, cached, dout, Bd, Hq, Hkv, dmax_blocks,
        ctx_cap, num_blocks, qk_scale, v_scale);
  }
}

template <int D, int kTR, int BS, bool FP8>
hipError_t run_mixed(const KvDesc& c, int32_t Hq, float scale, const MixedPrefill& p,
                     const MixedDecode& d, hipStream_t s) {
  const int32_t nqt = (p.max_chunk + kBq - 1) / kBq;
  const int64_t pairs = static_cast<int64_t>(p.B) * Hq;
  const int64_t n_prefill = (pairs + kXcds - 1) / kXcds * kXcds * nqt;
  const int64_t n_decode = static_cast<int64_t>(d.B) * Hq;
  const int32_t ctx_cap =
      static_cast<int32_t>(std::min<int64_t>(static_cast<int64_t>(d.max_blocks) * BS, d.max_ctx));
  mixed_step_kernel<D, kTR, BS, FP8><<<dim3(static_cast<uint32_t>(n_prefill + n_decode)), dim3(kThreads), 0, s>>>(
      static_cast<const half_t*>(p.q), static_cast<const elem_t<FP8>*>(c.k),
      static_cast<const elem_t<FP8>*>(c.v), p.cu_q, p.prior, p.tables, p.out, p.B, Hq, c.num_kv_heads,
      p.total_q, p.max_blocks, c.num_blocks, nqt, scale * kLog2e * (FP8 ? c.k_scale : 1.0f),
      FP8 ? c.v_scale : 1.0f, static_cast<int32_t>(n_prefill),
      static_cast<const half_t*>(d.q), d.tables, d.lens, d.cached, d.out, d.B, d.max_blocks, ctx_cap);
  return hipGetLastError();
}

template <int D, int BS, bool FP8>
hipError_t launch_mixed_typed(const KvDesc& c, int32_t Hq, float scale, const MixedPrefill& p,
                              const MixedDecode& d, hipStream_t s, int tr) {
  if constexpr (FP8 && (BS < 16 ? BS : 16) * D < 1024) {
    return hipErrorInvalidValue;  // an e4m3 unit below 1 KiB is refused by the argument checks
  } else {
    if (tr == 1) return run_mixed<D, 1, BS, FP8>(c, Hq, scale, p, d, s);
    if (tr == 2) return run_mixed<D, 2, BS, FP8>(c, Hq, scale, p, d, s);
    return run_mixed<D, 4, BS, FP8>(c, Hq, scale, p, d, s);
  }
}

template <int BS>
hipError_t launch_mixed_bs(const KvDesc& c, int32_t Hq, float scale, const MixedPrefill& p,
                           const MixedDecode& d, hipStream_t s) {
  // blocks per decode wave decide the block-id registers (64 per register)
  using G = Geom<128, false, BS>;
  const int64_t ctx = std::min<int64_t>(static_cast<int64_t>(d.max_blocks) * BS, d.max_ctx);
  const int64_t units = (ctx + G::kUnit - 1) / G::kUnit;
  const int64_t per_wave = run_blocks((units + kMixW - 1) / kMixW, G::kSub);
  const int tr = per_wave <= 64 ? 1 : per_wave <= 128 ? 2 : 4;
  if (c.head_dim == 128) return c.fp8 ? launch_mixed_typed<128, BS, true>(c, Hq, scale, p, d, s, tr)
                                      : launch_mixed_typed<128, BS, false>(c, Hq, scale, p, d, s, tr);
  return c.fp8 ? launch_mixed_typed<64, BS, true>(c, Hq, scale, p, d, s, tr)
               : launch_mixed_typed<64, BS, false>(c, Hq, scale, p, d, s, tr);
}

}  // namespace

// A decode wave holds up to 4 block-id registers of 64 ids each: the longest
// context whose per-wave run of units touches at most 256 blocks.
int32_t mixed_max_context(int32_t block_size) {
  const int unit = block_size < 16 ? block_size : 16;
  const int sub = block_size / unit;
  const int units_per_wave = sub == 1 ? 256 : 255 * sub + 1;
  return kMixW * units_per_wave * unit;
}

hipError_t launch_mixed(const KvDesc& c, int32_t Hq, float scale, const MixedPrefill& p,
                        const MixedDecode& d, hipStream_t s) {
  switch (c.block_size) {
    case 8:
      return launch_mixed_bs<8>(c, Hq, scale, p, d, s);
    case 32:
      return launch_mixed_bs<32>(c, Hq, scale, p, d, s);
    case 64:
      return launch_mixed_bs<64>(c, Hq, scale, p, d, s);
    default:
      return launch_mixed_bs<16>(c, Hq, scale, p, d, s);
  }
}

}  // namespace pa
