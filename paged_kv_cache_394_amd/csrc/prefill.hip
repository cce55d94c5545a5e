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
// Tiling.  A workgroup owns 128 query rows of one (sequence, head): 4 wave64s of
// 32 rows (two 16-row sub-tiles).  Keys are walked in tiles of 64 (four 16-token
// blocks looked up in the block table), staged through LDS: K row-major, V
// transposed, so both MFMA operands are read as short contiguous runs.
// Each wave computes S^T = K Q^T (so a lane ends up holding the scores of one
// query row, which makes the row max / sum and the output rescale lane-local up
// to two cross-lane steps) and then O^T = V^T P^T with P taken straight from the
// S^T registers: the 32-key contraction of one MFMA is permuted so that lane
// group g's 8 slots are keys {4g..4g+3} and {16+4g..16+4g+3} of a 32-key pair,
// exactly the scores that lane already holds; the V^T operand is read with the
// same permutation.  Online softmax in the log2 domain, fp32 statistics, P
// rounded to fp16 for the MFMA, fp32 accumulation.  The causal mask is applied
// only on tiles that cross the diagonal.
#include <cmath>

#include "device_common.hpp"
#include "launch.hpp"

namespace pa {
namespace {

using namespace dev;

constexpr int kBq = 128;       // query rows per workgroup
constexpr int kBk = 64;        // keys per tile
constexpr int kThreads = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void prefill_kernel(
    const half_t* __restrict__ q, const half_t* __restrict__ kc, const half_t* __restrict__ vc,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ prior,
    const int32_t* __restrict__ tables, float* __restrict__ out, int32_t Hq, int32_t Hkv,
    int32_t total_q, int32_t max_blocks, int32_t num_blocks, float qk_scale) {
  constexpr int KP = D + 8;     // LDS row stride of K (halfs)
  constexpr int VP = kBk + 8;   // LDS row stride of V^T (halfs)
  constexpr int DK = D / 32;    // MFMA steps over head_dim for S
  constexpr int DT = D / 16;    // 16-wide output tiles over head_dim
  constexpr int CPR = D / 8;    // 16-byte chunks per K/V row
  constexpr int CHUNKS = kBk * CPR;
  static_assert(CHUNKS % kThreads == 0, "tile load must split evenly");
  __shared__ __attribute__((aligned(16))) half_t sK[kBk * KP];
  __shared__ __attribute__((aligned(16))) half_t sVt[D * VP];

  const int qt = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int g = lane >> 4;
  const int c16 = lane & 15;

  const int row0 = cu_q[b];
  const int C = cu_q[b + 1] - row0;
  const int P = max(prior[b], 0);
  const int q0 = qt * kBq;
  if (q0 >= C || row0 < 0) return;
  const int L_total = min(P + C, max_blocks * kBlock);
  const int kvh = h / (Hq / Hkv);
  const int32_t* trow = tables + static_cast<int64_t>(b) * max_blocks;

  // Q as the B operand of S^T = K Q^T: lane holds q[row = c16][d = 32 kk + 8 g .. +8]
  half8_t qb[2][DK];
  int qrow[2];
  bool qvalid[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    qrow[st] = q0 + 32 * w + 16 * st + c16;
    qvalid[st] = qrow[st] < C && (row0 + qrow[st]) < total_q;
    const half_t* qp = q + (static_cast<int64_t>(row0 + qrow[st]) * Hq + h) * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) {
      qb[st][kk] = qvalid[st] ? *reinterpret_cast<const half8_t*>(qp + 32 * kk) : half8_t{};
    }
  }

  float4_t o[2][DT];
  float m[2], l[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    m[st] = -INFINITY;
    l[st] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[st][dt] = float4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int wq_first = q0 + 32 * w;                      // first query row of this wave
  const int wq_last = min(q0 + 32 * w + 32, C) - 1;      // last valid one (< first if none)
  const int n_keys = min(P + min(q0 + kBq, C), L_total);  // keys any row of the group needs
  const int ntiles = (n_keys + kBk - 1) / kBk;

  for (int kt = 0; kt < ntiles; ++kt) {
    const int key0 = kt * kBk;
    __syncthreads();  // previous tile fully consumed
#pragma unroll
    for (int pass = 0; pass < CHUNKS / kThreads; ++pass) {
      const int cidx = pass * kThreads + tid;
      const int key = cidx / CPR;        // key within the tile
      const int d0 = (cidx % CPR) * 8;
      const int kabs = key0 + key;
      u32x4_t kv = u32x4_t{0u, 0u, 0u, 0u};
      u32x4_t vv = u32x4_t{0u, 0u, 0u, 0u};
      if (kabs < L_total) {
        int phys = trow[kabs >> 4];
        phys = (static_cast<uint32_t>(phys) < static_cast<uint32_t>(num_blocks)) ? phys : 0;
        const int64_t off =
            ((static_cast<int64_t>(phys) * Hkv + kvh) * kBlock + (kabs & 15)) * D + d0;
        kv = *reinterpret_cast<const u32x4_t*>(kc + off);
        vv = *reinterpret_cast<const u32x4_t*>(vc + off);
      }
      *reinterpret_cast<u32x4_t*>(&sK[key * KP + d0]) = kv;
      const half8_t vh = __builtin_bit_cast(half8_t, vv);
#pragma unroll
      for (int e = 0; e < 8; ++e) sVt[(d0 + e) * VP + key] = vh[e];
    }
    __syncthreads();

    if (wq_last < wq_first || key0 > P + wq_last) continue;  // nothing visible to this wave

    // S^T tiles: [st][ks] holds keys key0 + 16 ks + 4 g + i for query row c16
    float4_t sacc[2][4];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sacc[st][ks] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int kk = 0; kk < DK; ++kk) {
        const half8_t a = *reinterpret_cast<const half8_t*>(&sK[(ks * 16 + c16) * KP + 32 * kk + 8 * g]);
#pragma unroll
        for (int st = 0; st < 2; ++st)
          sacc[st][ks] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qb[st][kk], sacc[st][ks], 0, 0, 0);
      }
    }

    const bool need_mask = key0 + kBk - 1 > P + wq_first;
    half_t ph[2][4][4];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int lim = P + qrow[st];  // last visible key of this lane's row
      float mt = -INFINITY;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = sacc[st][ks][i] * qk_scale;
          if (need_mask && (key0 + 16 * ks + 4 * g + i) > lim) v = -INFINITY;
          sacc[st][ks][i] = v;
          mt = fmaxf(mt, v);
        }
      }
      mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float m_new = fmaxf(m[st], mt);
      const float corr = (m[st] == -INFINITY) ? 0.f : fast_exp2(m[st] - m_new);
      m[st] = m_new;
      l[st] *= corr;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[st][dt] *= corr;
      float ps = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pr = fast_exp2(sacc[st][ks][i] - m_new);
          ps += pr;
          ph[st][ks][i] = static_cast<half_t>(pr);
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
        bp[st] = half8_t{ph[st][2 * kp][0], ph[st][2 * kp][1], ph[st][2 * kp][2], ph[st][2 * kp][3],
                         ph[st][2 * kp + 1][0], ph[st][2 * kp + 1][1], ph[st][2 * kp + 1][2],
                         ph[st][2 * kp + 1][3]};
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const half_t* vrow = &sVt[(dt * 16 + c16) * VP + kp * 32 + 4 * g];
        const half4_t a0 = *reinterpret_cast<const half4_t*>(vrow);
        const half4_t a1 = *reinterpret_cast<const half4_t*>(vrow + 16);
        const half8_t a = half8_t{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
        for (int st = 0; st < 2; ++st)
          o[st][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bp[st], o[st][dt], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int st = 0; st < 2; ++st) {
    float lt = l[st];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    if (!qvalid[st]) continue;
    const float inv = 1.0f / lt;
    float* orow = out + (static_cast<int64_t>(row0 + qrow[st]) * Hq + h) * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      *reinterpret_cast<float4_t*>(orow + dt * 16) = o[st][dt] * inv;
    }
  }
}

}  // namespace

hipError_t launch_prefill(const KvDesc& c, const void* q, int32_t Hq, int32_t total_q,
                          const int32_t* cu_q, const int32_t* prior, const int32_t* tables,
                          int32_t B, int32_t max_blocks, int32_t max_chunk, float scale, float* out,
                          hipStream_t s) {
  if (B <= 0 || max_chunk <= 0 || total_q <= 0) return hipSuccess;
  const int32_t nqt = (max_chunk + kBq - 1) / kBq;
  const float qk_scale = scale * kLog2e;
  const dim3 grid(nqt, Hq, B);
  if (c.head_dim == 128) {
    prefill_kernel<128><<<grid, dim3(kThreads), 0, s>>>(
        static_cast<const half_t*>(q), static_cast<const half_t*>(c.k),
        static_cast<const half_t*>(c.v), cu_q, prior, tables, out, Hq, c.num_kv_heads, total_q,
        max_blocks, c.num_blocks, qk_scale);
  } else {
    prefill_kernel<64><<<grid, dim3(kThreads), 0, s>>>(
        static_cast<const half_t*>(q), static_cast<const half_t*>(c.k),
        static_cast<const half_t*>(c.v), cu_q, prior, tables, out, Hq, c.num_kv_heads, total_q,
        max_blocks, c.num_blocks, qk_scale);
  }
  return hipGetLastError();
}

}  // namespace pa
