// Projection for M <= 16 rows of activations: the weight-streaming regime.
//
// With at most 16 tokens the product C[M, N] = A[M, K] . W[N, K]^T reads the
// weight once and does little arithmetic per byte, so time is set by how fast
// W streams from HBM.  Two facts shape the kernel:
//   * a compute unit sustains only a limited number of outstanding HBM misses,
//     so every CU must stream an equal share of W: a workgroup owns R weight
//     rows (R in {16, 12, 8}, chosen on the host so that ceil(N / R) workgroups
//     spread evenly over the 256 CUs, e.g. N = 6144 -> R = 12, 512 workgroups);
//   * the activations (at most 16 x K bf16) are tiny and stay in L2; they are
//     already normed and rounded (the norm runs once per token in a pre-pass),
//     so the loop does no vector arithmetic at all.
//
// Per workgroup: four wavefronts take four contiguous quarters of K.  Each
// k-step (32 k) is one v_mfma_f32_16x16x32_bf16 with the weight as the MFMA A
// source (lane l: weight row l & 15, 16 bytes at k-chunk l >> 4) and the
// activations as the B source (lane l: token l & 15, same k-chunk).  Weight
// rows >= R, tokens >= M and the K tail read as zero through the buffer
// bounds.  Loads run KU k-steps ahead in two alternating register batches.
// The four wavefront accumulators are added through LDS in a fixed order.
#include "common.cuh"
#include "launch.h"

namespace rnl {
namespace {

// NB: 16-row MFMA blocks per workgroup (R <= 16 * NB weight rows); NW: wavefronts,
// each taking one of NW contiguous parts of K; KU: k-steps per load batch.
template <int NB, int NW, int KU, bool OUT_BF16>
__global__ __launch_bounds__(NW * 64) void small_m_kernel(const uint16_t* __restrict__ A,
                                                          const uint16_t* __restrict__ W,
                                                          void* __restrict__ C, int M, int K, int N,
                                                          int R) {
  __shared__ f32x4 red[NW - 1][NB][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * R;
  const int rows = min(R, N - n0);

  const int nsteps = (K + 31) / 32;
  const int per = (nsteps + NW - 1) / NW;
  const int s_beg = min(nsteps, wave * per), s_end = min(nsteps, s_beg + per);

  const uint32_t kbytes = (uint32_t)K * 2u;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + (size_t)n0 * K, (uint32_t)rows * kbytes);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)M * kbytes);
  const uint32_t row_off = (uint32_t)r * kbytes;  // weight row r (+16 b) and token r of this lane
  // offset of k-step s for this lane, or kOOB outside this wavefront's range / past K
  auto off = [&](int s) -> uint32_t {
    const uint32_t kb = (uint32_t)(s * 32 + g * 8) * 2u;
    return (s < s_end && kb < kbytes) ? row_off + kb : kOOB;
  };
  auto at_block = [&](uint32_t o, int b) -> uint32_t { return o == kOOB ? kOOB : o + (uint32_t)(16 * b) * kbytes; };

  struct Batch {
    u32x4 w[KU][NB], a[KU];
  };
  auto issue = [&](Batch& bt, int s0) {
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const uint32_t o = off(s0 + u);
#pragma unroll
      for (int b = 0; b < NB; ++b) bt.w[u][b] = buf_load16(rw, at_block(o, b));
      bt.a[u] = buf_load16(ra, o);
    }
  };
  f32x4 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto consume = [&](const Batch& bt) {
#pragma unroll
    for (int u = 0; u < KU; ++u)
#pragma unroll
      for (int b = 0; b < NB; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, bt.w[u][b]),
                                                         __builtin_bit_cast(bf16x8, bt.a[u]), acc[b], 0, 0, 0);
  };

  // Two batches alternate so that no batch is copied (a register copy of a
  // batch in flight would wait for its loads); the loop is unrolled by two.
  Batch cur, alt;
  issue(cur, s_beg);
  int s0 = s_beg;
  for (; s0 + KU < s_end; s0 += 2 * KU) {
    issue(alt, s0 + KU);
    __builtin_amdgcn_sched_barrier(0);
    consume(cur);
    __builtin_amdgcn_sched_barrier(0);
    issue(cur, s0 + 2 * KU);
    __builtin_amdgcn_sched_barrier(0);
    consume(alt);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (s0 < s_end) consume(cur);

  if (wave > 0) {
#pragma unroll
    for (int b = 0; b < NB; ++b) red[wave - 1][b][lane] = acc[b];
  }
  __syncthreads();
  if (wave != 0 || r >= M) return;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int w = 0; w < NW - 1; ++w) acc[b] += red[w][b][lane];
    // lane holds C[token r][n0 + 16b + 4g + j], j = 0..3 (MFMA D layout: A rows 4g + j, B column r)
    const int i0 = 16 * b + 4 * g;
    if (i0 >= rows) continue;
    const f32x4 v = acc[b];
    const size_t o = (size_t)r * (size_t)N + (size_t)(n0 + i0);
    const bool full = ((N & 3) == 0) && (i0 + 3 < rows);
    if constexpr (OUT_BF16) {
      uint16_t* c = static_cast<uint16_t*>(C) + o;
      if (full) {
        *reinterpret_cast<u32x2*>(c) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      } else {
        for (int j = 0; j < 4 && i0 + j < rows; ++j) c[j] = (uint16_t)(pack_bf16x2(v[j], 0.f) & 0xFFFFu);
      }
    } else {
      float* c = static_cast<float*>(C) + o;
      if (full) {
        *reinterpret_cast<f32x4*>(c) = v;
      } else {
        for (int j = 0; j < 4 && i0 + j < rows; ++j) c[j] = v[j];
      }
    }
  }
}

constexpr int kCUs = 256;

}  // namespace

int small_m_rows(int64_t N) {
  // weight rows per workgroup: the fewest rows on the busiest CU, then the
  // largest R (fewer workgroups re-read the activations)
  int best = 32;
  int64_t best_load = INT64_MAX;
  for (int R = 32; R >= 4; R -= 4) {
    const int64_t wgs = (N + R - 1) / R;
    const int64_t load = ((wgs + kCUs - 1) / kCUs) * R;
    if (load < best_load) {
      best_load = load;
      best = R;
    }
  }
  return best;
}

hipError_t launch_small_m_bf16(const uint16_t* A, const uint16_t* W, void* C, int out_kind, int64_t M,
                               int64_t N, int64_t K, int R, hipStream_t s) {
  if (R <= 0) R = small_m_rows(N);
  dim3 grid((unsigned)((N + R - 1) / R)), block(256);
  const bool ob = out_kind == OUT_BF16;
#define RNL_SMALL_M(NB, O) \
  hipLaunchKernelGGL((small_m_kernel<NB, 4, 4, O>), grid, block, 0, s, A, W, C, (int)M, (int)K, (int)N, R)
  if (R <= 16) {
    if (ob) RNL_SMALL_M(1, true); else RNL_SMALL_M(1, false);
  } else {
    if (ob) RNL_SMALL_M(2, true); else RNL_SMALL_M(2, false);
  }
#undef RNL_SMALL_M
  return hipGetLastError();
}

}  // namespace rnl
