// Projection for M <= 16 rows of activations: the weight-streaming regime.
//
// With at most 16 tokens the product C[M, N] = A[M, K] . W[N, K]^T reads the
// weight once and does little arithmetic per byte, so time is set by how fast
// W streams from HBM.  Two facts shape the kernel:
//   * a compute unit sustains only a limited number of outstanding HBM misses,
//     so every CU must stream an equal share of W: a workgroup owns R weight
//     rows (R a multiple of 4, at most 32 = two 16-row MFMA blocks, chosen on
//     the host so that the busiest CU holds the fewest rows, then the largest
//     R: N = 6144 -> R = 24, 256 workgroups, one per CU);
//   * the activations (at most 16 x K bf16) are tiny and stay in L2; they are
//     already normed and rounded (the norm runs once per token in a pre-pass),
//     so the loop does no vector arithmetic at all.  For at most four rows the
//     norm is fused instead (small_m_norm_kernel below).
//
// Per workgroup: four wavefronts take four contiguous quarters of K.  Each
// k-step (32 k) is one v_mfma_f32_16x16x32_bf16 with the weight as the MFMA A
// source (lane l: weight row l & 15, 16 bytes at k-chunk l >> 4) and the
// activations as the B source (lane l: token l & 15, same k-chunk).  Weight
// rows >= R, tokens >= M and the K tail read as zero through the buffer
// bounds.  Loads run KU k-steps ahead in two alternating register batches
// (KU = 2: at N = 6144, K = 4096, T = 16 the kernel takes 13.0 us against 13.7
// with KU = 4, 14.5 with 3 and 15.4 with 1).
// The four wavefront accumulators are added through LDS in a fixed order.
#include "launch.h"
#include "rows.hpp"

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

// The same weight streaming with the RMSNorm of the (raw) activation rows fused
// in, for a few tokens, where the pre-pass would cost a launch and an HBM round
// trip of its own for a handful of rows.  Every workgroup norms the M rows
// itself, once, into LDS (k-step major: the 32 values of token t at k-step s
// sit at byte (s * M + t) * 64, so a wavefront's B fragments of one k-step are
// M * 64 contiguous bytes): wavefront w takes tokens w, w + NW, ..., sums the
// squares of its row in fp32 (chunk lane + 64 c of the row in lane `lane`, then
// a wavefront sum), derives rstd, and stores a = bf16(fl(fl(x * rstd) * gamma))
// -- the value the pre-pass writes.  The row (and gamma) is requested before
// the first two weight batches, so it does not queue behind them.  The main
// loop is the one above with the B fragments read from LDS.  Lanes of tokens r >= M read token M - 1's fragment: their
// MFMA output column is never stored, and columns of an MFMA do not mix.
// LDS: M * ceil(K / 32) * 64 bytes (k-steps past K hold zeros), reused for
// the cross-wave sum at the end.
//
// RPW > 0 selects the prologue for up to NW * RPW rows of at most 64 * CPL
// chunks: wavefront w norms rows w, w + NW, ... and requests every chunk of all
// of them (and gamma's) at once, so the norm costs one L2 round trip instead
// of one per row; the weight batches are issued right after those requests.
template <int NB, int NW, int KU, bool OUT_BF16, bool GAMMA, int RPW = 0, int CPL = 8>
__global__ __launch_bounds__(NW * 64) void small_m_norm_kernel(const uint16_t* __restrict__ X,
                                                               const uint16_t* __restrict__ gamma, float eps,
                                                               float inv_k, const uint16_t* __restrict__ W,
                                                               void* __restrict__ C, float* __restrict__ rstd_out,
                                                               int M, int K, int N, int R) {
  extern __shared__ __attribute__((aligned(16))) char xs[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * R;
  const int rows = min(R, N - n0);

  const int nsteps = (K + 31) / 32;
  const int per = (nsteps + NW - 1) / NW;
  const int s_beg = min(nsteps, wave * per), s_end = min(nsteps, s_beg + per);

  const uint32_t kbytes = (uint32_t)K * 2u;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + (size_t)n0 * K, (uint32_t)rows * kbytes);
  const uint32_t row_off = (uint32_t)r * kbytes;
  auto off = [&](int s) -> uint32_t {
    const uint32_t kb = (uint32_t)(s * 32 + g * 8) * 2u;
    return (s < s_end && kb < kbytes) ? row_off + kb : kOOB;
  };
  auto at_block = [&](uint32_t o, int b) -> uint32_t { return o == kOOB ? kOOB : o + (uint32_t)(16 * b) * kbytes; };
  // LDS byte offset of this lane's B fragment of k-step s (a k-step outside this
  // wavefront's range reads k-step 0, which always exists; its weight reads as zero)
  const uint32_t lds_lane = (uint32_t)(min(r, M - 1) * 64 + g * 16);
  auto lds_off = [&](int s) -> uint32_t { return (uint32_t)((s < s_end ? s : 0) * M) * 64u + lds_lane; };

  struct Batch {
    u32x4 w[KU][NB], a[KU];
  };
  auto issue_w = [&](Batch& bt, int s0) {
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const uint32_t o = off(s0 + u);
#pragma unroll
      for (int b = 0; b < NB; ++b) bt.w[u][b] = buf_load16(rw, at_block(o, b));
    }
  };
  auto read_a = [&](Batch& bt, int s0) {
#pragma unroll
    for (int u = 0; u < KU; ++u) bt.a[u] = *reinterpret_cast<const u32x4*>(xs + lds_off(s0 + u));
  };

  // The first activation batch (and gamma) is requested before the weight
  // batches, so that the norm does not wait behind them in the load queue.
  const int nch = K >> 3;          // 16-byte chunks of a row
  const int nch_pad = nsteps * 4;  // chunks up to the next whole k-step
  const u32x4* gr = reinterpret_cast<const u32x4*>(gamma);
  u32x4 v[8], gv[8];
  auto load_x = [&](int t, int c0) {
    const u32x4* xr = reinterpret_cast<const u32x4*>(X + (size_t)t * K);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int idx = c0 + lane + kWave * c;
      v[c] = idx < nch ? xr[idx] : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto load_g = [&](int c0) {
    if constexpr (GAMMA) {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int idx = c0 + lane + kWave * c;
        gv[c] = idx < nch ? gr[idx] : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  // n = fl(fl(x * rstd) * gamma) of one chunk, rounded to bf16, stored at its
  // k-step-major place (zeros past K, up to the next whole k-step)
  auto store_normed = [&](int t, int idx, u32x4 xv, u32x4 gvv, float rstd) {
    float n[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      n[2 * j] = __fmul_rn(bf16lo(xv[j]), rstd);
      n[2 * j + 1] = __fmul_rn(bf16hi(xv[j]), rstd);
      if constexpr (GAMMA) {
        n[2 * j] = __fmul_rn(n[2 * j], bf16lo(gvv[j]));
        n[2 * j + 1] = __fmul_rn(n[2 * j + 1], bf16hi(gvv[j]));
      }
    }
    const u32x4 q = idx < nch ? u32x4{pack_bf16x2(n[0], n[1]), pack_bf16x2(n[2], n[3]), pack_bf16x2(n[4], n[5]),
                                      pack_bf16x2(n[6], n[7])}
                              : u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(xs + ((uint32_t)((idx >> 2) * M + t) * 64u + (uint32_t)(idx & 3) * 16u)) = q;
  };
  Batch cur, alt;
  if constexpr (RPW > 0) {
    u32x4 rv[RPW][CPL], rg[CPL];
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const int t = wave + NW * j;
      const u32x4* xr = reinterpret_cast<const u32x4*>(X + (size_t)min(t, M - 1) * K);
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int idx = lane + kWave * c;
        rv[j][c] = (t < M && idx < nch) ? xr[idx] : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int idx = lane + kWave * c;
      rg[c] = (GAMMA && idx < nch) ? gr[idx] : u32x4{0u, 0u, 0u, 0u};
    }
    __builtin_amdgcn_sched_barrier(0);
    issue_w(cur, s_beg);
    issue_w(alt, s_beg + KU);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const int t = wave + NW * j;
      if (t >= M) break;  // wavefront-uniform
      float ss = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) ss += sumsq8(rv[j][c]);
      const float rstd = rstd_from_sumsq(wave_sum(ss), inv_k, eps);
      if (blockIdx.x == 0 && lane == 0 && rstd_out != nullptr) rstd_out[t] = rstd;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int idx = lane + kWave * c;
        if (idx < nch_pad) store_normed(t, idx, rv[j][c], rg[c], rstd);
      }
    }
  } else {
  if (wave < M) {
    load_x(wave, 0);
    load_g(0);
  }
  __builtin_amdgcn_sched_barrier(0);
  issue_w(cur, s_beg);
  issue_w(alt, s_beg + KU);
  __builtin_amdgcn_sched_barrier(0);

  // norm the M rows into LDS, one wavefront per row
  for (int t = wave; t < M; t += NW) {
    float ss = 0.f;
    for (int c0 = 0; c0 < nch; c0 += 8 * kWave) {
      if (c0 > 0 || t != wave) load_x(t, c0);
#pragma unroll
      for (int c = 0; c < 8; ++c) ss += sumsq8(v[c]);
    }
    const float rstd = rstd_from_sumsq(wave_sum(ss), inv_k, eps);
    if (blockIdx.x == 0 && lane == 0 && rstd_out != nullptr) rstd_out[t] = rstd;
    for (int c0 = 0; c0 < nch_pad; c0 += 8 * kWave) {
      if (nch > 8 * kWave) {  // the row did not fit one batch: read this part again (from cache)
        load_x(t, c0);
        load_g(c0);
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int idx = c0 + lane + kWave * c;
        if (idx < nch_pad) store_normed(t, idx, v[c], gv[c], rstd);
      }
    }
  }
  }
  __syncthreads();
  read_a(cur, s_beg);
  read_a(alt, s_beg + KU);

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

  // cur holds k-steps s0 .. s0+KU-1 and alt the next KU when an iteration starts
  int s0 = s_beg;
  for (; s0 + KU < s_end; s0 += 2 * KU) {
    consume(cur);
    __builtin_amdgcn_sched_barrier(0);
    issue_w(cur, s0 + 2 * KU);
    read_a(cur, s0 + 2 * KU);
    __builtin_amdgcn_sched_barrier(0);
    consume(alt);
    __builtin_amdgcn_sched_barrier(0);
    issue_w(alt, s0 + 3 * KU);
    read_a(alt, s0 + 3 * KU);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (s0 < s_end) consume(cur);

  // the row buffer becomes the cross-wave sum buffer once every wave is done with it
  __syncthreads();
  f32x4* red = reinterpret_cast<f32x4*>(xs);  // [NW - 1][NB][64]
  if (wave > 0) {
#pragma unroll
    for (int b = 0; b < NB; ++b) red[((wave - 1) * NB + b) * 64 + lane] = acc[b];
  }
  __syncthreads();
  if (wave != 0 || r >= M) return;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int w = 0; w < NW - 1; ++w) acc[b] += red[(w * NB + b) * 64 + lane];
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

namespace {
// Weight rows per workgroup of the fused-norm kernel: one 16-row MFMA block
// (R <= 16), the fewest rows on the busiest CU, then the largest R.  Measured
// against small_m_rows' choice (which allows two blocks): N = 6144, K = 4096:
// R = 12 12.7 us against R = 24 13.3; N = 24576, K = 1536: R = 16 16.9 us
// against R = 32 20.1.
int small_m_norm_rows(int64_t N) {
  int best = 16;
  int64_t best_load = INT64_MAX;
  for (int R = 16; R >= 4; R -= 4) {
    const int64_t wgs = (N + R - 1) / R;
    const int64_t load = ((wgs + kCUs - 1) / kCUs) * R;
    if (load < best_load) {
      best_load = load;
      best = R;
    }
  }
  return best;
}
}  // namespace

size_t small_m_norm_lds(int64_t M, int64_t K) {
  const size_t rows = (size_t)M * (size_t)((K + 31) / 32) * 64u;
  const size_t red = 3u * 2u * 64u * sizeof(f32x4);  // (NW - 1) x NB x 64 accumulators, at most
  return rows > red ? rows : red;
}

namespace {
// Launch of the prologue that requests every row at once (RPW = 4 rows per
// wavefront, rows of at most 512 * CPL values): NB = 2 row blocks per
// workgroup, so that one workgroup per CU covers N = 6144 in one round (the
// normed rows take up to 128 KiB of LDS, one workgroup per CU).
template <int NB, bool O, bool G, int CPL>
hipError_t launch_all_rows(const uint16_t* X, const uint16_t* gamma, float eps, float inv_k, const uint16_t* W,
                           void* C, float* rstd_out, int M, int K, int N, int R, size_t lds, hipStream_t s) {
  auto kern = small_m_norm_kernel<NB, 4, 4, O, G, 4, CPL>;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)kSmallNormLdsAllRows);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(kern, dim3((unsigned)((N + R - 1) / R)), dim3(256), lds, s, X, gamma, eps, inv_k, W, C, rstd_out,
                     M, K, N, R);
  return hipGetLastError();
}

template <int NB, bool O, bool G>
hipError_t launch_all_rows_cpl(int cpl, const uint16_t* X, const uint16_t* gamma, float eps, float inv_k,
                               const uint16_t* W, void* C, float* rstd_out, int M, int K, int N, int R, size_t lds,
                               hipStream_t s) {
  switch (cpl) {
    case 1: return launch_all_rows<NB, O, G, 1>(X, gamma, eps, inv_k, W, C, rstd_out, M, K, N, R, lds, s);
    case 2: return launch_all_rows<NB, O, G, 2>(X, gamma, eps, inv_k, W, C, rstd_out, M, K, N, R, lds, s);
    case 4: return launch_all_rows<NB, O, G, 4>(X, gamma, eps, inv_k, W, C, rstd_out, M, K, N, R, lds, s);
    default: return launch_all_rows<NB, O, G, 8>(X, gamma, eps, inv_k, W, C, rstd_out, M, K, N, R, lds, s);
  }
}
}  // namespace

// Where fusing pays (graph-timed A/B against pre-pass + weight streaming, rotated
// weights, us): T = 8, K = 1024, N = 4096: 4.5 against 6.6; T = 16, K = 1024: 5.4
// against 6.9; T = 8, K = 2048, N = 6144: 9.0 against 10.3; T = 16, K = 2048:
// 10.7 against 11.0; T = 8, K = 256, N = 128: 3.3 against 4.1; T = 8, K = 4096,
// N = 6144: 14.6 against 14.9.  Past 64 KiB of normed rows it loses (T = 12, K =
// 4096: 15.8 against 15.5; T = 16, K = 4096: 17.2 against 16.1): one workgroup
// per CU cannot overlap a 16-row prologue with the weight stream.
bool small_m_norm_fits(int64_t M, int64_t K) {
  if (M < 1 || M > kFusedNormAllM || small_m_norm_lds(M, K) > kSmallNormLds) return false;
  return M <= kFusedNormRowsM || K <= kFusedNormAllK;
}

hipError_t launch_small_m_norm_bf16(const uint16_t* X, const uint16_t* gamma, float eps, const uint16_t* W,
                                    void* C, int out_kind, float* rstd_out, int64_t M, int64_t N, int64_t K,
                                    hipStream_t s) {
  if (!small_m_norm_fits(M, K)) return hipErrorInvalidValue;
  if (M > kFusedNormRowsM) {
    const int R = small_m_rows(N);
    const int64_t nch = K / 8;
    const int cpl = nch <= 64 ? 1 : nch <= 128 ? 2 : nch <= 256 ? 4 : 8;
    const size_t lds = small_m_norm_lds(M, K);
    const float ik = 1.0f / (float)K;
    const bool ob = out_kind == OUT_BF16, g = gamma != nullptr;
#define RNL_ALL_ROWS(NB, O, G) \
  return launch_all_rows_cpl<NB, O, G>(cpl, X, gamma, eps, ik, W, C, rstd_out, (int)M, (int)K, (int)N, R, lds, s)
    if (R <= 16) {
      if (ob) { if (g) RNL_ALL_ROWS(1, true, true); else RNL_ALL_ROWS(1, true, false); }
      else { if (g) RNL_ALL_ROWS(1, false, true); else RNL_ALL_ROWS(1, false, false); }
    } else {
      if (ob) { if (g) RNL_ALL_ROWS(2, true, true); else RNL_ALL_ROWS(2, true, false); }
      else { if (g) RNL_ALL_ROWS(2, false, true); else RNL_ALL_ROWS(2, false, false); }
    }
#undef RNL_ALL_ROWS
  }
  const int R = small_m_norm_rows(N);
  dim3 grid((unsigned)((N + R - 1) / R)), block(256);
  const bool ob = out_kind == OUT_BF16;
  const float inv_k = 1.0f / (float)K;
  const size_t lds = small_m_norm_lds(M, K);
#define RNL_SMALL_MN(NB, O, G)                                                                                 \
  hipLaunchKernelGGL((small_m_norm_kernel<NB, 4, 4, O, G>), grid, block, lds, s, X, gamma, eps, inv_k, W, C, \
                     rstd_out, (int)M, (int)K, (int)N, R)
#define RNL_SMALL_MN_G(NB, O) \
  if (gamma != nullptr) RNL_SMALL_MN(NB, O, true); else RNL_SMALL_MN(NB, O, false)
  // R <= 16: one MFMA block of weight rows
  if (ob) RNL_SMALL_MN_G(1, true); else RNL_SMALL_MN_G(1, false);
#undef RNL_SMALL_MN_G
#undef RNL_SMALL_MN
  return hipGetLastError();
}

hipError_t launch_small_m_bf16(const uint16_t* A, const uint16_t* W, void* C, int out_kind, int64_t M,
                               int64_t N, int64_t K, int R, hipStream_t s) {
  if (R <= 0) R = small_m_rows(N);
  dim3 grid((unsigned)((N + R - 1) / R)), block(256);
  const bool ob = out_kind == OUT_BF16;
#define RNL_SMALL_M(NB, O) \
  hipLaunchKernelGGL((small_m_kernel<NB, 4, 2, O>), grid, block, 0, s, A, W, C, (int)M, (int)K, (int)N, R)
  if (R <= 16) {
    if (ob) RNL_SMALL_M(1, true); else RNL_SMALL_M(1, false);
  } else {
    if (ob) RNL_SMALL_M(2, true); else RNL_SMALL_M(2, false);
  }
#undef RNL_SMALL_M
  return hipGetLastError();
}

}  // namespace rnl
