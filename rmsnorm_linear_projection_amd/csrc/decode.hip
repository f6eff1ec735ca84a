// Fused RMSNorm -> Linear for T <= 16 tokens: the weight-streaming regime.
//
// With few tokens the projection reads W[N, K] once and does little arithmetic
// per byte, so the kernel is bound by HBM bandwidth on W.  One workgroup owns
// 16 weight rows (one MFMA block of output columns) and all T tokens; its four
// wavefronts take four contiguous quarters of K, so every 128-byte line of a
// weight row is consumed by one wavefront in consecutive steps.
//
// Per workgroup:
//   1. the first batch of weight, x and gamma loads is issued;
//   2. each wavefront sums x^2 over its quarter of K for the T rows; the four
//      quarters are combined through LDS and every lane derives rstd for its
//      token (AT-10 page section 3, variant B, fp32);
//   3. for each 32-wide k-step, x (re-read, an L2 hit) is normed in fp32
//      (fl(fl(x * rstd) * gamma)), rounded to bf16 and fed with the weight
//      fragment to v_mfma_f32_16x16x32_bf16 (weight = MFMA A source, 16 rows;
//      tokens = MFMA B source, 16 columns, rows >= T read as zero);
//   4. the four partial accumulators are summed through LDS in a fixed order
//      and written as y[t, n .. n+3].
#include "common.cuh"
#include "launch.h"

namespace rnl {
namespace {

constexpr int kU = 4;   // k-steps of weight per prefetch batch
constexpr int kXS = 32; // x chunks per round trip of the sum-of-squares pass

__device__ __forceinline__ float sumsq8(u32x4 w) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float a = bf16lo(w[j]), b = bf16hi(w[j]);
    s += a * a;
    s += b * b;
  }
  return s;
}

template <bool GAMMA>
__device__ __forceinline__ u32x4 norm_bf16x8(u32x4 xv, u32x4 gv, float rstd) {
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float a = __fmul_rn(bf16lo(xv[j]), rstd);
    float b = __fmul_rn(bf16hi(xv[j]), rstd);
    if constexpr (GAMMA) {
      a = __fmul_rn(a, bf16lo(gv[j]));
      b = __fmul_rn(b, bf16hi(gv[j]));
    }
    r[j] = pack_bf16x2(a, b);
  }
  return r;
}

template <bool GAMMA, bool OUT_BF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void decode_kernel(const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ gamma, float eps,
                                                     float inv_k, const uint16_t* __restrict__ W,
                                                     void* __restrict__ y, float* __restrict__ rstd_out,
                                                     int T, int K, int N) {
  __shared__ float red_ss[4][16];
  __shared__ f32x4 red_acc[3][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16;

  const int nsteps = (K + 31) / 32;
  const int per = (nsteps + 3) / 4;
  const int s_beg = min(nsteps, wave * per), s_end = min(nsteps, s_beg + per);

  const uint32_t kbytes = (uint32_t)K * 2u;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)T * kbytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + (size_t)n0 * K, (uint32_t)min(16, N - n0) * kbytes);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(gamma, GAMMA ? kbytes : 0u);
  const uint32_t row_off = (uint32_t)t * kbytes;  // lane & 15 is the token row and the weight row
  // byte offset of k-step s inside a row for this lane, or kOOB past the range
  auto koff = [&](int s) -> uint32_t {
    const uint32_t kb = (uint32_t)(s * 32 + g * 8) * 2u;
    return (s < s_end && kb < kbytes) ? kb : kOOB;
  };
  auto at = [&](uint32_t k, uint32_t base) -> uint32_t { return k == kOOB ? kOOB : base + k; };

  // Operands of a batch of kU k-steps: weight rows, raw x rows and gamma, requested
  // together one batch ahead of their use (vector memory requests complete in
  // order, so a use never waits on a later prefetch).
  struct Batch {
    u32x4 w[kU], x[kU], g[kU];
  };
  auto issue = [&](Batch& b, int s0) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t k = koff(s0 + u);
      b.w[u] = buf_load16(rw, at(k, row_off));
      b.x[u] = buf_load16(rx, at(k, row_off));
      if constexpr (GAMMA) b.g[u] = buf_load16(rg, k);
      else b.g[u] = u32x4{0u, 0u, 0u, 0u};
    }
  };

  // phase 1: first weight batch in flight, then the sum of squares of token t over
  // this wavefront's quarter of K, kXS x chunks per round trip
  Batch cur;
  issue(cur, s_beg);
  float ss = 0.f;
  for (int s0 = s_beg; s0 < s_end; s0 += kXS) {
    u32x4 xb[kXS];
#pragma unroll
    for (int i = 0; i < kXS; ++i) xb[i] = buf_load16(rx, at(koff(s0 + i), row_off));
#pragma unroll
    for (int i = 0; i < kXS; ++i) ss += sumsq8(xb[i]);
  }
  ss += __shfl_xor(ss, 16, 64);
  ss += __shfl_xor(ss, 32, 64);
  if (g == 0) red_ss[wave][t] = ss;
  __syncthreads();
  const float S = red_ss[0][t] + red_ss[1][t] + red_ss[2][t] + red_ss[3][t];
  const float rstd = rstd_from_sumsq(S, inv_k, eps);
  if (rstd_out != nullptr && blockIdx.x == 0 && tid < T) rstd_out[tid] = rstd;

  // phase 2: normed bf16 tokens x weight rows on MFMA.  Two batch buffers alternate
  // (the loop is unrolled by two) so that no batch is ever copied: a register copy
  // of a prefetched batch would wait for its loads.
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto consume = [&](const Batch& b) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const u32x4 a = norm_bf16x8<GAMMA>(b.x[u], b.g[u], rstd);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b.w[u]),
                                                    __builtin_bit_cast(bf16x8, a), acc, 0, 0, 0);
    }
  };
  Batch alt;
  int s0 = s_beg;
  for (; s0 + kU < s_end; s0 += 2 * kU) {
    issue(alt, s0 + kU);
    __builtin_amdgcn_sched_barrier(0);  // all loads of the next batch go out first
    consume(cur);
    __builtin_amdgcn_sched_barrier(0);
    issue(cur, s0 + 2 * kU);
    __builtin_amdgcn_sched_barrier(0);
    consume(alt);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (s0 < s_end) consume(cur);  // an odd batch count leaves one batch in `cur`

  if (wave > 0) red_acc[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  acc += red_acc[0][lane];
  acc += red_acc[1][lane];
  acc += red_acc[2][lane];
  // lane holds D[n0 + 4g + r][t]
  if (t >= T) return;
  const int n = n0 + 4 * g;
  if (n >= N) return;
  const size_t off = (size_t)t * (size_t)N + (size_t)n;
  const bool full = ((N & 3) == 0) && (n + 3 < N);
  if constexpr (OUT_BF16) {
    uint16_t* c = static_cast<uint16_t*>(y) + off;
    if (full) {
      *reinterpret_cast<u32x2*>(c) = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    } else {
      for (int r = 0; r < 4 && n + r < N; ++r) c[r] = (uint16_t)(pack_bf16x2(acc[r], 0.f) & 0xFFFFu);
    }
  } else {
    float* c = static_cast<float*>(y) + off;
    if (full) {
      *reinterpret_cast<f32x4*>(c) = acc;
    } else {
      for (int r = 0; r < 4 && n + r < N; ++r) c[r] = acc[r];
    }
  }
}

}  // namespace

hipError_t launch_decode_bf16(const uint16_t* x, const uint16_t* gamma, float eps,
                              const uint16_t* W, void* y, int out_kind, float* rstd_out, int64_t T,
                              int64_t K, int64_t N, hipStream_t s) {
  const float inv_k = 1.0f / (float)K;
  dim3 grid((unsigned)((N + 15) / 16)), block(256);
  const bool ob = out_kind == OUT_BF16;
#define RNL_DEC(G, O) \
  hipLaunchKernelGGL((decode_kernel<G, O>), grid, block, 0, s, x, gamma, eps, inv_k, W, y, rstd_out, (int)T, (int)K, (int)N)
  if (gamma != nullptr) {
    if (ob) RNL_DEC(true, true); else RNL_DEC(true, false);
  } else {
    if (ob) RNL_DEC(false, true); else RNL_DEC(false, false);
  }
#undef RNL_DEC
  return hipGetLastError();
}

}  // namespace rnl
