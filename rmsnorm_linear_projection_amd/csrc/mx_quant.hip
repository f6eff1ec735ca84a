// RMSNorm + MX quantisation pre-pass for the MXFP8 projection (gfx950).
//
// AT-10 with AT-09's MXFP8 mode: the fp32 normed rows are cut into blocks of 64
// consecutive values; each block gets one E8M0 scale X = 2^e with
// e = floor(log2(amax)) - 8 (8 is the largest exponent of E4M3; e clamped to
// [-127, 127]; an all-zero block takes e = -127), and each value becomes the
// E4M3 code nearest to n / X (ties to the even mantissa, magnitudes beyond 448
// clamped to 448, a zero result encoded as +0).
//
// One wavefront per row.  Pass 1 streams the row for the fp32 sum of squares;
// pass 2 streams it again (from cache), norms each 8-value chunk, and the 8
// lanes that hold one 64-block exchange their maxima with xor shuffles.  Every
// lane runs the same number of iterations, so the shuffles never run in
// divergent code.
#include "launch.h"
#include "rows.cuh"

namespace rnl {
namespace {

constexpr int kMxThreads = 256;

// E4M3 code of v: nearest even, saturating at 448, +0 for a zero result.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t ab = b & 0x7FFFFFFFu;
  const float a = __uint_as_float(ab);
  uint32_t mag;
  if (!(a < 448.0f)) {
    mag = 0x7Eu;
  } else if (a < 0.015625f) {
    // below 2^-6 the spacing is 2^-9: the code is the rounded multiple itself
    // (a rounded value of 8 is 2^-6, whose code is 0x08)
    mag = (uint32_t)rintf(a * 512.0f);
  } else {
    // keep 3 mantissa bits, round to nearest even at bit 20, rebias 127 -> 7
    const uint32_t r = (ab + 0x7FFFFu + ((ab >> 20) & 1u)) >> 20;
    mag = r - ((127u - 7u) << 3);
    if (mag > 0x7Eu) mag = 0x7Eu;
  }
  return mag == 0u ? 0u : (mag | ((b >> 24) & 0x80u));
}

template <bool GAMMA>
__global__ __launch_bounds__(kMxThreads) void norm_rows_mx_kernel(const uint16_t* __restrict__ x,
                                                                  const uint16_t* __restrict__ gamma, float eps,
                                                                  float inv_k, int64_t T, int64_t K,
                                                                  uint8_t* __restrict__ q_out,
                                                                  uint8_t* __restrict__ s_out,
                                                                  float* __restrict__ rstd_out) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (kMxThreads / kWave) + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wavefront; no barrier follows
  const int nch = (int)(K >> 3);  // a multiple of 8: a 64-block is 8 whole chunks
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + t * K);
  const u32x4* gr = GAMMA ? reinterpret_cast<const u32x4*>(gamma) : nullptr;

  float ss = 0.f;
  for (int base = 0; base < nch; base += kWave) {
    const int idx = base + lane;
    if (idx < nch) ss += sumsq8(xr[idx]);
  }
  const float rstd = rstd_from_sumsq(wave_sum(ss), inv_k, eps);
  if (lane == 0 && rstd_out != nullptr) rstd_out[t] = rstd;

  u32x2* qrow = reinterpret_cast<u32x2*>(q_out + t * K);
  uint8_t* srow = s_out + t * (K >> 6);
  for (int base = 0; base < nch; base += kWave) {
    const int idx = base + lane;
    const bool live = idx < nch;  // the same for all 8 lanes of a 64-block
    const u32x4 w = live ? xr[idx] : u32x4{0u, 0u, 0u, 0u};
    float n[8];
    normed8(w, gr, live ? idx : 0, rstd, n);
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(n[j]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 4, kWave));
    // floor(log2(amax)) is the exponent field of amax (a subnormal or zero amax
    // gives a field of 0, which the clamp turns into -127)
    const int ebits = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
    const int e = max(ebits - 127 - 8, -127);
    const float inv_x = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, exact
    uint32_t c[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j >> 2] |= e4m3_rne(n[j] * inv_x) << (8 * (j & 3));
    if (live) {
      qrow[idx] = u32x2{c[0], c[1]};
      if ((lane & 7) == 0) srow[idx >> 3] = (uint8_t)(e + 127);
    }
  }
}

}  // namespace

hipError_t launch_norm_rows_mx(const uint16_t* x, const uint16_t* gamma, float eps, int64_t T, int64_t K,
                               uint8_t* q_out, uint8_t* s_out, float* rstd_out, hipStream_t s) {
  const float inv_k = 1.0f / (float)K;
  const dim3 grid((unsigned)((T + 3) / 4)), block(kMxThreads);
  if (gamma != nullptr)
    hipLaunchKernelGGL(norm_rows_mx_kernel<true>, grid, block, 0, s, x, gamma, eps, inv_k, T, K, q_out, s_out,
                       rstd_out);
  else
    hipLaunchKernelGGL(norm_rows_mx_kernel<false>, grid, block, 0, s, x, gamma, eps, inv_k, T, K, q_out, s_out,
                       rstd_out);
  return hipGetLastError();
}

}  // namespace rnl
