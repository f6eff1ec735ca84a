// RMSNorm + MX quantisation pre-pass for the MXFP8 projection (gfx950).
//
// AT-10 with AT-09's MXFP8 mode: the fp32 normed rows are cut into blocks of 64
// consecutive values; each block gets one E8M0 scale X = 2^e with
// e = floor(log2(amax)) - 8 (8 is the largest exponent of E4M3; e clamped to
// [-127, 127]; an all-zero block takes e = -127), and each value becomes the
// E4M3 code nearest to n / X (ties to the even mantissa, magnitudes beyond 448
// clamped to 448, a zero result encoded as +0).
//
// One wavefront per row.  Rows of up to 64 * 8 * CPL values are loaded once
// into registers (all CPL 16-byte loads of a lane in flight together); longer
// rows (CPL = 0) are streamed twice, the second time from cache.  The fp32 sum
// of squares is a wavefront reduction; each 8-value chunk is then normed, and
// the 8 lanes that hold one 64-block exchange their maxima with DPP moves.
// Every lane runs the same number of iterations, so the cross-lane moves never
// run in divergent code.
#include "launch.h"
#include "rows.hpp"

namespace rnl {
namespace {

constexpr int kMxThreads = 256;

// Four E4M3 codes (nearest even) of v[0..3], packed low byte first.  The values
// are first clamped to +-448 (the largest E4M3 value, so the conversion never
// overflows); v_cvt_pk_fp8_f32 then rounds to nearest even, subnormals included.
// A negative value that rounds to zero comes out as 0x80 (-0); it is turned
// into +0, the code the reading of the pages takes for any zero.
__device__ __forceinline__ uint32_t e4m3x4(const float* v) {
  float c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) c[j] = fminf(fmaxf(v[j], -448.0f), 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w, true);
  const uint32_t u = (uint32_t)w;
  // bytes equal to 0x80: t has a zero byte there
  const uint32_t t = u ^ 0x80808080u;
  const uint32_t zero = ~(((t & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | t) & 0x80808080u;
  return u & ~zero;
}

// max over the 8 lanes 8q .. 8q+7 (DPP: swap neighbours, swap pairs, mirror the half-row)
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true)));   // quad_perm 1,0,3,2
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true)));   // quad_perm 2,3,0,1
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true)));  // row_half_mirror
  return v;
}

// MX-quantise the 8 normed values of chunk idx (8 lanes hold one 64-block)
__device__ __forceinline__ void mx_emit(const float n[8], bool live, int idx, int lane, u32x2* qrow, uint8_t* srow) {
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(n[j]));
  amax = max8(amax);
  // floor(log2(amax)) is the exponent field of amax (a subnormal or zero amax
  // gives a field of 0, which the clamp turns into -127)
  const int ebits = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  const int e = max(ebits - 127 - 8, -127);
  const float inv_x = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, exact
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = n[j] * inv_x;
  if (live) {
    qrow[idx] = u32x2{e4m3x4(v), e4m3x4(v + 4)};
    if ((lane & 7) == 0) srow[idx >> 3] = (uint8_t)(e + 127);
  }
}

template <int CPL, bool GAMMA>
__global__ __launch_bounds__(kMxThreads) void norm_rows_mx_kernel(const uint16_t* __restrict__ x,
                                                                  const uint16_t* __restrict__ gamma, float eps,
                                                                  float inv_k, int64_t T, int64_t K,
                                                                  uint8_t* __restrict__ q_out,
                                                                  uint8_t* __restrict__ s_out,
                                                                  float* __restrict__ rstd_out) {
  const int lane = threadIdx.x & 63;
  // the row index is wavefront-uniform: readfirstlane keeps the row's buffer resource in scalar registers
  const int64_t t = (int64_t)blockIdx.x * (kMxThreads / kWave) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= T) return;  // whole wavefront; no barrier follows
  const int nch = (int)(K >> 3);  // a multiple of 8: a 64-block is 8 whole chunks
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + t * K);
  const u32x4* gr = GAMMA ? reinterpret_cast<const u32x4*>(gamma) : nullptr;
  u32x2* qrow = reinterpret_cast<u32x2*>(q_out + t * K);
  uint8_t* srow = s_out + t * (K >> 6);

  if constexpr (CPL > 0) {
    // x and gamma chunks all requested up front (buffer loads: chunks past K read as
    // zero); the stores of the normed codes then never wait on a gamma load
    const uint32_t kb = (uint32_t)K * 2u;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + t * K, kb);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(gamma, GAMMA ? kb : 0u);
    u32x4 v[CPL], gv[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const uint32_t o = (uint32_t)(lane + kWave * c) * 16u;
      v[c] = buf_load16(rx, o);
      if constexpr (GAMMA) gv[c] = buf_load16(rg, o);
    }
    __builtin_amdgcn_sched_barrier(0);  // the gamma loads stay in flight with the row's
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) ss += sumsq8(v[c]);
    const float rstd = rstd_from_sumsq(wave_sum(ss), inv_k, eps);
    if (lane == 0 && rstd_out != nullptr) rstd_out[t] = rstd;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int idx = lane + kWave * c;
      float n[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        n[2 * j] = __fmul_rn(bf16lo(v[c][j]), rstd);
        n[2 * j + 1] = __fmul_rn(bf16hi(v[c][j]), rstd);
        if constexpr (GAMMA) {
          n[2 * j] = __fmul_rn(n[2 * j], bf16lo(gv[c][j]));
          n[2 * j + 1] = __fmul_rn(n[2 * j + 1], bf16hi(gv[c][j]));
        }
      }
      mx_emit(n, idx < nch, idx, lane, qrow, srow);
    }
  } else {
    float ss = 0.f;
    for (int base = 0; base < nch; base += kWave) {
      const int idx = base + lane;
      if (idx < nch) ss += sumsq8(xr[idx]);
    }
    const float rstd = rstd_from_sumsq(wave_sum(ss), inv_k, eps);
    if (lane == 0 && rstd_out != nullptr) rstd_out[t] = rstd;
    for (int base = 0; base < nch; base += kWave) {
      const int idx = base + lane;
      const bool live = idx < nch;
      const u32x4 w = live ? xr[idx] : u32x4{0u, 0u, 0u, 0u};
      float n[8];
      normed8(w, gr, live ? idx : 0, rstd, n);
      mx_emit(n, live, idx, lane, qrow, srow);
    }
  }
}

}  // namespace

hipError_t launch_norm_rows_mx(const uint16_t* x, const uint16_t* gamma, float eps, int64_t T, int64_t K,
                               uint8_t* q_out, uint8_t* s_out, float* rstd_out, hipStream_t s) {
  const float inv_k = 1.0f / (float)K;
  const dim3 grid((unsigned)((T + 3) / 4)), block(kMxThreads);
  const int64_t per = (K / 8 + kWave - 1) / kWave;  // chunks per lane
#define RNL_MX(C, G)                                                                                          \
  hipLaunchKernelGGL((norm_rows_mx_kernel<C, G>), grid, block, 0, s, x, gamma, eps, inv_k, T, K, q_out, s_out, \
                     rstd_out)
#define RNL_MX_G(C) \
  if (gamma != nullptr) RNL_MX(C, true); else RNL_MX(C, false)
  if (per <= 1) RNL_MX_G(1);
  else if (per <= 2) RNL_MX_G(2);
  else if (per <= 4) RNL_MX_G(4);
  else if (per <= 8) RNL_MX_G(8);
  else if (per <= 16) RNL_MX_G(16);
  else RNL_MX_G(0);
#undef RNL_MX_G
#undef RNL_MX
  return hipGetLastError();
}

}  // namespace rnl
