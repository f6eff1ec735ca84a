// Row helpers shared by the norm kernels (the pre-pass, the per-head stage and
// the per-head epilogue of the projection GEMM).
#pragma once

#include "common.hpp"

namespace rnl {

// fp32 sum of the squares of 8 packed bf16 values
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

// normed values of one 8-element chunk: n = fl(fl(xf * rstd) * g), with gamma
// chunk idx of gr (no gamma when gr is null)
__device__ __forceinline__ void normed8(u32x4 w, const u32x4* gr, int idx, float rstd, float n[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    n[2 * j] = __fmul_rn(bf16lo(w[j]), rstd);
    n[2 * j + 1] = __fmul_rn(bf16hi(w[j]), rstd);
  }
  if (gr != nullptr) {
    u32x4 g = gr[idx];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      n[2 * j] = __fmul_rn(n[2 * j], bf16lo(g[j]));
      n[2 * j + 1] = __fmul_rn(n[2 * j + 1], bf16hi(g[j]));
    }
  }
}

// Sum over the GP lanes of a group (GP a power of two <= 32, groups aligned to
// GP lanes); every lane of the group ends with the same value.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

template <int GP>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (GP >= 2) v += dpp_f<0xB1>(v);   // quad_perm 1,0,3,2: lane ^ 1
  if constexpr (GP >= 4) v += dpp_f<0x4E>(v);   // quad_perm 2,3,0,1: lane ^ 2
  if constexpr (GP >= 8) v += dpp_f<0x141>(v);  // row_half_mirror: the two quads of 8 lanes
  if constexpr (GP >= 16) v += dpp_f<0x140>(v); // row_mirror: the two halves of 16 lanes
  if constexpr (GP >= 32) v += __shfl_xor(v, 16, kWave);
  return v;
}

// A lane's share of one head's sum of squares: its two 8-element chunks.
__device__ __forceinline__ float head_sumsq(u32x4 v0, u32x4 v1) {
#pragma clang fp contract(off)
  return sumsq8(v0) + sumsq8(v1);
}

// Head norm (+ rotate-half RoPE) of a lane's two chunks of one head: chunk v0
// holds elements i .. i+7 and v1 elements i+D/2 .. i+D/2+7, so every rotate-half
// pair is inside the lane.  n = fl(fl(y * rstd) * g) (no gamma when g_on is
// false), then, with ROPE, out[i] = fl(fl(n[i] c) - fl(n[i+D/2] s)) and
// out[i+D/2] = fl(fl(n[i+D/2] c) + fl(n[i] s)) with c, s = cs, sn of element i;
// results rounded to bf16.  Every product and sum is rounded on its own.
template <bool ROPE>
__device__ __forceinline__ void head_chunks(u32x4 v0, u32x4 v1, u32x4 g0, u32x4 g1, bool g_on, const f32x4 cs[2],
                                            const f32x4 sn[2], float rstd, u32x4& o0, u32x4& o1) {
#pragma clang fp contract(off)
  float n0[8], n1[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    n0[2 * j] = bf16lo(v0[j]) * rstd;
    n0[2 * j + 1] = bf16hi(v0[j]) * rstd;
    n1[2 * j] = bf16lo(v1[j]) * rstd;
    n1[2 * j + 1] = bf16hi(v1[j]) * rstd;
  }
  if (g_on) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      n0[2 * j] = n0[2 * j] * bf16lo(g0[j]);
      n0[2 * j + 1] = n0[2 * j + 1] * bf16hi(g0[j]);
      n1[2 * j] = n1[2 * j] * bf16lo(g1[j]);
      n1[2 * j + 1] = n1[2 * j + 1] * bf16hi(g1[j]);
    }
  }
  if constexpr (ROPE) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float c = cs[e >> 2][e & 3], s = sn[e >> 2][e & 3];
      const float lo = n0[e] * c - n1[e] * s;  // element i
      const float hi = n1[e] * c + n0[e] * s;  // element i + D/2
      n0[e] = lo;
      n1[e] = hi;
    }
  }
  o0 = u32x4{pack_bf16x2(n0[0], n0[1]), pack_bf16x2(n0[2], n0[3]), pack_bf16x2(n0[4], n0[5]), pack_bf16x2(n0[6], n0[7])};
  o1 = u32x4{pack_bf16x2(n1[0], n1[1]), pack_bf16x2(n1[2], n1[3]), pack_bf16x2(n1[4], n1[5]), pack_bf16x2(n1[6], n1[7])};
}

}  // namespace rnl
