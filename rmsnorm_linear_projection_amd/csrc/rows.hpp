// Row helpers shared by the norm kernels (the pre-pass and the per-head stage).
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

}  // namespace rnl
