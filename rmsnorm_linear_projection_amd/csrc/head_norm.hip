// Per-head RMSNorm and rotary embedding after the projection (gfx950).
//
// The fused QKV output y[T, ld] holds, from column col0 on, H heads of D
// columns each.  Every head is normed on its own: S = sum of its D squares in
// fp32, rstd = 1/sqrt(fl(fl(S * fl(1/D)) + eps)), n = fl(fl(y * rstd) * gamma)
// (heads h < H1 take gamma1, the others gamma2, so one launch covers the query
// and the key heads), then, when angle tables are given, rotated by the
// rotate-half RoPE in fp32:
//   out[i]       = fl(fl(n[i] c[i])       - fl(n[i + D/2] s[i]))
//   out[i + D/2] = fl(fl(n[i + D/2] c[i]) + fl(n[i] s[i]))
// with c, s = cos[t, i], sin[t, i] (i < D/2), and rounded to bf16.  Every
// product and sum is rounded on its own (the rotation is written with plain
// operators under contract(off), so no FMA is formed), and the result is a
// fixed function of the fp32 rstd.
//
// Layout of the work: a head of D bf16 values is D/8 16-byte chunks, one per
// lane; a group of GP lanes (D/8 rounded up to a power of two) takes one head,
// so a wavefront takes 64/GP heads at once.  The sum of squares is reduced
// with xor shuffles inside the group; the RoPE partner chunk (i + D/2 for the
// first half, i - D/2 for the second) comes from the partner lane by a
// shuffle, so every chunk is read from memory once, by the lane that writes
// it back -- y_out may therefore be y_in.
#include "launch.h"
#include "rows.cuh"

namespace rnl {
namespace {

constexpr int kHeadThreads = 256;

template <int GP, bool ROPE>
__global__ __launch_bounds__(kHeadThreads) void head_norm_kernel(
    const uint16_t* y_in, uint16_t* y_out, int64_t ld, int64_t col0, int64_t nheads_total, int H, int D,
    int H1, const uint16_t* __restrict__ gamma1, const uint16_t* __restrict__ gamma2, float eps, float inv_d,
    const float* __restrict__ cos_t, const float* __restrict__ sin_t, float* __restrict__ rstd_out) {
#pragma clang fp contract(off)
  constexpr int HPW = kWave / GP;  // heads per wavefront
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gl = lane & (GP - 1);
  const int64_t head = ((int64_t)blockIdx.x * (kHeadThreads / kWave) + wave) * HPW + lane / GP;
  const int G = D >> 3;  // chunks per head
  const bool live = head < nheads_total;
  const bool act = live && gl < G;
  const int64_t t = live ? head / H : 0;
  const int h = live ? (int)(head - t * H) : 0;
  const uint16_t* row_in = y_in + t * ld + col0 + (int64_t)h * D;

  u32x4 v = act ? *reinterpret_cast<const u32x4*>(row_in + gl * 8) : u32x4{0u, 0u, 0u, 0u};
  float ss = sumsq8(v);
#pragma unroll
  for (int off = GP / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, kWave);
  const float rstd = rstd_from_sumsq(ss, inv_d, eps);
  const u32x4* gr = reinterpret_cast<const u32x4*>(h < H1 ? gamma1 : gamma2);

  float n[8];
  normed8(v, gr, act ? gl : 0, rstd, n);
  if constexpr (ROPE) {
    // partner chunk of the rotate-half pairing, fetched from its lane
    const int half = G >> 1;
    const int partner = gl < half ? gl + half : gl - half;
    const int src = (lane & ~(GP - 1)) + (gl < G ? partner : gl);
    u32x4 pv;
#pragma unroll
    for (int j = 0; j < 4; ++j) pv[j] = (uint32_t)__shfl((int)v[j], src, kWave);
    float pn[8];
    normed8(pv, gr, act ? partner : 0, rstd, pn);
    if (act) {
      const int64_t ab = t * (int64_t)(D >> 1) + (int64_t)(gl < half ? gl : gl - half) * 8;
      const f32x4 c0 = *reinterpret_cast<const f32x4*>(cos_t + ab);
      const f32x4 c1 = *reinterpret_cast<const f32x4*>(cos_t + ab + 4);
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(sin_t + ab);
      const f32x4 s1 = *reinterpret_cast<const f32x4*>(sin_t + ab + 4);
      const float c[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
      const float s[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
      const bool first = gl < half;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float a = n[e] * c[e];
        const float b = pn[e] * s[e];
        n[e] = first ? a - b : a + b;
      }
    }
  }
  if (act) {
    uint16_t* row_out = y_out + t * ld + col0 + (int64_t)h * D;
    *reinterpret_cast<u32x4*>(row_out + gl * 8) =
        u32x4{pack_bf16x2(n[0], n[1]), pack_bf16x2(n[2], n[3]), pack_bf16x2(n[4], n[5]), pack_bf16x2(n[6], n[7])};
    if (gl == 0 && rstd_out != nullptr) rstd_out[head] = rstd;
  }
}

}  // namespace

hipError_t launch_head_norm_bf16(const uint16_t* y_in, uint16_t* y_out, int64_t T, int64_t ld, int64_t col0,
                                 int64_t H, int64_t D, int64_t H1, const uint16_t* gamma1, const uint16_t* gamma2,
                                 float eps, const float* cos_t, const float* sin_t, float* rstd_out,
                                 hipStream_t s) {
  const int G = (int)(D / 8);
  int gp = 8;
  while (gp < G) gp *= 2;
  const int64_t total = T * H;
  const int64_t heads_per_block = (kHeadThreads / kWave) * (kWave / gp);
  const dim3 grid((unsigned)((total + heads_per_block - 1) / heads_per_block)), block(kHeadThreads);
  const float inv_d = 1.0f / (float)D;
  const bool rope = cos_t != nullptr;
#define RNL_HEAD(GP, R)                                                                                      \
  hipLaunchKernelGGL((head_norm_kernel<GP, R>), grid, block, 0, s, y_in, y_out, ld, col0, total, (int)H, \
                     (int)D, (int)H1, gamma1, gamma2, eps, inv_d, cos_t, sin_t, rstd_out)
#define RNL_HEAD_GP(GP) \
  if (rope) RNL_HEAD(GP, true); else RNL_HEAD(GP, false)
  switch (gp) {
    case 8: RNL_HEAD_GP(8); break;
    case 16: RNL_HEAD_GP(16); break;
    case 32: RNL_HEAD_GP(32); break;
    default: RNL_HEAD_GP(64); break;
  }
#undef RNL_HEAD_GP
#undef RNL_HEAD
  return hipGetLastError();
}

}  // namespace rnl
