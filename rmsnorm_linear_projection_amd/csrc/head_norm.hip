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
// Layout of the work: a head of D bf16 values is D/8 16-byte chunks, and lane
// i of the head's group of GP lanes (D/16 rounded up to a power of two) holds
// chunk i and chunk i + D/16, i.e. both members of every rotate-half pair it
// owns, so the rotation needs no data from other lanes and reads each angle
// once.  All loads (the two chunks, their gammas, the angles) are issued
// together.  The sum of squares is reduced inside the group with DPP moves;
// each chunk is written back by the lane that read it, so y_out may be y_in.
// The arithmetic (head_sumsq, group_sum, head_chunks) is shared with the
// projection GEMM's per-head epilogue, so both give the same bits.
#include <algorithm>

#include "launch.h"
#include "rows.hpp"

namespace rnl {
namespace {

constexpr int kHeadThreads = 256;

template <int GP, bool ROPE>
__global__ __launch_bounds__(kHeadThreads) void head_norm_kernel(
    const uint16_t* y_in, uint16_t* y_out, int64_t ld, int64_t col0, int64_t nheads_total, int H, int D,
    int H1, const uint16_t* __restrict__ gamma1, const uint16_t* __restrict__ gamma2, float eps, float inv_d,
    const float* __restrict__ cos_t, const float* __restrict__ sin_t, float* __restrict__ rstd_out) {
  constexpr int HPW = kWave / GP;  // heads per wavefront
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gl = lane & (GP - 1);
  // a two-axis grid (the x axis alone would overflow the 32-bit work-item count past 2^28 heads)
  const int64_t blk = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  const int64_t head = (blk * (kHeadThreads / kWave) + wave) * HPW + lane / GP;
  const int P = D >> 4;  // chunk pairs per head
  const bool live = head < nheads_total;
  const bool act = live && gl < P;
  // nheads_total = T * H < 2^31 (checked on the host): 32-bit division
  const uint32_t hu = live ? (uint32_t)head : 0u;
  const uint32_t tu = hu / (uint32_t)H;
  const int64_t t = (int64_t)tu;
  const int h = (int)(hu - tu * (uint32_t)H);
  const int64_t row = t * ld + col0 + (int64_t)h * D;
  const int c0 = gl * 8, c1 = (gl + P) * 8;  // first elements of the lane's two chunks
  const uint16_t* gamma = h < H1 ? gamma1 : gamma2;

  // Every lane loads unconditionally (inactive lanes from the first chunk of y,
  // always in bounds, and never store), so that all the loads are issued back
  // to back without branches between them.
  const int64_t e0 = act ? row + c0 : 0, e1 = act ? row + c1 : 0;
  const u32x4 v0 = *reinterpret_cast<const u32x4*>(y_in + e0);
  const u32x4 v1 = *reinterpret_cast<const u32x4*>(y_in + e1);
  const bool g_on = act && gamma != nullptr;
  const uint16_t* gsrc = g_on ? gamma : y_in;
  const u32x4 g0 = *reinterpret_cast<const u32x4*>(gsrc + (g_on ? c0 : 0));
  const u32x4 g1 = *reinterpret_cast<const u32x4*>(gsrc + (g_on ? c1 : 0));
  f32x4 cs[2], sn[2];
  if constexpr (ROPE) {
    const int64_t ab = act ? t * (int64_t)(D >> 1) + c0 : 0;  // angles of pair elements c0 .. c0 + 7
    cs[0] = *reinterpret_cast<const f32x4*>(cos_t + ab);
    cs[1] = *reinterpret_cast<const f32x4*>(cos_t + ab + 4);
    sn[0] = *reinterpret_cast<const f32x4*>(sin_t + ab);
    sn[1] = *reinterpret_cast<const f32x4*>(sin_t + ab + 4);
  }
  // lanes that own no chunk (past D/16, or past the last head) add nothing to their group's sum
  const float ss = act ? head_sumsq(v0, v1) : 0.f;
  const float rstd = rstd_from_sumsq(group_sum<GP>(ss), inv_d, eps);
  u32x4 o0, o1;
  head_chunks<ROPE>(v0, v1, g0, g1, g_on, cs, sn, rstd, o0, o1);
  if (act) {
    *reinterpret_cast<u32x4*>(y_out + row + c0) = o0;
    *reinterpret_cast<u32x4*>(y_out + row + c1) = o1;
    if (gl == 0 && rstd_out != nullptr) rstd_out[head] = rstd;
  }
}

}  // namespace

hipError_t launch_head_norm_bf16(const uint16_t* y_in, uint16_t* y_out, int64_t T, int64_t ld, int64_t col0,
                                 int64_t H, int64_t D, int64_t H1, const uint16_t* gamma1, const uint16_t* gamma2,
                                 float eps, const float* cos_t, const float* sin_t, float* rstd_out,
                                 hipStream_t s) {
  const int P = (int)(D / 16);  // lanes per head
  int gp = 1;
  while (gp < P) gp *= 2;
  const int64_t total = T * H;
  if (total > 0x7fffffff) return hipErrorInvalidValue;  // the kernel divides head indices in 32 bits
  const int64_t heads_per_block = (kHeadThreads / kWave) * (kWave / gp);
  const int64_t wgs = (total + heads_per_block - 1) / heads_per_block;
  const int64_t gx = std::min<int64_t>(wgs, int64_t(1) << 16);
  const dim3 grid((unsigned)gx, (unsigned)((wgs + gx - 1) / gx)), block(kHeadThreads);
  const float inv_d = 1.0f / (float)D;
  const bool rope = cos_t != nullptr;
#define RNL_HEAD(GP, R)                                                                                      \
  hipLaunchKernelGGL((head_norm_kernel<GP, R>), grid, block, 0, s, y_in, y_out, ld, col0, total, (int)H, \
                     (int)D, (int)H1, gamma1, gamma2, eps, inv_d, cos_t, sin_t, rstd_out)
#define RNL_HEAD_GP(GP) \
  if (rope) RNL_HEAD(GP, true); else RNL_HEAD(GP, false)
  switch (gp) {
    case 1: RNL_HEAD_GP(1); break;
    case 2: RNL_HEAD_GP(2); break;
    case 4: RNL_HEAD_GP(4); break;
    case 8: RNL_HEAD_GP(8); break;
    case 16: RNL_HEAD_GP(16); break;
    default: RNL_HEAD_GP(32); break;
  }
#undef RNL_HEAD_GP
#undef RNL_HEAD
  return hipGetLastError();
}

}  // namespace rnl
