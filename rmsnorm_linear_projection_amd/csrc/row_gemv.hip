// One- and two-token RMSNorm -> projection (decode at T <= 2) for gfx950.
//
// What it computes is the fused RMSNorm -> Linear of the AT-10 page (compute
// flow, section 2; the AT-03 norm of section 3; bf16 operands with the weight
// stored [N, K], section 4) for each of the M <= 2 activation rows:
//   rstd = 1 / sqrt(fl(fl(S / K) + eps)),  S = fp32 sum of x[k]^2,
//   a[k] = bf16(fl(fl(x[k] * rstd) * gamma[k])),
//   y[n] = sum_k a[k] * W[n, k]  (fp32 accumulation, then bf16 or fp32).
//
// One output row is a dot product of K bf16 pairs, so the weight read is the
// whole cost (HBM-bound).  Layout of the work:
//   * wavefront v (four to a workgroup, which share nothing) owns RW
//     consecutive weight rows (RW is a template argument: rows past N are
//     skipped by the buffer resource, but rows the wavefront never uses would
//     still cost load slots and registers);
//   * lane l owns the 16-byte chunks c * 64 + l (c < KC) of every row, so each
//     load instruction reads 1 KiB of one row, contiguous; all RW x KC weight
//     chunks are requested at once, right after the wavefront's share of the
//     token row and gamma;
//   * the four wavefronts of a workgroup share the norm of each token row:
//     wavefront v loads the
//     chunks c = v, v + 4, ... of x and gamma, the four partial sums of squares
//     meet in LDS and are added in a fixed order, and each wavefront writes its
//     normed chunks of a to LDS, from which every wavefront reads the whole
//     row (wavefronts with no weight rows past N still take part);
//   * the products run on the VALU (v_dot2c_f32_bf16: two bf16 products added
//     to an fp32 accumulator per instruction); one token needs no matrix core;
//   * with a residual (the pre-attention add of the AT-10 page, section 6) each
//     chunk of x is first replaced by x_add = bf16(float(x) + float(residual)),
//     rounded to nearest even -- the value the norm pre-pass forms -- and the
//     wavefronts of workgroup 0 write x_add out;
//   * each output's 64 lane partials are summed across the wavefront (DPP, no
//     LDS) and lane t * RW + r stores token t's output r.  Measured at K = 4096,
//     N = 6144: 10.1 us at T = 1, 11.4 at T = 2 (against 12.5 for the MFMA
//     kernel); at T = 3 and 4 (13.5, 14.0 against 12.4) the MFMA kernel stays.
// Rows past N and chunks past K read as zero through the buffer resource.
#include "common.hpp"
#include "launch.h"

namespace rnl {
namespace {

// fp32 dot product of 8 bf16 pairs, added to acc (element copies go through a
// scalar before the bit cast: a cast of a vector element reference reads
// element 0)
__device__ __forceinline__ float dot8(u32x4 w, u32x4 a, float acc) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t wj = w[j], aj = a[j];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wj), __builtin_bit_cast(bf16x2, aj), acc,
                                          false);
  }
  return acc;
}

// bf16(float(x) + float(r)) for 8 elements
__device__ __forceinline__ u32x4 add8(u32x4 x, u32x4 r) {
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = pack_bf16x2(__fadd_rn(bf16lo(x[j]), bf16lo(r[j])), __fadd_rn(bf16hi(x[j]), bf16hi(r[j])));
  return o;
}

// a = bf16(fl(fl(x * rstd) * g)) for 8 elements (g = 1 without gamma)
template <bool GAMMA>
__device__ __forceinline__ u32x4 norm8(u32x4 x, u32x4 g, float rstd) {
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float lo = __fmul_rn(bf16lo(x[j]), rstd), hi = __fmul_rn(bf16hi(x[j]), rstd);
    if constexpr (GAMMA) {
      lo = __fmul_rn(lo, bf16lo(g[j]));
      hi = __fmul_rn(hi, bf16hi(g[j]));
    }
    o[j] = pack_bf16x2(lo, hi);
  }
  return o;
}

__device__ __forceinline__ float sumsq8(u32x4 w) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a = bf16lo(w[j]), b = bf16hi(w[j]);
    s += a * a;
    s += b * b;
  }
  return s;
}

// the sum of v over the 64 lanes, on every lane: DPP adds within rows of 16
// lanes, two row broadcasts carry the partial sums up to lane 63, which is
// read out.  No LDS round trips, so the sums of several rows interleave.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ float wave_total(float v) {
  v = dpp_add<0xB1, 0xF>(v);   // quad_perm 1,0,3,2: lane ^ 1
  v = dpp_add<0x4E, 0xF>(v);   // quad_perm 2,3,0,1: lane ^ 2
  v = dpp_add<0x141, 0xF>(v);  // row_half_mirror: the two quads of 8 lanes
  v = dpp_add<0x140, 0xF>(v);  // row_mirror: the two halves of 16 lanes
  v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3: rows 0+1 and 2+3
  v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3: lane 63 holds all four
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// KC: 16-byte chunks per lane and row (K <= 512 * KC); RW: rows per wavefront
template <int MT, int KC, int RW>
__global__ __launch_bounds__(256) void row_gemv_norm_kernel(const uint16_t* __restrict__ X,
                                                           const uint16_t* __restrict__ residual,
                                                           uint16_t* __restrict__ x_add,
                                                           const uint16_t* __restrict__ gamma, float eps,
                                                           float inv_k, const uint16_t* __restrict__ W,
                                                           void* __restrict__ C, bool out_bf16,
                                                           float* __restrict__ rstd_out, int M, int K, int N) {
  constexpr int XC = (KC + 3) / 4;  // chunks of x and gamma each wavefront norms
  __shared__ u32x4 as[MT * KC * 64];  // normed rows: token t, chunk c of lane l at (t * KC + c) * 64 + l
  __shared__ float red[MT][4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wv = blockIdx.x * 4 + wave;
  const int n0 = wv * RW;
  const int rows = n0 < N ? min(RW, N - n0) : 0;  // 0: the wavefront only helps with the norm
  const bool has_g = gamma != nullptr;
  const bool has_r = residual != nullptr;
  const uint32_t kbytes = (uint32_t)K * 2u;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, (uint32_t)M * kbytes);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(has_g ? gamma : X, has_g ? kbytes : 0u);
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(has_r ? residual : X, has_r ? (uint32_t)M * kbytes : 0u);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + (size_t)min(n0, N - 1) * K, (uint32_t)rows * kbytes);

  u32x4 xv[MT][XC], gv[XC], w[RW][KC];
#pragma unroll
  for (int i = 0; i < XC; ++i) {
    const int c = wave + 4 * i;
    const uint32_t o = (uint32_t)(c * 64 + lane) * 16u;
    const bool in = c < KC && o < kbytes;
#pragma unroll
    for (int t = 0; t < MT; ++t) xv[t][i] = buf_load16(rx, (in && t < M) ? o + (uint32_t)t * kbytes : kOOB);
    gv[i] = buf_load16(rg, in ? o : kOOB);  // zeros without gamma (an empty resource), not used then
  }
  u32x4 rv[MT][XC];
  if (has_r) {
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      const int c = wave + 4 * i;
      const uint32_t o = (uint32_t)(c * 64 + lane) * 16u;
      const bool in = c < KC && o < kbytes;
#pragma unroll
      for (int t = 0; t < MT; ++t) rv[t][i] = buf_load16(rr, (in && t < M) ? o + (uint32_t)t * kbytes : kOOB);
    }
  }
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const uint32_t o = (uint32_t)(c * 64 + lane) * 16u;
      w[r][c] = buf_load16(rw, (o < kbytes && r < rows) ? o + (uint32_t)r * kbytes : kOOB);
    }
  // keep every load above issued before the norm arithmetic waits on the first
  __builtin_amdgcn_sched_barrier(0);

  if (has_r) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int i = 0; i < XC; ++i) {
        xv[t][i] = add8(xv[t][i], rv[t][i]);
        const int c = wave + 4 * i;
        const uint32_t o = (uint32_t)(c * 64 + lane) * 16u;
        if (blockIdx.x == 0 && t < M && c < KC && o < kbytes)
          *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(x_add) + (size_t)t * kbytes + o) = xv[t][i];
      }
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < XC; ++i) ss += sumsq8(xv[t][i]);
    ss = wave_total(ss);
    if (lane == 0) red[t][wave] = ss;
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const float S = (red[t][0] + red[t][1]) + (red[t][2] + red[t][3]);
    const float rstd = rstd_from_sumsq(S, inv_k, eps);
    if (wv == 0 && lane == 0 && t < M && rstd_out != nullptr) rstd_out[t] = rstd;
#pragma unroll
    for (int i = 0; i < XC; ++i) {
      const int c = wave + 4 * i;
      if (c < KC)
        as[(t * KC + c) * 64 + lane] =
            has_g ? norm8<true>(xv[t][i], gv[i], rstd) : norm8<false>(xv[t][i], gv[i], rstd);
    }
  }
  __syncthreads();
  if (rows == 0) return;  // after the last barrier

  float acc[MT][RW];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int r = 0; r < RW; ++r) acc[t][r] = 0.f;
#pragma unroll
  for (int c = 0; c < KC; ++c)
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const u32x4 a = as[(t * KC + c) * 64 + lane];
#pragma unroll
      for (int r = 0; r < RW; ++r) acc[t][r] = dot8(w[r][c], a, acc[t][r]);
    }
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    if (t >= M) break;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      if (r >= rows) break;
      const float v = wave_total(acc[t][r]);
      if (lane == t * RW + r) {
        const size_t o = (size_t)t * (size_t)N + (size_t)(n0 + r);
        if (out_bf16)
          static_cast<uint16_t*>(C)[o] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xFFFFu);
        else
          static_cast<float*>(C)[o] = v;
      }
    }
  }
}

// Most rows per wavefront for KC chunks per lane and row (K = 512 * KC).
// Measured at T = 1 (rotated weights, same box): K = 1536, N = 24576: RW = 4
// 14.0 us, 6 14.7, 8 15.0; K = 2048, N = 4096: 4 rows 5.0 us against 6.6 at 2;
// K = 512, N = 4096: 4 rows 3.3 us, 8 rows 3.9; K = 4096, N = 6144: 3 rows
// 11.0 us, 2 rows 12.2.  Past 8 chunks the cap keeps the weight registers
// near 24 chunks (96 VGPRs).  With the norm shared through LDS the registers
// would allow more, but caps of 4, 3 and 2 rows up to 8, 12 and 16 chunks were
// slower: K = 4096, N = 6144 11.0 us against 10.1.
constexpr int rw_cap(int kc) { return kc <= 6 ? 4 : kc <= 8 ? 3 : kc <= 12 ? 2 : 1; }

}  // namespace

bool row_gemv_fits(int64_t M, int64_t K) { return M >= 1 && M <= kRowGemvMaxM && K >= 8 && K <= kRowGemvMaxK; }

int row_gemv_rows(int64_t N, int kc) {
  const int64_t rw = (N + kRowGemvWaves - 1) / kRowGemvWaves;
  const int cap = rw_cap(kc);
  return (int)(rw < cap ? rw : cap);
}

hipError_t launch_row_gemv_norm_bf16(const uint16_t* X, const uint16_t* residual, uint16_t* x_add,
                                     const uint16_t* gamma, float eps, const uint16_t* W, void* C, int out_kind,
                                     float* rstd_out, int64_t M, int64_t N, int64_t K, hipStream_t s) {
  if ((residual == nullptr) != (x_add == nullptr)) return hipErrorInvalidValue;
  if (!row_gemv_fits(M, K) || N < 1 || N > 0x7fffffff) return hipErrorInvalidValue;
  const int mt = M <= 1 ? 1 : 2;
  const int kc = (int)((K + 511) / 512);
  const bool ob = out_kind == OUT_BF16;
  const float inv_k = 1.0f / (float)K;
  const int rw = row_gemv_rows(N, kc);
  const int64_t waves = (N + rw - 1) / rw;
  const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
#define RNL_ROW_GEMV1(MT, KC, RW)                                                                           \
  hipLaunchKernelGGL((row_gemv_norm_kernel<MT, KC, RW>), grid, block, 0, s, X, residual, x_add, gamma, eps,     \
                     inv_k, W, C, ob,                                                                         \
                     rstd_out, (int)M, (int)K, (int)N)
#define RNL_ROW_GEMV(KC, RW)                                     \
  do {                                                           \
    if (mt == 1) RNL_ROW_GEMV1(1, KC, RW);                       \
    else RNL_ROW_GEMV1(2, KC, RW);                               \
  } while (0)
#define RNL_ROW_GEMV_KC(KC)                                                          \
  case KC:                                                                           \
    if (rw == 1) RNL_ROW_GEMV(KC, 1);                                                \
    else if constexpr (rw_cap(KC) >= 2) {                                            \
      if (rw == 2) RNL_ROW_GEMV(KC, 2);                                              \
      else if constexpr (rw_cap(KC) >= 3) {                                          \
        if (rw == 3) RNL_ROW_GEMV(KC, 3);                                            \
        else if constexpr (rw_cap(KC) >= 4) RNL_ROW_GEMV(KC, 4);                     \
      }                                                                              \
    }                                                                                \
    break
  switch (kc) {
    RNL_ROW_GEMV_KC(1); RNL_ROW_GEMV_KC(2); RNL_ROW_GEMV_KC(3); RNL_ROW_GEMV_KC(4);
    RNL_ROW_GEMV_KC(5); RNL_ROW_GEMV_KC(6); RNL_ROW_GEMV_KC(7); RNL_ROW_GEMV_KC(8);
    RNL_ROW_GEMV_KC(9); RNL_ROW_GEMV_KC(10); RNL_ROW_GEMV_KC(11); RNL_ROW_GEMV_KC(12);
    RNL_ROW_GEMV_KC(13); RNL_ROW_GEMV_KC(14); RNL_ROW_GEMV_KC(15); RNL_ROW_GEMV_KC(16);
    default: return hipErrorInvalidValue;
  }
#undef RNL_ROW_GEMV_KC
#undef RNL_ROW_GEMV
#undef RNL_ROW_GEMV1
  return hipGetLastError();
}

}  // namespace rnl
