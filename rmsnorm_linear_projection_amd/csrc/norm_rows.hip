// Row-wise RMSNorm pre-pass for the large-T GEMM paths (gfx950).
//
// Rows of up to 8192 values, at least 256 of them or shorter than 2048: one
// wavefront per row (shuffle reductions only).  Longer rows, or fewer rows than
// CUs: one 256-thread workgroup per row, the row read once with 16-byte
// coalesced loads (kept in registers when K <= 16384) and the fp32 sum of
// squares reduced across the wavefronts.  The normed row is written either as
// bf16 (the A operand of the bf16 GEMM) or as per-token symmetric int8 plus
// its dequant scale (the A operand of the int8 GEMM).
//
// Arithmetic (AT-10 page, section 3, variant B; AT-10 page section 4, AT-05):
//   S = sum_k xf^2 (fp32, any order), rstd = 1/sqrt(fl(fl(S*fl(1/K)) + eps)),
//   n = fl(fl(xf * rstd) * gamma), bf16 out = round_nearest_even(n);
//   int8: amax = max|n|, s = fl(127/amax), q = clamp(rint(fl(n*s)), -127, 127),
//   x_scale = fl(amax/127); an all-zero row gives q = 0, x_scale = 0.
//
// The row may also be the bf16 rounding of the sum of split-K partial rows of
// a preceding projection (the q_a -> norm step of the low-rank chain): the
// partials are added in split order, so the result does not depend on timing.
#include <algorithm>

#include "launch.h"
#include "rows.hpp"

namespace rnl {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

// Four int8 codes q = clamp(rint(fl(n * s)), -127, 127), packed little-endian.
// With s = fl(127/amax) and |n| <= amax, |fl(n * s)| <= 127 + 2^-17, so the
// clamp never binds and rint is all that is left: adding 1.5 * 2^23 rounds the
// product to the nearest integer, ties to even (floats in [2^23, 2^24) are
// spaced 1 apart), and the low byte of the sum's bit pattern is that integer's
// two's-complement byte.  v_perm gathers the four bytes.  (s = +inf, for amax
// below 127 / FLT_MAX, would give 0 instead of +-127; rows with such an amax
// need denormal inputs.)
__device__ __forceinline__ uint32_t q4(const float n[8], int base, float s) {
#pragma clang fp contract(off)
  constexpr float kRound = 12582912.0f;  // 1.5 * 2^23
  uint32_t b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = __float_as_uint(n[base + j] * s + kRound);
  // perm selector bytes 0-3 pick bytes of the second operand, 4-7 of the first, 0x0c gives 0
  return __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u) | __builtin_amdgcn_perm(b[3], b[2], 0x04000c0cu);
}

// x + residual for 8 packed bf16 pairs: each sum in fp32 (one rounding), then
// rounded to bf16 (nearest even) -- the residual-add reading of the AT-10 page,
// section 6 (the norm reads the bf16 sum, which is also written back).
__device__ __forceinline__ u32x4 add_bf16x8(u32x4 a, u32x4 b) {
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    r[j] = pack_bf16x2(__fadd_rn(bf16lo(a[j]), bf16lo(b[j])), __fadd_rn(bf16hi(a[j]), bf16hi(b[j])));
  return r;
}

// normed8 with the gamma chunk already loaded (g is ignored when has_g is false)
__device__ __forceinline__ void normed8g(u32x4 w, u32x4 g, bool has_g, float rstd, float n[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    n[2 * j] = __fmul_rn(bf16lo(w[j]), rstd);
    n[2 * j + 1] = __fmul_rn(bf16hi(w[j]), rstd);
  }
  if (has_g) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      n[2 * j] = __fmul_rn(n[2 * j], bf16lo(g[j]));
      n[2 * j + 1] = __fmul_rn(n[2 * j + 1], bf16hi(g[j]));
    }
  }
}

// Row sources: chunk idx (8 consecutive elements, packed bf16) of row t.
// keep(t, idx, v) is called once per chunk in the first pass over the row.
struct RowBf16 {
  const uint16_t* x;  // row t at x + t * ld, K bf16 values
  int64_t ld;
  __device__ u32x4 operator()(int64_t t, int idx) const {
    return reinterpret_cast<const u32x4*>(x + t * ld)[idx];
  }
  __device__ void keep(int64_t, int, u32x4) const {}
};
struct RowAddBf16 {
  const uint16_t* x;  // [T, K] bf16
  const uint16_t* r;  // [T, K] bf16 residual
  uint16_t* x_add;    // [T, K] bf16: x + r, written in the first pass
  int64_t K;
  __device__ u32x4 operator()(int64_t t, int idx) const {
    return add_bf16x8(reinterpret_cast<const u32x4*>(x + t * K)[idx], reinterpret_cast<const u32x4*>(r + t * K)[idx]);
  }
  __device__ void keep(int64_t t, int idx, u32x4 v) const { reinterpret_cast<u32x4*>(x_add + t * K)[idx] = v; }
};
struct RowPartials {
  const float* part;  // slice z, row t at part + z * TK + t * ld
  int64_t TK;         // slice stride
  int64_t ld;         // row stride
  int S;
  uint16_t* sum_out;  // when not null, the bf16 row sums go to row t at sum_out + t * sum_ld
  int64_t sum_ld;
  __device__ u32x4 operator()(int64_t t, int idx) const {
    f32x4 lo = {0.f, 0.f, 0.f, 0.f}, hi = lo;
    for (int z = 0; z < S; ++z) {
      const f32x4* p = reinterpret_cast<const f32x4*>(part + (size_t)z * (size_t)TK + (size_t)t * (size_t)ld) + 2 * idx;
      lo += p[0];
      hi += p[1];
    }
    return u32x4{pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                 pack_bf16x2(hi[2], hi[3])};
  }
  __device__ void keep(int64_t t, int idx, u32x4 v) const {
    if (sum_out != nullptr) reinterpret_cast<u32x4*>(sum_out + t * sum_ld)[idx] = v;
  }
};

// CPT > 0: each thread keeps CPT 16-byte chunks of the row in registers.
// CPT == 0: the row is re-read (re-derived) for each pass.
// One row t, the whole workgroup (red: four floats of LDS for the reductions).
template <int CPT, bool INT8, class Row>
__device__ __forceinline__ void norm_row(Row row, const uint16_t* __restrict__ gamma, float eps, float inv_k,
                                         int64_t K, void* __restrict__ out, float* __restrict__ x_scale_out,
                                         float* __restrict__ rstd_out, int64_t t, float* red) {
  const int tid = threadIdx.x;
  const int nch = (int)(K >> 3);
  const u32x4* gr = reinterpret_cast<const u32x4*>(gamma);

  constexpr int NV = CPT > 0 ? CPT : 1;
  u32x4 v[NV], gv[NV];
  const bool has_g = gamma != nullptr;
  float ss = 0.f;
  if constexpr (CPT > 0) {
    // the gamma chunks are requested with the row's, not after the reduction
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * kThreads;
      v[c] = idx < nch ? row(t, idx) : u32x4{0u, 0u, 0u, 0u};
      gv[c] = (has_g && idx < nch) ? gr[idx] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int idx = tid + c * kThreads;
      if (idx < nch) row.keep(t, idx, v[c]);
      ss += sumsq8(v[c]);
    }
  } else {
    for (int idx = tid; idx < nch; idx += kThreads) {
      const u32x4 w = row(t, idx);
      row.keep(t, idx, w);
      ss += sumsq8(w);
    }
  }
  const float S = block_sum(ss, red);
  const float rstd = rstd_from_sumsq(S, inv_k, eps);
  if (tid == 0 && rstd_out != nullptr) rstd_out[t] = rstd;

  if constexpr (!INT8) {
    u32x4* orow = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + t * K);
    auto store = [&](const float n[8], int idx) {
      orow[idx] = u32x4{pack_bf16x2(n[0], n[1]), pack_bf16x2(n[2], n[3]), pack_bf16x2(n[4], n[5]),
                        pack_bf16x2(n[6], n[7])};
    };
    if constexpr (CPT > 0) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int idx = tid + c * kThreads;
        float n[8];
        normed8g(v[c], gv[c], has_g, rstd, n);
        if (idx < nch) store(n, idx);
      }
    } else {
      for (int idx = tid; idx < nch; idx += kThreads) {
        float n[8];
        normed8(row(t, idx), gr, idx, rstd, n);
        store(n, idx);
      }
    }
  } else {
    float amax = 0.f;
    auto amax_of = [&](u32x4 w, int idx) {
      float n[8];
      normed8(w, gr, idx, rstd, n);
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(n[j]));
    };
    if constexpr (CPT > 0) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        float n[8];
        normed8g(v[c], gv[c], has_g, rstd, n);  // chunks past K are zero
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(n[j]));
      }
    } else {
      for (int idx = tid; idx < nch; idx += kThreads) amax_of(row(t, idx), idx);
    }
    amax = block_max(amax, red);
    const float s = amax > 0.f ? __fdiv_rn(127.0f, amax) : 0.f;
    if (tid == 0 && x_scale_out != nullptr) x_scale_out[t] = __fdiv_rn(amax, 127.0f);
    u32x2* orow = reinterpret_cast<u32x2*>(static_cast<int8_t*>(out) + t * K);
    auto emit = [&](u32x4 w, int idx) {
      float n[8];
      normed8(w, gr, idx, rstd, n);
      orow[idx] = u32x2{q4(n, 0, s), q4(n, 4, s)};
    };
    if constexpr (CPT > 0) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int idx = tid + c * kThreads;
        float n[8];
        normed8g(v[c], gv[c], has_g, rstd, n);
        if (idx < nch) orow[idx] = u32x2{q4(n, 0, s), q4(n, 4, s)};
      }
    } else {
      for (int idx = tid; idx < nch; idx += kThreads) emit(row(t, idx), idx);
    }
  }
}

template <int CPT, bool INT8, class Row>
__global__ __launch_bounds__(kThreads) void norm_rows_kernel(
    Row row, const uint16_t* __restrict__ gamma, float eps, float inv_k, int64_t K,
    void* __restrict__ out, float* __restrict__ x_scale_out, float* __restrict__ rstd_out) {
  __shared__ float red[4];
  norm_row<CPT, INT8>(row, gamma, eps, inv_k, K, out, x_scale_out, rstd_out, (int64_t)blockIdx.x, red);
}

// Two row sets normed in one launch (the query and the key-value parts of the MLA
// prolog's stage-1 rows): grid row 0 takes part a, grid row 1 part b (a second
// grid axis, so that the x axis holds T workgroups, not 2T).
template <class Row>
struct NormPart {
  Row row;
  const uint16_t* gamma;
  float inv_k;
  int64_t K;
  uint16_t* out;
  float* rstd_out;
};

template <int CPT, class Row>
__global__ __launch_bounds__(kThreads) void norm_rows_pair_kernel(NormPart<Row> a, NormPart<Row> b, float eps) {
  __shared__ float red[4];
  const NormPart<Row> p = blockIdx.y != 0 ? b : a;  // uniform over the workgroup
  norm_row<CPT, false>(p.row, p.gamma, eps, p.inv_k, p.K, p.out, nullptr, p.rstd_out, (int64_t)blockIdx.x, red);
}

// Short rows (K <= 8192): one wavefront per row, four rows per workgroup.  Each
// lane loads its CPL chunks of x and of gamma in one round trip, the sum of
// squares and amax are reduced with wavefront shuffles (no barriers), and the
// normed values stay in registers between the amax and the quantisation.
template <int CPL, bool INT8, bool ADD, bool G>
__global__ __launch_bounds__(kThreads) void norm_rows_wave_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ residual, uint16_t* __restrict__ x_add,
    const uint16_t* __restrict__ gamma, float eps, float inv_k, int64_t T, int64_t K,
    void* __restrict__ out, float* __restrict__ x_scale_out, float* __restrict__ rstd_out) {
  const int lane = threadIdx.x & 63;
  // the row index is wavefront-uniform: readfirstlane lets the buffer resources live in scalar registers
  const int64_t t = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= T) return;  // whole wavefront: no barrier follows
  // Chunk c of this lane is the 16 bytes at (lane + 64 c) * 16 of the row.  All
  // row accesses go through buffer resources sized to the row, so chunks past K
  // read as zero and their stores are dropped: no per-chunk branches.
  const uint32_t kb = (uint32_t)K * 2u;  // K <= 8192
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + t * K, kb);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(gamma, G ? kb : 0u);
  auto off = [&](int c) -> uint32_t { return (uint32_t)(lane + 64 * c) * 16u; };
  u32x4 v[CPL], gv[CPL];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    v[c] = buf_load16(rx, off(c));
    if constexpr (G) gv[c] = buf_load16(rg, off(c));
  }
  // keep the gamma loads here, in flight with the row's (the scheduler would
  // otherwise sink them past the reduction, adding a round trip)
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (ADD) {
    // x + residual: the sum is what the norm reads, and is written back
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(residual + t * K, kb);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(x_add + t * K, kb);
    u32x4 rv[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) rv[c] = buf_load16(rr, off(c));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      v[c] = add_bf16x8(v[c], rv[c]);
      __builtin_amdgcn_raw_buffer_store_b128(v[c], ra, off(c), 0, 0);
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) ss += sumsq8(v[c]);
  const float rstd = rstd_from_sumsq(wave_sum(ss), inv_k, eps);
  if (lane == 0 && rstd_out != nullptr) rstd_out[t] = rstd;

  float n[CPL][8];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      n[c][2 * j] = __fmul_rn(bf16lo(v[c][j]), rstd);
      n[c][2 * j + 1] = __fmul_rn(bf16hi(v[c][j]), rstd);
      if constexpr (G) {
        n[c][2 * j] = __fmul_rn(n[c][2 * j], bf16lo(gv[c][j]));
        n[c][2 * j + 1] = __fmul_rn(n[c][2 * j + 1], bf16hi(gv[c][j]));
      }
    }
  }
  if constexpr (!INT8) {
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(static_cast<uint16_t*>(out) + t * K, kb);
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      __builtin_amdgcn_raw_buffer_store_b128(
          u32x4{pack_bf16x2(n[c][0], n[c][1]), pack_bf16x2(n[c][2], n[c][3]), pack_bf16x2(n[c][4], n[c][5]),
                pack_bf16x2(n[c][6], n[c][7])},
          ro, off(c), 0, 0);
  } else {
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(n[c][j]));  // chunks past K are 0
    amax = wave_max(amax);
    const float s = amax > 0.f ? __fdiv_rn(127.0f, amax) : 0.f;
    if (lane == 0 && x_scale_out != nullptr) x_scale_out[t] = __fdiv_rn(amax, 127.0f);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(static_cast<int8_t*>(out) + t * K, (uint32_t)K);
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{q4(n[c], 0, s), q4(n[c], 4, s)}, ro, off(c) / 2u, 0, 0);
  }
}

template <bool INT8, bool ADD>
hipError_t launch_norm_wave(const uint16_t* x, const uint16_t* residual, uint16_t* x_add, const uint16_t* gamma,
                            float eps, int64_t T, int64_t K, void* out, float* x_scale_out, float* rstd_out,
                            hipStream_t s) {
  const float inv_k = 1.0f / (float)K;
  const int64_t per = (K / 8 + 63) / 64;
  dim3 grid((unsigned)((T + 3) / 4)), block(kThreads);
#define RNL_NORM_WAVE(C)                                                                                      \
  do {                                                                                                          \
    if (gamma != nullptr)                                                                                       \
      hipLaunchKernelGGL((norm_rows_wave_kernel<C, INT8, ADD, true>), grid, block, 0, s, x, residual, x_add,    \
                         gamma, eps, inv_k, T, K, out, x_scale_out, rstd_out);                                  \
    else                                                                                                        \
      hipLaunchKernelGGL((norm_rows_wave_kernel<C, INT8, ADD, false>), grid, block, 0, s, x, residual, x_add,   \
                         gamma, eps, inv_k, T, K, out, x_scale_out, rstd_out);                                  \
  } while (0)
  if (per <= 1) RNL_NORM_WAVE(1);
  else if (per <= 2) RNL_NORM_WAVE(2);
  else if (per <= 4) RNL_NORM_WAVE(4);
  else if (per <= 8) RNL_NORM_WAVE(8);
  else RNL_NORM_WAVE(16);
#undef RNL_NORM_WAVE
  return hipGetLastError();
}

constexpr int64_t kWaveRowMaxK = 8192;
// Fewer rows than CUs, each with a chunk for every thread of a workgroup: a
// workgroup per row (four wavefronts share the row, so each runs a quarter of the
// arithmetic) finishes sooner than a wavefront per row.
constexpr int64_t kWaveRowMinT = 256;
inline bool wave_rows(int64_t T, int64_t K) {
  return K <= kWaveRowMaxK && (T >= kWaveRowMinT || K < 8 * kThreads);
}

template <bool INT8, class Row>
hipError_t launch_norm(Row row, const uint16_t* gamma, float eps, int64_t T, int64_t K, void* out,
                       float* x_scale_out, float* rstd_out, hipStream_t s) {
  const float inv_k = 1.0f / (float)K;  // fl(1/K): K < 2^24 converts exactly
  const int64_t nch = K / 8;
  const int64_t per = (nch + kThreads - 1) / kThreads;
  dim3 grid((unsigned)T), block(kThreads);
#define RNL_NORM_LAUNCH(C)                                                                              \
  hipLaunchKernelGGL((norm_rows_kernel<C, INT8, Row>), grid, block, 0, s, row, gamma, eps, inv_k, K, out, \
                     x_scale_out, rstd_out)
  if (per <= 1) RNL_NORM_LAUNCH(1);
  else if (per <= 2) RNL_NORM_LAUNCH(2);
  else if (per <= 4) RNL_NORM_LAUNCH(4);
  else if (per <= 8) RNL_NORM_LAUNCH(8);
  else RNL_NORM_LAUNCH(0);
#undef RNL_NORM_LAUNCH
  return hipGetLastError();
}

template <class Row>
hipError_t launch_norm_pair(const NormPart<Row>& a, const NormPart<Row>& b, float eps, int64_t T, hipStream_t s) {
  const int64_t per = (std::max(a.K, b.K) / 8 + kThreads - 1) / kThreads;
  dim3 grid((unsigned)T, 2u), block(kThreads);
#define RNL_NORM_PAIR(C) hipLaunchKernelGGL((norm_rows_pair_kernel<C, Row>), grid, block, 0, s, a, b, eps)
  if (per <= 1) RNL_NORM_PAIR(1);
  else if (per <= 2) RNL_NORM_PAIR(2);
  else if (per <= 4) RNL_NORM_PAIR(4);
  else if (per <= 8) RNL_NORM_PAIR(8);
  else RNL_NORM_PAIR(0);
#undef RNL_NORM_PAIR
  return hipGetLastError();
}

}  // namespace

hipError_t launch_norm_rows_bf16(const uint16_t* x, const uint16_t* gamma, float eps, int64_t T,
                                 int64_t K, uint16_t* a_out, float* rstd_out, hipStream_t s) {
  if (wave_rows(T, K))
    return launch_norm_wave<false, false>(x, nullptr, nullptr, gamma, eps, T, K, a_out, nullptr, rstd_out, s);
  return launch_norm<false>(RowBf16{x, K}, gamma, eps, T, K, a_out, nullptr, rstd_out, s);
}

hipError_t launch_norm_rows_int8(const uint16_t* x, const uint16_t* gamma, float eps, int64_t T,
                                 int64_t K, int8_t* q_out, float* x_scale_out, float* rstd_out,
                                 hipStream_t s) {
  if (wave_rows(T, K))
    return launch_norm_wave<true, false>(x, nullptr, nullptr, gamma, eps, T, K, q_out, x_scale_out, rstd_out, s);
  return launch_norm<true>(RowBf16{x, K}, gamma, eps, T, K, q_out, x_scale_out, rstd_out, s);
}

hipError_t launch_add_norm_rows_bf16(const uint16_t* x, const uint16_t* residual, uint16_t* x_add,
                                     const uint16_t* gamma, float eps, int64_t T, int64_t K, uint16_t* a_out,
                                     float* rstd_out, hipStream_t s) {
  if (wave_rows(T, K))
    return launch_norm_wave<false, true>(x, residual, x_add, gamma, eps, T, K, a_out, nullptr, rstd_out, s);
  return launch_norm<false>(RowAddBf16{x, residual, x_add, K}, gamma, eps, T, K, a_out, nullptr, rstd_out, s);
}

hipError_t launch_add_norm_rows_int8(const uint16_t* x, const uint16_t* residual, uint16_t* x_add,
                                     const uint16_t* gamma, float eps, int64_t T, int64_t K, int8_t* q_out,
                                     float* x_scale_out, float* rstd_out, hipStream_t s) {
  if (wave_rows(T, K))
    return launch_norm_wave<true, true>(x, residual, x_add, gamma, eps, T, K, q_out, x_scale_out, rstd_out, s);
  return launch_norm<true>(RowAddBf16{x, residual, x_add, K}, gamma, eps, T, K, q_out, x_scale_out, rstd_out, s);
}

namespace {
__global__ __launch_bounds__(kThreads) void add_rows_kernel(const u32x4* __restrict__ x, const u32x4* __restrict__ r,
                                                            u32x4* __restrict__ out, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kThreads)
    out[i] = add_bf16x8(x[i], r[i]);
}
}  // namespace

hipError_t launch_add_rows(const uint16_t* x, const uint16_t* residual, uint16_t* x_add, int64_t T, int64_t K,
                           hipStream_t s) {
  const int64_t n = T * K / 8;
  const int64_t blocks = std::min<int64_t>((n + kThreads - 1) / kThreads, 4096);
  hipLaunchKernelGGL(add_rows_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                     reinterpret_cast<const u32x4*>(x), reinterpret_cast<const u32x4*>(residual),
                     reinterpret_cast<u32x4*>(x_add), n);
  return hipGetLastError();
}

hipError_t launch_reduce_norm_pair_bf16(const float* part, int S, int64_t ld, int64_t T, const NormCols& a,
                                        const NormCols& b, float eps, uint16_t* sum_out, hipStream_t s) {
  auto mk = [&](const NormCols& c) {
    return NormPart<RowPartials>{RowPartials{part + c.col0, T * ld, ld, S, sum_out ? sum_out + c.col0 : nullptr, ld},
                                 c.gamma, 1.0f / (float)c.K, c.K, c.out, c.rstd_out};
  };
  return launch_norm_pair(mk(a), mk(b), eps, T, s);
}

hipError_t launch_norm_rows_pair_bf16_strided(const uint16_t* x, int64_t ld, int64_t T, const NormCols& a,
                                              const NormCols& b, float eps, hipStream_t s) {
  auto mk = [&](const NormCols& c) {
    return NormPart<RowBf16>{RowBf16{x + c.col0, ld}, c.gamma, 1.0f / (float)c.K, c.K, c.out, c.rstd_out};
  };
  return launch_norm_pair(mk(a), mk(b), eps, T, s);
}

hipError_t launch_reduce_norm_bf16(const float* part, int S, int64_t ld, const uint16_t* gamma, float eps,
                                   int64_t T, int64_t K, uint16_t* out, float* rstd_out, uint16_t* sum_out,
                                   int64_t sum_ld, hipStream_t s) {
  return launch_norm<false>(RowPartials{part, T * ld, ld, S, sum_out, sum_ld}, gamma, eps, T, K, out, nullptr,
                            rstd_out, s);
}

}  // namespace rnl
