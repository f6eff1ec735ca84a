// fp32-weight projection of the fp32 normed rows, split over K: the SK-03
// page's mhc_pre variant (a very long reduction into a few output columns,
// computed in fp32, e.g. [B, 28672] x [28672, 24]).
//
// The output is tiny, so the only parallelism is along K: the reduction is
// split into S contiguous ranges of 512 k, each workgroup producing fp32 partial
// dot products and partial sums of squares for 64 tokens x 32 output columns;
// a second kernel adds the S partials in a fixed order (bit-reproducible) and
// applies rstd.
//
// x is read exactly once.  Without a gamma, n = x * rstd, so
// sum_k n[k] W[j,k] = rstd * sum_k x[k] W[j,k] in exact arithmetic: the
// partials use the raw bf16 x and rstd is applied in the epilogue (the pages'
// variant avoids materialising an fp32 copy of x for the same reason).  With a
// gamma the weight is first scaled by gamma[k] in fp32.
//
// The fp32 weight is split exactly into three bf16 parts, W = hi + mid + lo
// (each the top 16 bits of the running remainder; three 8-bit slices cover
// the 24-bit significand), so the contraction runs on bf16 MFMA
// (v_mfma_f32_16x16x32_bf16, exact products, fp32 accumulation) at three
// MFMAs per block instead of the much slower fp32 MFMA.  The weight
// ([N, K] fp32, a few MB) is re-read by every token group and stays in L2.
#include "common.cuh"
#include "launch.h"

namespace rnl {
namespace {

constexpr int kTG = 64;  // tokens per workgroup (4 MFMA column blocks)
constexpr int kNC = 32;  // output columns per workgroup (2 MFMA row blocks)

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

// high 16 bits of two fp32 words -> one packed bf16 pair (lo word first)
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xFFFF0000u);
}

struct Split3 {
  u32x4 hi, mid, lo;
};

// exact split of 8 fp32 values into three bf16x8 operands
__device__ __forceinline__ Split3 split_w(const float w[8]) {
  Split3 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t a = __float_as_uint(w[2 * j]), b = __float_as_uint(w[2 * j + 1]);
    const float ah = __uint_as_float(a & 0xFFFF0000u), bh = __uint_as_float(b & 0xFFFF0000u);
    const float ar = __fsub_rn(w[2 * j], ah), br = __fsub_rn(w[2 * j + 1], bh);
    const uint32_t ar_u = __float_as_uint(ar), br_u = __float_as_uint(br);
    const float am = __uint_as_float(ar_u & 0xFFFF0000u), bm = __uint_as_float(br_u & 0xFFFF0000u);
    const float al = __fsub_rn(ar, am), bl = __fsub_rn(br, bm);
    r.hi[j] = hi_halves(a, b);
    r.mid[j] = hi_halves(ar_u, br_u);
    r.lo[j] = hi_halves(__float_as_uint(al), __float_as_uint(bl));
  }
  return r;
}

__device__ __forceinline__ f32x4 mma(u32x4 p, u32x4 q, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, p),
                                                 __builtin_bit_cast(bf16x8, q), c, 0, 0, 0);
}

// One workgroup: 64 tokens x 32 output columns x one K range of 4 * kSPW k-steps
// (32 k each); wavefront w takes kSPW consecutive k-steps.  Each wavefront
// issues all of its loads (x, weight, gamma) before the first MFMA, so the whole
// grid's data is requested in one round trip.
constexpr int kSPW = 4;

template <bool GAMMA>
__global__ __launch_bounds__(256) void skinny_partial_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma, const float* __restrict__ W,
    float* __restrict__ part, float* __restrict__ ss_part, int T, int K, int N, int Npad) {
  __shared__ f32x4 red[3][8][64];
  __shared__ float red_ss[4][kTG];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * kTG, z = blockIdx.y, nc0 = blockIdx.z * kNC;
  const bool do_ss = blockIdx.z == 0;
  const int s_beg = (z * 4 + wave) * kSPW;  // first k-step of this wavefront

  const uint32_t kbytes = (uint32_t)K * 2u, wbytes = (uint32_t)K * 4u;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + (size_t)t0 * K, (uint32_t)min(kTG, T - t0) * kbytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + (size_t)nc0 * K, (uint32_t)min(kNC, N - nc0) * wbytes);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(gamma, GAMMA ? kbytes : 0u);

  u32x4 xv[kSPW][4], w0[kSPW][2], w1[kSPW][2], gv[kSPW];
#pragma unroll
  for (int u = 0; u < kSPW; ++u) {
    const int k = (s_beg + u) * 32 + g * 8;
    const bool in_k = k < K;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
      xv[u][tb] = buf_load16(rx, in_k ? (uint32_t)(tb * 16 + r16) * kbytes + (uint32_t)k * 2u : kOOB);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const uint32_t base = (uint32_t)(nb * 16 + r16) * wbytes + (uint32_t)k * 4u;
      w0[u][nb] = buf_load16(rw, in_k ? base : kOOB);
      w1[u][nb] = buf_load16(rw, in_k ? base + 16u : kOOB);
    }
    if constexpr (GAMMA) gv[u] = buf_load16(rg, in_k ? (uint32_t)k * 2u : kOOB);
    else gv[u] = u32x4{0u, 0u, 0u, 0u};
  }

  f32x4 acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss[4] = {0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int u = 0; u < kSPW; ++u) {
    float wv[2][8];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wv[nb][j] = __uint_as_float(w0[u][nb][j]);
        wv[nb][4 + j] = __uint_as_float(w1[u][nb][j]);
      }
    if constexpr (GAMMA) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          wv[nb][2 * j] = __fmul_rn(wv[nb][2 * j], bf16lo(gv[u][j]));
          wv[nb][2 * j + 1] = __fmul_rn(wv[nb][2 * j + 1], bf16hi(gv[u][j]));
        }
    }
    if (do_ss) {
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) ss[tb] += sumsq8(xv[u][tb]);
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const Split3 p = split_w(wv[nb]);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        acc[tb][nb] = mma(p.hi, xv[u][tb], acc[tb][nb]);
        acc[tb][nb] = mma(p.mid, xv[u][tb], acc[tb][nb]);
        acc[tb][nb] = mma(p.lo, xv[u][tb], acc[tb][nb]);
      }
    }
  }

  // combine the four wavefronts in a fixed order
  if (wave > 0) {
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) red[wave - 1][tb * 2 + nb][lane] = acc[tb][nb];
  }
  if (do_ss) {
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      float v = ss[tb];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      if (g == 0) red_ss[wave][tb * 16 + r16] = v;
    }
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const int t = t0 + tb * 16 + r16;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        f32x4 v = acc[tb][nb];
        v += red[0][tb * 2 + nb][lane];
        v += red[1][tb * 2 + nb][lane];
        v += red[2][tb * 2 + nb][lane];
        if (t < T) {
          const int n = nc0 + nb * 16 + 4 * g;  // < Npad always
          *reinterpret_cast<f32x4*>(part + ((size_t)z * T + t) * Npad + n) = v;
        }
      }
    }
  }
  if (do_ss && tid < kTG && t0 + tid < T) {
    ss_part[(size_t)z * T + t0 + tid] = red_ss[0][tid] + red_ss[1][tid] + red_ss[2][tid] + red_ss[3][tid];
  }
}

// Finalize: workgroup (t, column block of 64).  Lane c of wavefront w adds the
// partials z = w, w + 4, w + 8, ... of column c (eight loads in flight per
// round), then the four wavefront sums are added in wavefront order, so the
// summation order depends only on S and the result is bit-reproducible.
constexpr int kFinZ = 8;

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void skinny_finalize_kernel(
    const float* __restrict__ part, const float* __restrict__ ss_part, void* __restrict__ y,
    float* __restrict__ rstd_out, int T, int N, int Npad, int S, float inv_k, float eps) {
  __shared__ float red[2][4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x, n = blockIdx.y * 64 + lane;
  const bool col = n < N;
  float acc = 0.f, sq = 0.f;
  for (int z0 = wave; z0 < S; z0 += 4 * kFinZ) {
    float p[kFinZ], q[kFinZ];
#pragma unroll
    for (int i = 0; i < kFinZ; ++i) {
      const int z = z0 + 4 * i;
      const bool ok = z < S;
      p[i] = (ok && col) ? part[((size_t)z * T + t) * Npad + n] : 0.f;
      q[i] = ok ? ss_part[(size_t)z * T + t] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kFinZ; ++i) {
      acc += p[i];
      sq += q[i];
    }
  }
  red[0][wave][lane] = acc;
  red[1][wave][lane] = sq;
  __syncthreads();
  if (wave != 0) return;
  acc = ((red[0][0][lane] + red[0][1][lane]) + red[0][2][lane]) + red[0][3][lane];
  sq = ((red[1][0][lane] + red[1][1][lane]) + red[1][2][lane]) + red[1][3][lane];
  const float rstd = rstd_from_sumsq(sq, inv_k, eps);
  if (n == 0 && rstd_out != nullptr) rstd_out[t] = rstd;
  if (!col) return;
  const float v = __fmul_rn(rstd, acc);
  const size_t idx = (size_t)t * N + n;
  if constexpr (OUT_BF16) {
    static_cast<uint16_t*>(y)[idx] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xFFFFu);
  } else {
    static_cast<float*>(y)[idx] = v;
  }
}

struct Plan {
  int tg, nc, nsteps, S, sps, Npad;
};

Plan plan_of(int64_t T, int64_t K, int64_t N) {
  Plan p;
  p.tg = (int)((T + kTG - 1) / kTG);
  p.nc = (int)((N + kNC - 1) / kNC);
  p.Npad = p.nc * kNC;
  p.nsteps = (int)((K + 31) / 32);
  p.sps = 4 * kSPW;
  p.S = (p.nsteps + p.sps - 1) / p.sps;
  return p;
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

size_t skinny_workspace_bytes(int64_t T, int64_t K, int64_t N) {
  const Plan p = plan_of(T, K, N);
  return align256((size_t)p.S * (size_t)T * (size_t)p.Npad * 4) + align256((size_t)p.S * (size_t)T * 4);
}

hipError_t launch_skinny_fp32w(const uint16_t* x, const uint16_t* gamma, float eps, const float* W,
                               void* y, int out_kind, float* rstd_out, int64_t T, int64_t K,
                               int64_t N, void* workspace, hipStream_t s) {
  const Plan p = plan_of(T, K, N);
  float* part = static_cast<float*>(workspace);
  float* ss_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                            align256((size_t)p.S * (size_t)T * (size_t)p.Npad * 4));
  dim3 grid((unsigned)p.tg, (unsigned)p.S, (unsigned)p.nc), block(256);
  if (gamma != nullptr)
    hipLaunchKernelGGL((skinny_partial_kernel<true>), grid, block, 0, s, x, gamma, W, part, ss_part,
                       (int)T, (int)K, (int)N, p.Npad);
  else
    hipLaunchKernelGGL((skinny_partial_kernel<false>), grid, block, 0, s, x, gamma, W, part, ss_part,
                       (int)T, (int)K, (int)N, p.Npad);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float inv_k = 1.0f / (float)K;
  dim3 g2((unsigned)T, (unsigned)((N + 63) / 64));
  if (out_kind == OUT_BF16)
    hipLaunchKernelGGL((skinny_finalize_kernel<true>), g2, block, 0, s, part, ss_part, y, rstd_out,
                       (int)T, (int)N, p.Npad, p.S, inv_k, eps);
  else
    hipLaunchKernelGGL((skinny_finalize_kernel<false>), g2, block, 0, s, part, ss_part, y, rstd_out,
                       (int)T, (int)N, p.Npad, p.S, inv_k, eps);
  return hipGetLastError();
}

}  // namespace rnl
