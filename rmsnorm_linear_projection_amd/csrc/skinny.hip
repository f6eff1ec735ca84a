// fp32-weight projection of the fp32 normed rows, split over K: the SK-03
// page's mhc_pre variant (a very long reduction into a few output columns,
// computed in fp32, e.g. [B, 28672] x [28672, 24]).
//
// The output is tiny, so the only parallelism is along K: the reduction is
// split into S contiguous ranges (S chosen so that there is about one
// workgroup per CU), each workgroup producing fp32 partial dot products and
// partial sums of squares for 64 tokens x 32 output columns; a second kernel
// adds the S partials in a fixed order (bit-reproducible) and applies rstd.
// A single kernel in which the last workgroup of a token group to finish adds
// the partials was measured at 96 us against about 15 for the pair: reading
// other XCDs' partials takes an agent-scope release and acquire, which write
// back and invalidate the L2 of the workgroup's XCD.  A finalize with one
// wavefront per token (lanes over column quads and partials, fixed butterfly)
// measured 16.3 us for the pair against 14.6 for the one below.
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
#include <algorithm>

#include "common.hpp"
#include "launch.h"

namespace rnl {
namespace {

constexpr int kTG = 64;  // tokens per workgroup (4 MFMA column blocks)
constexpr int kNC = 32;  // output columns per workgroup (2 MFMA row blocks)
constexpr int kKU = 1;   // k-steps per load batch
constexpr int kNW = 4;   // wavefronts per workgroup of the partial kernel

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

// One workgroup: 64 tokens x 32 output columns x one contiguous range of k-steps
// (32 k each), split evenly over its NW wavefronts.  The grid holds about one
// workgroup per CU; each wavefront streams its range with the loads of the next
// KU k-steps in flight (two alternating register batches) while it splits and
// multiplies the current ones, and two wavefronts per SIMD hide each other's
// load latency.  The sum of squares of each token also runs
// on the MFMA: with the token fragment as both operands, the diagonal of the
// 16 x 16 product is sum_k x^2 for the 16 tokens (exact bf16 products, fp32
// accumulation), which spares the vector ALU a squaring pass.
template <int KU, int NW, int TG, bool GAMMA>
__global__ __launch_bounds__(NW * 64) void skinny_partial_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma, const float* __restrict__ W,
    float* __restrict__ part, float* __restrict__ ss_part, int T, int K, int N, int Npad,
    int steps_per_wg, int ntg, int nsplit) {
  constexpr int TB = TG / 16;  // MFMA column blocks of tokens
  __shared__ f32x4 red[NW - 1][2 * TB][64];
  __shared__ float red_ss[NW][TG];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  // Work item (token group, K piece, column block).  With a flat grid, the
  // workgroups that share a K piece (and so read the same weight slice) are
  // placed on one XCD: dispatch deals workgroup ids round-robin over the 8
  // XCDs, so id b is remapped to (b % 8) * (n / 8) + b / 8 and consecutive
  // remapped ids, which differ only in the token group, stay on one L2.
  int tgi, z, ncb;
  if (ntg > 0) {
    const int b = blockIdx.x, n = gridDim.x;
    const int L = (n % 8 == 0) ? (b % 8) * (n / 8) + b / 8 : b;
    tgi = L % ntg;
    z = (L / ntg) % nsplit;
    ncb = L / ntg / nsplit;
  } else {
    tgi = blockIdx.x;
    z = blockIdx.y;
    ncb = blockIdx.z;
  }
  const int t0 = tgi * TG, nc0 = ncb * kNC;
  const bool do_ss = ncb == 0;  // uniform: one column block derives the sums of squares

  const int nsteps = (K + 31) / 32;
  const int wg_beg = min(nsteps, z * steps_per_wg), wg_end = min(nsteps, wg_beg + steps_per_wg);
  const int per = (wg_end - wg_beg + NW - 1) / NW;
  const int s_beg = min(wg_end, wg_beg + wave * per), s_end = min(wg_end, s_beg + per);

  const uint32_t kbytes = (uint32_t)K * 2u, wbytes = (uint32_t)K * 4u;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x + (size_t)t0 * K, (uint32_t)min(TG, T - t0) * kbytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + (size_t)nc0 * K, (uint32_t)min(kNC, N - nc0) * wbytes);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(gamma, GAMMA ? kbytes : 0u);

  struct Batch {
    u32x4 xv[KU][TB], w0[KU][2], w1[KU][2], gv[KU];
  };
  auto issue = [&](Batch& b, int s0) {
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int k = (s0 + u) * 32 + g * 8;
      const bool in_k = (s0 + u) < s_end && k < K;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
        b.xv[u][tb] = buf_load16(rx, in_k ? (uint32_t)(tb * 16 + r16) * kbytes + (uint32_t)k * 2u : kOOB);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const uint32_t base = (uint32_t)(nb * 16 + r16) * wbytes + (uint32_t)k * 4u;
        b.w0[u][nb] = buf_load16(rw, in_k ? base : kOOB);
        b.w1[u][nb] = buf_load16(rw, in_k ? base + 16u : kOOB);
      }
      if constexpr (GAMMA) b.gv[u] = buf_load16(rg, in_k ? (uint32_t)k * 2u : kOOB);
      else b.gv[u] = u32x4{0u, 0u, 0u, 0u};
    }
  };

  f32x4 acc[TB][2], sq[TB];
#pragma unroll
  for (int a = 0; a < TB; ++a) {
    sq[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto consume = [&](const Batch& bt) {
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      if (do_ss) {
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) sq[tb] = mma(bt.xv[u][tb], bt.xv[u][tb], sq[tb]);
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float wv[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          wv[j] = __uint_as_float(bt.w0[u][nb][j]);
          wv[4 + j] = __uint_as_float(bt.w1[u][nb][j]);
        }
        if constexpr (GAMMA) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            wv[2 * j] = __fmul_rn(wv[2 * j], bf16lo(bt.gv[u][j]));
            wv[2 * j + 1] = __fmul_rn(wv[2 * j + 1], bf16hi(bt.gv[u][j]));
          }
        }
        const Split3 p = split_w(wv);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          acc[tb][nb] = mma(p.hi, bt.xv[u][tb], acc[tb][nb]);
          acc[tb][nb] = mma(p.mid, bt.xv[u][tb], acc[tb][nb]);
          acc[tb][nb] = mma(p.lo, bt.xv[u][tb], acc[tb][nb]);
        }
      }
    }
  };

  Batch b0, b1;
  issue(b0, s_beg);
  int s0 = s_beg;
  for (; s0 + KU < s_end; s0 += 2 * KU) {
    issue(b1, s0 + KU);
    __builtin_amdgcn_sched_barrier(0);
    consume(b0);
    __builtin_amdgcn_sched_barrier(0);
    issue(b0, s0 + 2 * KU);
    __builtin_amdgcn_sched_barrier(0);
    consume(b1);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (s0 < s_end) consume(b0);

  // combine the wavefronts in a fixed order
  if (wave > 0) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) red[wave - 1][tb * 2 + nb][lane] = acc[tb][nb];
  }
  if (do_ss && (r16 >> 2) == g) {
    // diagonal of the token x token product: lane (r16, g) with r16 / 4 == g holds
    // token r16's sum of squares in element r16 & 3
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) red_ss[wave][tb * 16 + r16] = sq[tb][r16 & 3];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int t = t0 + tb * 16 + r16;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        f32x4 v = acc[tb][nb];
#pragma unroll
        for (int w = 0; w < NW - 1; ++w) v += red[w][tb * 2 + nb][lane];
        if (t < T) {
          const int n = nc0 + nb * 16 + 4 * g;  // < Npad always
          *reinterpret_cast<f32x4*>(part + ((size_t)z * T + t) * Npad + n) = v;
        }
      }
    }
  }
  if (do_ss && tid < TG && t0 + tid < T) {
    float v = red_ss[0][tid];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += red_ss[w][tid];
    ss_part[(size_t)z * T + t0 + tid] = v;
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
  int tg, nc, nsteps, S, spw, Npad;
};

// About one workgroup per CU: the K range is split into S pieces of spw k-steps,
// spw the smallest multiple of 4 (>= 8) such that tg * nc * S does not exceed
// 256.  A piece of a token row is then a multiple of 256 bytes long and starts
// on a 256-byte boundary of the row (T = 512, K = 28672: spw = 28, 8 x 32 = 256
// workgroups).
Plan plan_of(int64_t T, int64_t K, int64_t N, int tg_rows = kTG) {
  Plan p;
  p.tg = (int)((T + tg_rows - 1) / tg_rows);
  p.nc = (int)((N + kNC - 1) / kNC);
  p.Npad = p.nc * kNC;
  p.nsteps = (int)((K + 31) / 32);
  const int64_t tiles = (int64_t)p.tg * p.nc;
  const int64_t per_tile = std::max<int64_t>(1, 256 / tiles);  // pieces per token tile
  int64_t spw = std::max<int64_t>(8, ((p.nsteps + per_tile - 1) / per_tile + 3) / 4 * 4);
  while (spw < 4096 && tiles * ((p.nsteps + spw - 1) / spw) > 256) spw += 4;
  p.spw = (int)spw;
  p.S = (int)((p.nsteps + spw - 1) / spw);
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
  // a flat grid (with the XCD placement) whenever the item count fits one axis
  const int64_t items = (int64_t)p.tg * p.S * p.nc;
  const bool flat = items <= 0x7fffffff;
  dim3 grid = flat ? dim3((unsigned)items) : dim3((unsigned)p.tg, (unsigned)p.S, (unsigned)p.nc);
  const int ntg = flat ? p.tg : 0;
  dim3 block(256);
  if (gamma != nullptr)
    hipLaunchKernelGGL((skinny_partial_kernel<kKU, kNW, kTG, true>), grid, dim3(kNW * 64), 0, s, x, gamma, W, part, ss_part,
                       (int)T, (int)K, (int)N, p.Npad, p.spw, ntg, p.S);
  else
    hipLaunchKernelGGL((skinny_partial_kernel<kKU, kNW, kTG, false>), grid, dim3(kNW * 64), 0, s, x, gamma, W, part, ss_part,
                       (int)T, (int)K, (int)N, p.Npad, p.spw, ntg, p.S);
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
