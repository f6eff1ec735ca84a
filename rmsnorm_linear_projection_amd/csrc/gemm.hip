// Tiled MFMA GEMM for the projection step: C[M,N] = A[M,K] . B[N,K]^T (b_trans).
//
// A is the normed activation tile (bf16, or per-token int8), B the weight
// stored [N, K] (AT-10 page section 2: the weight enters with b_trans=True).
// Both operands are K-contiguous, so both are staged through LDS the same way:
// a k-step is 128 bytes of every tile row (64 bf16 or 128 int8), one 16-byte
// chunk per lane, which is exactly one MFMA operand register quad:
//   bf16: v_mfma_f32_16x16x32_bf16  (8 bf16 per lane, fp32 accumulate)
//   int8: v_mfma_i32_16x16x64_i8    (16 int8 per lane, int32 accumulate)
//
// Workgroup: 256 threads = 4 wavefronts in a 2 x 2 grid over a BM x BN tile.
// The weight fragment is the MFMA "A" source and the activation fragment the
// "B" source, so each lane ends up holding 4 consecutive output columns of one
// token row, which it stores as one 8- or 16-byte vector.
//
// Data movement: buffer loads (out-of-range rows and the K tail read as zero)
// into registers one k-step ahead, then into a double-buffered LDS stage with
// an XOR swizzle of the 16-byte chunk index so that the 16 lanes reading one
// operand column hit distinct banks.  Workgroup ids are remapped so that each
// of the 8 XCDs (dispatched round-robin) works on a contiguous, grouped block
// of tiles that share A and B panels in its L2.
#include "common.cuh"
#include "launch.h"

namespace rnl {
namespace {

template <typename TIn>
struct Mfma;

template <>
struct Mfma<uint16_t> {
  using Acc = f32x4;
  static __device__ __forceinline__ Acc mma(u32x4 p, u32x4 q, Acc c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, p),
                                                   __builtin_bit_cast(bf16x8, q), c, 0, 0, 0);
  }
};

template <>
struct Mfma<int8_t> {
  using Acc = i32x4;
  static __device__ __forceinline__ Acc mma(u32x4 p, u32x4 q, Acc c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, p),
                                                 __builtin_bit_cast(i32x4, q), c, 0, 0, 0);
  }
};

enum Epi : int { EPI_BF16 = 0, EPI_F32 = 1, EPI_I32 = 2, EPI_DEQ_BF16 = 3, EPI_DEQ_F32 = 4 };

// 16-byte chunk slot of tile row r: distinct over any 16 consecutive rows that
// share a parity and over any 8 consecutive rows, so a 16-lane column read is
// conflict-free whether the LDS serves 8 or 16 lanes of a b128 read per cycle.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <typename TIn, int BM, int BN, int GROUP_M, int EPI>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void gemm_nt_kernel(const TIn* __restrict__ A, const TIn* __restrict__ B, void* __restrict__ C,
                    const float* __restrict__ xs, const float* __restrict__ ws, int M, int N, int K,
                    int tiles_m, int tiles_n) {
  using Acc = typename Mfma<TIn>::Acc;
  constexpr int ROWB = 128;
  constexpr int A_CH = BM * 8 / 256;
  constexpr int B_CH = BN * 8 / 256;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MI = WM / 16, NI = WN / 16;
  constexpr int STAGE = (BM + BN) * ROWB;
  static_assert(BM % 32 == 0 && BN % 32 == 0, "tile rows must be multiples of 32");
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // workgroup -> tile: contiguous range per XCD, grouped along M inside it
  const int bid = blockIdx.x, nwg = gridDim.x;
  const int logical = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;
  const int per_group = GROUP_M * tiles_n;
  const int group = logical / per_group;
  const int first_m = group * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int in_group = logical - group * per_group;
  const int tm = first_m + in_group % gm;
  const int tn = in_group / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  const uint32_t kbytes = (uint32_t)K * (uint32_t)sizeof(TIn);
  const int nk = (int)((kbytes + ROWB - 1) / ROWB);
  const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (size_t)m0 * K, (uint32_t)rows_a * kbytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + (size_t)n0 * K, (uint32_t)rows_b * kbytes);

  // global chunk owned by this thread: row (tid >> 3) of each 32-row slab, chunk (tid & 7)
  const int crow = tid >> 3, ccol = tid & 7;
  const uint32_t g_base = (uint32_t)crow * kbytes + (uint32_t)ccol * 16u;
  const uint32_t g_slab = 32u * kbytes;
  const uint32_t l_base = (uint32_t)crow * ROWB + (uint32_t)((ccol ^ swz(crow)) * 16);

  // fragment read offsets: operand row = lane & 15, chunk = kk * 4 + (lane >> 4)
  const int frow = lane & 15;
  const uint32_t f_off0 = (uint32_t)frow * ROWB + (uint32_t)((((lane >> 4)) ^ swz(frow)) * 16);
  const uint32_t f_off1 = (uint32_t)frow * ROWB + (uint32_t)(((4 + (lane >> 4)) ^ swz(frow)) * 16);

  u32x4 ga[A_CH], gb[B_CH];
  auto gload = [&](int kt) {
    const uint32_t kb = (uint32_t)kt * ROWB;
    const bool in_k = kb + (uint32_t)ccol * 16u < kbytes;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) ga[i] = buf_load16(ra, in_k ? g_base + i * g_slab + kb : kOOB);
#pragma unroll
    for (int i = 0; i < B_CH; ++i) gb[i] = buf_load16(rb, in_k ? g_base + i * g_slab + kb : kOOB);
  };
  auto lstore = [&](int buf) {
    char* s = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) *reinterpret_cast<u32x4*>(s + l_base + i * 32 * ROWB) = ga[i];
#pragma unroll
    for (int i = 0; i < B_CH; ++i)
      *reinterpret_cast<u32x4*>(s + BM * ROWB + l_base + i * 32 * ROWB) = gb[i];
  };

  Acc acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = Acc{0, 0, 0, 0};

  gload(0);
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const char* sa = smem + cur * STAGE + (wm * WM) * ROWB;
    const char* sb = smem + cur * STAGE + BM * ROWB + (wn * WN) * ROWB;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint32_t fo = kk ? f_off1 : f_off0;
      u32x4 fa[MI], fb[NI];
#pragma unroll
      for (int i = 0; i < MI; ++i) fa[i] = *reinterpret_cast<const u32x4*>(sa + i * 16 * ROWB + fo);
#pragma unroll
      for (int j = 0; j < NI; ++j) fb[j] = *reinterpret_cast<const u32x4*>(sb + j * 16 * ROWB + fo);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = Mfma<TIn>::mma(fb[j], fa[i], acc[i][j]);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds C[m][n .. n+3]
  const bool vec_ok = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int m = m0 + wm * WM + i * 16 + (lane & 15);
    if (m >= M) continue;
    float xsm = 0.f;
    if constexpr (EPI == EPI_DEQ_BF16 || EPI == EPI_DEQ_F32) xsm = xs[m];
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int n = n0 + wn * WN + j * 16 + 4 * (lane >> 4);
      if (n >= N) continue;
      const size_t off = (size_t)m * (size_t)N + (size_t)n;
      const bool full = vec_ok && (n + 3 < N);
      if constexpr (EPI == EPI_I32) {
        int32_t* c = static_cast<int32_t*>(C) + off;
        if (full) {
          *reinterpret_cast<i32x4*>(c) = acc[i][j];
        } else {
          for (int r = 0; r < 4 && n + r < N; ++r) c[r] = acc[i][j][r];
        }
      } else {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (EPI == EPI_DEQ_BF16 || EPI == EPI_DEQ_F32) {
            const float wsn = (n + r < N) ? ws[n + r] : 0.f;
            v[r] = __fmul_rn((float)acc[i][j][r], __fmul_rn(xsm, wsn));
          } else {
            v[r] = (float)acc[i][j][r];
          }
        }
        if constexpr (EPI == EPI_F32 || EPI == EPI_DEQ_F32) {
          float* c = static_cast<float*>(C) + off;
          if (full) {
            *reinterpret_cast<f32x4*>(c) = f32x4{v[0], v[1], v[2], v[3]};
          } else {
            for (int r = 0; r < 4 && n + r < N; ++r) c[r] = v[r];
          }
        } else {
          uint16_t* c = static_cast<uint16_t*>(C) + off;
          if (full) {
            *reinterpret_cast<u32x2*>(c) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          } else {
            for (int r = 0; r < 4 && n + r < N; ++r)
              c[r] = (uint16_t)(pack_bf16x2(v[r], 0.f) & 0xFFFFu);
          }
        }
      }
    }
  }
}

template <typename TIn, int BM, int BN, int EPI>
hipError_t launch_tile(const TIn* A, const TIn* B, void* C, const float* xs, const float* ws,
                       int64_t M, int64_t N, int64_t K, hipStream_t s) {
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  const int nwg = tiles_m * tiles_n;
  hipLaunchKernelGGL((gemm_nt_kernel<TIn, BM, BN, 8, EPI>), dim3(nwg), dim3(256), 0, s, A, B, C,
                     xs, ws, (int)M, (int)N, (int)K, tiles_m, tiles_n);
  return hipGetLastError();
}

int64_t tiles_of(int64_t M, int64_t N, int bm, int bn) {
  return ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
}

template <typename TIn, int EPI>
hipError_t launch_shape(const TIn* A, const TIn* B, void* C, const float* xs, const float* ws,
                        int64_t M, int64_t N, int64_t K, hipStream_t s) {
  // Largest tile that still gives every CU at least one workgroup.
  if (tiles_of(M, N, 256, 192) >= 256) return launch_tile<TIn, 256, 192, EPI>(A, B, C, xs, ws, M, N, K, s);
  if (tiles_of(M, N, 256, 128) >= 256) return launch_tile<TIn, 256, 128, EPI>(A, B, C, xs, ws, M, N, K, s);
  return launch_tile<TIn, 128, 128, EPI>(A, B, C, xs, ws, M, N, K, s);
}

}  // namespace

hipError_t launch_gemm_bf16(const uint16_t* A, const uint16_t* B, void* C, int out_kind, int64_t M,
                            int64_t N, int64_t K, hipStream_t s) {
  if (out_kind == OUT_F32) return launch_shape<uint16_t, EPI_F32>(A, B, C, nullptr, nullptr, M, N, K, s);
  return launch_shape<uint16_t, EPI_BF16>(A, B, C, nullptr, nullptr, M, N, K, s);
}

hipError_t launch_gemm_int8(const int8_t* A, const int8_t* B, void* C, int out_kind,
                            const float* xs, const float* ws, int64_t M, int64_t N, int64_t K,
                            hipStream_t s) {
  if (out_kind == OUT_I32) return launch_shape<int8_t, EPI_I32>(A, B, C, xs, ws, M, N, K, s);
  if (out_kind == OUT_F32) return launch_shape<int8_t, EPI_DEQ_F32>(A, B, C, xs, ws, M, N, K, s);
  return launch_shape<int8_t, EPI_DEQ_BF16>(A, B, C, xs, ws, M, N, K, s);
}

}  // namespace rnl
