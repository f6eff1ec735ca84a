// MXFP8 GEMM for the projection step (gfx950): C[M,N] = A[M,K] . B[N,K]^T with
// E4M3 operands and one E8M0 scale per 64 consecutive k of every row of A (the
// MX-quantised normed activations, scales As[M, K/64]) and of B (the weight,
// scales Bs[N, K/64]) -- AT-09's MXFP8 mode, the scaled product of the AT-10
// page section 4, accumulated in fp32.
//
// One k-step is 128 bytes (= 128 k) of every tile row and one
// v_mfma_scale_f32_16x16x128_f8f6f4 per 16 x 16 output block.  The instruction
// takes from lane l (row l & 15, group g = l >> 4) the 16-byte chunks g and
// 4 + g of its row's k-step (k = 16g..16g+15 and 64+16g..64+16g+15), and the
// scale of the 32-wide k block g of its row; a 64-block of the pages is two
// such blocks, so lane group g passes the scale of 64-block 2 kt + g / 2.
//
// Scales: every 32 k-steps (4096 k) the tile's scale bytes for those k-steps
// (64 per row) are staged in LDS with 16-byte loads, rows padded to 68 bytes (an
// odd number of dwords) so that the 16 rows one instruction reads fall in
// distinct banks; every second
// k-step each lane reads one dword per operand row (the scales of both k-steps)
// and picks its byte by shifting.
//
// Staging follows the bf16 / int8 GEMM: global -> LDS by direct-to-LDS DMA,
// 128-byte rows with 16-byte chunk c of row r at slot c ^ (r & 7), XCD-aware
// tile order, and a WMW x WNW grid of wavefronts: 4 x 2 (two per SIMD, each
// 64 x 96) for the 256 x 192 tile, 2 x 2 for the others.  With two LDS stages
// every wait on the DMA is a wait for all loads (vmcnt 0).
// Per k-step, phase A issues the MFMAs of the first half of the activation
// fragments while the second half is read; after the barrier, phase B issues
// the rest while the free stage is refilled and the next k-step's first half
// is read.  Both phases run weight fragment by weight fragment, and phase B
// reloads weight fragment j for the next k-step right after its last MFMA, so
// the weight fragments need no second register set.
#include "common.hpp"
#include "launch.h"

namespace rnl {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// s_waitcnt with vmcnt(n), lgkmcnt(0), expcnt unchanged (gfx9 encoding)
#define RNL_MX_WAIT_VM_LGKM0(n) __builtin_amdgcn_s_waitcnt(0x0070 | ((n) & 15) | (((n) >> 4) << 14))

__device__ __forceinline__ uint32_t buf_load_u8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

template <int BM, int BN, bool OUT_BF16, int WMW = 2, int WNW = 2>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WMW * WNW, 64 * WMW * WNW),
                          amdgpu_waves_per_eu(WMW * WNW / 4, WMW * WNW / 4)))
void gemm_mx_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, const uint8_t* __restrict__ As,
                    const uint8_t* __restrict__ Bs, void* __restrict__ C, int M, int N, int K, int tiles_m,
                    int tiles_n) {
  constexpr int NST = 2;
  constexpr int GROUP_M = 4;
  constexpr int ROWB = 128;
  constexpr int NT = 64 * WMW * WNW;  // threads
  constexpr int A_CH = BM / (8 * WMW * WNW);  // DMA instructions per wave and stage for A
  constexpr int B_CH = BN / (8 * WMW * WNW);
  static_assert(A_CH * 8 * WMW * WNW == BM && B_CH * 8 * WMW * WNW == BN, "DMA rows must split evenly");
  constexpr int LPS = A_CH + B_CH;
  constexpr int WM = BM / WMW, WN = BN / WNW;
  constexpr int NMI = WM / 16, NNI = WN / 16;
  constexpr int HM = NMI / 2;  // activation fragments per phase
  constexpr int STAGE = (BM + BN) * ROWB;
  constexpr int SC_CHUNK = 32;  // k-steps per scale chunk
  constexpr int SC_ROW = 68;    // LDS bytes per scale row (64 used; 17 dwords)
  static_assert(BM % 64 == 0 && BN % 32 == 0, "tile shape");
  __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE + (BM + BN) * SC_ROW];
  char* const sscale = smem + NST * STAGE;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WNW, wn = wave % WNW;

  // workgroup -> tile: contiguous range per XCD, grouped along M inside it
  const int bid = blockIdx.x, nwg = gridDim.x;
  const int tile = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;
  const int per_group = GROUP_M * tiles_n;
  const int group = tile / per_group;
  const int first_m = group * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int in_group = tile - group * per_group;
  const int tm = first_m + in_group % gm;
  const int tn = in_group / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  const uint32_t kbytes = (uint32_t)K;
  const int nk = (K + ROWB - 1) / ROWB;
  const int kb64 = K >> 6;  // scale bytes per row
  const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (size_t)m0 * K, (uint32_t)rows_a * kbytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + (size_t)n0 * K, (uint32_t)rows_b * kbytes);
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(As + (size_t)m0 * kb64, (uint32_t)(rows_a * kb64));
  const __amdgpu_buffer_rsrc_t rsb = make_rsrc(Bs + (size_t)n0 * kb64, (uint32_t)(rows_b * kb64));

  // DMA: one instruction fills 8 consecutive tile rows (1 KiB); lane -> row lane/8, slot lane%8
  const int drow = lane >> 3, dslot = lane & 7;
  const int dchunk = dslot ^ drow;
  const uint32_t d_goff = (uint32_t)drow * kbytes + (uint32_t)dchunk * 16u;
  auto dload_one = [&](int kt, int buf, int g) {
    const uint32_t kb = (uint32_t)kt * ROWB;
    const bool live = kt < nk && kb + (uint32_t)dchunk * 16u < kbytes;
    char* s = smem + buf * STAGE;
    if (g < A_CH) {
      const int j = wave * A_CH + g;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)(s + j * 1024), 16,
          live ? d_goff + (uint32_t)j * 8u * kbytes + kb : kOOB, 0, 0, 0);
    } else {
      const int j = wave * B_CH + (g - A_CH);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, (__attribute__((address_space(3))) void*)(s + BM * ROWB + j * 1024), 16,
          live ? d_goff + (uint32_t)j * 8u * kbytes + kb : kOOB, 0, 0, 0);
    }
  };

  // fragment reads: operand row = lane & 15, chunks (lane >> 4) and 4 + (lane >> 4)
  const int frow = lane & 15, fg = lane >> 4;
  const uint32_t foff0 = (uint32_t)frow * ROWB + (uint32_t)((fg ^ (frow & 7)) * 16);
  const uint32_t foff1 = (uint32_t)frow * ROWB + (uint32_t)(((4 + fg) ^ (frow & 7)) * 16);
  auto lds16 = [&](int buf, int row0, uint32_t fo) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(smem + buf * STAGE + row0 * ROWB + fo);
  };
  struct Frag {
    u32x4 lo, hi;
  };
  Frag a[NMI];
  Frag b[NNI];
  // scale dwords of the current pair of k-steps (bytes: blocks 2kt .. 2kt+3 of the row)
  uint32_t sw[NNI], sx[NMI];

  auto read_a = [&](int buf, int i) {
    const int r0 = wm * WM + i * 16;
    a[i].lo = lds16(buf, r0, foff0);
    a[i].hi = lds16(buf, r0, foff1);
  };
  auto read_b = [&](int buf, int j) {
    const int r0 = BM + wn * WN + j * 16;
    b[j].lo = lds16(buf, r0, foff0);
    b[j].hi = lds16(buf, r0, foff1);
  };
  // stage the scale bytes of k-steps [32 c, 32 c + 32) for all tile rows; bytes past
  // K read as 127 (scale 1: their data are zero), rows past M / N as 0
  auto stage_scales = [&](int c) {
    const int b0 = c * 2 * SC_CHUNK;
    for (int p = tid; p < (BM + BN) * 4; p += NT) {
      const int row = p >> 2, q = p & 3;
      const int byte0 = b0 + 16 * q;
      const bool is_a = row < BM;
      const __amdgpu_buffer_rsrc_t rs = is_a ? rsa : rsb;
      const uint32_t roff = (uint32_t)((is_a ? row : row - BM) * kb64);
      u32x4 v;
      if ((kb64 & 15) == 0) {
        v = byte0 < kb64 ? buf_load16(rs, roff + (uint32_t)byte0)
                         : u32x4{0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu};
      } else {
        v = u32x4{0u, 0u, 0u, 0u};
        for (int e = 0; e < 16; ++e) {
          const uint32_t bv = byte0 + e < kb64 ? buf_load_u8(rs, roff + (uint32_t)(byte0 + e)) : 127u;
          v[e >> 2] |= bv << (8 * (e & 3));
        }
      }
      uint32_t* d = reinterpret_cast<uint32_t*>(sscale + row * SC_ROW + 16 * q);  // 4-byte aligned only
#pragma unroll
      for (int e = 0; e < 4; ++e) d[e] = v[e];
    }
  };
  auto read_scales = [&](int kt) {  // kt even: the dword holds the blocks of kt and kt + 1
    const int o = 2 * (kt % SC_CHUNK);
#pragma unroll
    for (int j = 0; j < NNI; ++j)
      sw[j] = *reinterpret_cast<const uint32_t*>(sscale + (BM + wn * WN + j * 16 + frow) * SC_ROW + o);
#pragma unroll
    for (int i = 0; i < NMI; ++i)
      sx[i] = *reinterpret_cast<const uint32_t*>(sscale + (wm * WM + i * 16 + frow) * SC_ROW + o);
  };

  f32x4 acc[NMI][NNI];
#pragma unroll
  for (int i = 0; i < NMI; ++i)
#pragma unroll
    for (int j = 0; j < NNI; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](int shift, int i, int j) {
    const i32x8 wv = __builtin_bit_cast(i32x8, __builtin_shufflevector(b[j].lo, b[j].hi, 0, 1, 2, 3, 4, 5, 6, 7));
    const i32x8 xv = __builtin_bit_cast(i32x8, __builtin_shufflevector(a[i].lo, a[i].hi, 0, 1, 2, 3, 4, 5, 6, 7));
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wv, xv, acc[i][j], 0, 0, 0, (int)(sw[j] >> shift), 0,
                                                                 (int)(sx[i] >> shift));
  };

  // one k-step; PAR = kt & 1.  (The loop runs one k-step per iteration: with two
  // k-steps per iteration and a compile-time parity the register allocator moves
  // accumulators between AGPRs and VGPRs around the MFMAs.)
  auto kstep = [&](int kt, int PAR) {
    const int slot = PAR, nslot = PAR ^ 1;
    if (PAR == 0) {
      if (kt > 0 && kt % SC_CHUNK == 0) {
        // every wave read the previous chunk two k-steps ago, before the barrier of
        // the previous k-step; the new chunk is visible after this barrier
        stage_scales(kt / SC_CHUNK);
        __syncthreads();
      }
      read_scales(kt);
    }
    // this lane's scale byte sits at bit 8 * (2 PAR + g / 2) of the row's dword
    const int shift = 8 * (2 * PAR + (fg >> 1));
    // phase A: MFMAs of activation fragments [0, HM); read [HM, NMI) of this k-step
#pragma unroll
    for (int j = 0; j < NNI; ++j) {
      if (j < HM) read_a(slot, HM + j);
#pragma unroll
      for (int i = 0; i < HM; ++i) mma(shift, i, j);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = NNI; i < HM; ++i) read_a(slot, HM + i);
    // k-step kt + 1 has landed and every wave has finished reading stage `slot`
    RNL_MX_WAIT_VM_LGKM0(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // phase B: refill `slot` with k-step kt + 2; MFMAs of [HM, NMI); read the next
    // k-step's first half and, after its last use, each weight fragment
#pragma unroll
    for (int j = 0; j < NNI; ++j) {
      // the refill is spread over the weight-fragment groups: issued as one burst by all
      // eight wavefronts, it filled the texture unit's address and command queues (5x the
      // stall cycles of the bf16 GEMM, which interleaves its refill the same way) and the
      // MFMAs behind it waited
#pragma unroll
      for (int g = j * LPS / NNI; g < (j + 1) * LPS / NNI; ++g) dload_one(kt + 2, slot, g);
      if (j < HM) read_a(nslot, j);
#pragma unroll
      for (int i = HM; i < NMI; ++i) mma(shift, i, j);
      read_b(nslot, j);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = NNI; i < HM; ++i) read_a(nslot, i);
  };

  // prologue: both stages, the scales of k-step 0, the first half and weights of k-step 0
#pragma unroll
  for (int st = 0; st < NST; ++st)
#pragma unroll
    for (int g = 0; g < LPS; ++g) dload_one(st, st, g);
  stage_scales(0);
  RNL_MX_WAIT_VM_LGKM0(0);
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int i = 0; i < HM; ++i) read_a(0, i);
#pragma unroll
  for (int j = 0; j < NNI; ++j) read_b(0, j);

  int kt = 0;
  for (; kt < nk; ++kt) kstep(kt, kt & 1);
  RNL_MX_WAIT_VM_LGKM0(0);

  // epilogue: lane holds C[m][n .. n+3]
  const bool vec_ok = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < NMI; ++i) {
    const int m = m0 + wm * WM + i * 16 + (lane & 15);
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < NNI; ++j) {
      const int n = n0 + wn * WN + j * 16 + 4 * (lane >> 4);
      if (n >= N) continue;
      const size_t off = (size_t)m * (size_t)N + (size_t)n;
      const bool full = vec_ok && (n + 3 < N);
      const f32x4 v = acc[i][j];
      if constexpr (OUT_BF16) {
        uint16_t* c = static_cast<uint16_t*>(C) + off;
        if (full) {
          *reinterpret_cast<u32x2*>(c) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        } else {
          for (int r = 0; r < 4 && n + r < N; ++r) c[r] = (uint16_t)(pack_bf16x2(v[r], 0.f) & 0xFFFFu);
        }
      } else {
        float* c = static_cast<float*>(C) + off;
        if (full) {
          *reinterpret_cast<f32x4*>(c) = v;
        } else {
          for (int r = 0; r < 4 && n + r < N; ++r) c[r] = v[r];
        }
      }
    }
  }
}

#undef RNL_MX_WAIT_VM_LGKM0

int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <int BM, int BN, int WMW = 2, int WNW = 2>
hipError_t launch_mx_tile(const uint8_t* A, const uint8_t* B, const uint8_t* As, const uint8_t* Bs, void* C,
                          bool out_bf16, int64_t M, int64_t N, int64_t K, hipStream_t s) {
  const int tiles_m = (int)cdiv64(M, BM), tiles_n = (int)cdiv64(N, BN);
  const dim3 grid((unsigned)(tiles_m * tiles_n)), block(64 * WMW * WNW);
  if (out_bf16)
    hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, true, WMW, WNW>), grid, block, 0, s, A, B, As, Bs, C, (int)M, (int)N,
                       (int)K, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL((gemm_mx_kernel<BM, BN, false, WMW, WNW>), grid, block, 0, s, A, B, As, Bs, C, (int)M, (int)N,
                       (int)K, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mx(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs, void* C,
                          int out_kind, int64_t M, int64_t N, int64_t K, hipStream_t s) {
  const bool ob = out_kind == OUT_BF16;
  // largest tile that still gives every CU a workgroup
  if (cdiv64(M, 256) * cdiv64(N, 192) >= 256) return launch_mx_tile<256, 192, 4, 2>(A, B, As, Bs, C, ob, M, N, K, s);
  if (cdiv64(M, 256) * cdiv64(N, 128) >= 256) return launch_mx_tile<256, 128>(A, B, As, Bs, C, ob, M, N, K, s);
  if (cdiv64(M, 128) * cdiv64(N, 256) >= 256) return launch_mx_tile<128, 256>(A, B, As, Bs, C, ob, M, N, K, s);
  return launch_mx_tile<128, 128>(A, B, As, Bs, C, ob, M, N, K, s);
}

}  // namespace rnl
