// Tiled MFMA GEMM for the projection step: C[M,N] = A[M,K] . B[N,K]^T (b_trans).
//
// A is the normed activation (bf16, or per-token int8), B the weight stored
// [N, K] (AT-10 page section 2: the weight enters transposed).  Both
// operands are K-contiguous and staged through LDS identically: a k-step is 128
// bytes of every tile row (64 bf16 or 128 int8), cut into 16-byte chunks, and
// one chunk is exactly one lane's MFMA operand:
//   bf16: v_mfma_f32_16x16x32_bf16  (8 bf16 per lane, fp32 accumulation)
//   int8: v_mfma_i32_16x16x64_i8    (16 int8 per lane, int32 accumulation)
// A k-step therefore holds two MFMA k-chunks ("halves").
//
// Workgroup: WMW x WNW wavefronts over a BM x BN tile: 8 (two per SIMD, 4 x 2)
// for the 256 x 192 tile (64 x 96 each) and the 128 x 128 one (32 x 64 each),
// whose two wavefronts per SIMD hide each other's LDS reads; 4 (one per SIMD,
// 2 x 2) for the others.  The weight fragment is the
// MFMA "A" source and the activation fragment the "B" source, so each lane ends
// up with 4 consecutive output columns of one token row and stores them as one
// vector.
//
// Pipeline (one barrier per k-step):
//   * global -> LDS with buffer_load ... lds (direct-to-LDS DMA, no VGPR
//     staging); out-of-range rows and the K tail read as zero;
//   * NST LDS stages; a stage is refilled as soon as every wavefront has read
//     its fragments, so NST-1 stages are in flight;
//   * per half: the MFMAs of the fragments already in registers are issued
//     interleaved with the LDS reads of the next half's fragments and with the
//     DMA loads of the refill, in fixed groups, so the in-order issue of a
//     wavefront never stalls behind a burst of memory instructions.
// LDS layout: row-major, 128 bytes per row, 16-byte chunk c of row r stored at
// slot c ^ (r & 7); the 16 lanes that read one MFMA operand column then hit
// distinct banks (measured conflict-free on gfx950).
//
// Workgroup ids are remapped so that each of the 8 XCDs (dispatched
// round-robin) works on a contiguous block of tiles, grouped GROUP_M tiles
// tall, which share A and B panels in that XCD's L2.
//
// The kernel template lives in this header so that the bf16 and int8 instantiations
// can be compiled as separate units with different code-generation options.
//
// Split-K: with KSPLIT > 1 the grid holds KSPLIT workgroups per tile, each
// reducing one contiguous range of k-steps and writing a partial tile (fp32 or
// int32) to slice z of a [KSPLIT, M, N] buffer; the caller reduces the slices.
#pragma once

#include "common.hpp"
#include "launch.h"
#include "rows.hpp"

namespace rnl {
namespace gemm_detail {

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

enum Epi : int {
  EPI_BF16 = 0,      // C bf16 = round(acc)
  EPI_F32 = 1,       // C fp32 = acc
  EPI_I32 = 2,       // C int32 = acc
  EPI_DEQ_BF16 = 3,  // C bf16 = round(fl(float(acc) * fl(xs[m] * ws[n])))
  EPI_DEQ_F32 = 4,   // C fp32 = fl(float(acc) * fl(xs[m] * ws[n]))
  EPI_PART = 5,      // C[z] = acc (fp32 or int32 partial of split z)
  EPI_HEADS = 6,     // C bf16 = round(acc), then the per-head stage (HeadArgs) on whole heads of the tile
};

// s_waitcnt with vmcnt(n), lgkmcnt(0), expcnt unchanged (gfx9 encoding)
#define RNL_WAIT_VM_LGKM0(n) __builtin_amdgcn_s_waitcnt(0x0070 | ((n) & 15) | (((n) >> 4) << 14))

// WPE: workgroups per CU the kernel is built for (1, or 2 for tiles that fit twice
// in LDS and in half the register file); WMW x WNW: the wavefront grid (M x N).
template <typename TIn, int BM, int BN, int NST, int GROUP_M, int EPI, int WPE = 1, int WNW = 2, int WMW = 2>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WMW * WNW, 64 * WMW * WNW), amdgpu_waves_per_eu(WPE * WMW * WNW / 4, WPE * WMW * WNW / 4)))
void gemm_nt_kernel(const TIn* __restrict__ A, const TIn* __restrict__ B, void* __restrict__ C,
                    const float* __restrict__ xs, const float* __restrict__ ws, int M, int N, int K,
                    int tiles_m, int tiles_n, int ksplit, int steps_per_split, const HeadArgs ha) {
  using Acc = typename Mfma<TIn>::Acc;
  constexpr int ROWB = 128;
  constexpr int NWV = WMW * WNW;       // wavefronts: WMW along M x WNW along N
  constexpr int A_CH = BM / (8 * NWV);  // DMA instructions per wave and stage for A
  constexpr int B_CH = BN / (8 * NWV);
  static_assert(A_CH * 8 * NWV == BM && B_CH * 8 * NWV == BN, "DMA rows must split evenly over the waves");
  constexpr int LPS = A_CH + B_CH;    // DMA instructions per wave and stage
  constexpr int WM = BM / WMW, WN = BN / WNW;
  constexpr int NMI = WM / 16, NNI = WN / 16;
  constexpr int NF = NMI + NNI;       // fragment reads per half
  constexpr int NMM = NMI * NNI;      // MFMAs per half
  constexpr int STAGE = (BM + BN) * ROWB;
  static_assert(BM % 32 == 0 && BN % 32 == 0, "tile rows must be multiples of 32");
  static_assert(LPS * (NST - 1) < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WNW, wn = wave % WNW;

  // workgroup -> (split, tile): contiguous range per XCD, grouped along M inside it
  const int bid = blockIdx.x, nwg = gridDim.x;
  const int logical = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;
  const int z = logical % ksplit;
  const int tile = logical / ksplit;
  const int per_group = GROUP_M * tiles_n;
  const int group = tile / per_group;
  const int first_m = group * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int in_group = tile - group * per_group;
  const int tm = first_m + in_group % gm;
  const int tn = in_group / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  const uint32_t kbytes = (uint32_t)K * (uint32_t)sizeof(TIn);
  const int nk_all = (int)((kbytes + ROWB - 1) / ROWB);
  const int kbeg = min(nk_all, z * steps_per_split);
  const int nk = min(nk_all, kbeg + steps_per_split) - kbeg;
  const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (size_t)m0 * K, (uint32_t)rows_a * kbytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + (size_t)n0 * K, (uint32_t)rows_b * kbytes);

  // DMA: one instruction fills 8 consecutive tile rows (1 KiB); lane -> row lane/8, slot lane%8
  const int drow = lane >> 3, dslot = lane & 7;
  const int dchunk = dslot ^ drow;  // the chunk that lands in this lane's slot
  const uint32_t d_goff = (uint32_t)drow * kbytes + (uint32_t)dchunk * 16u;
  auto dload_one = [&](int kt, int buf, int g) {
    const uint32_t kb = (uint32_t)(kbeg + kt) * ROWB;
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

  // fragment reads: operand row = lane & 15, chunk = half * 4 + (lane >> 4)
  const int frow = lane & 15;
  const uint32_t foff0 = (uint32_t)frow * ROWB + (uint32_t)(((lane >> 4) ^ (frow & 7)) * 16);
  const uint32_t foff1 = (uint32_t)frow * ROWB + (uint32_t)(((4 + (lane >> 4)) ^ (frow & 7)) * 16);
  struct Frag {
    u32x4 a[NMI];
    u32x4 b[NNI];
  };
  auto fload_one = [&](Frag& f, int buf, int half, int q) {
    const uint32_t fo = half ? foff1 : foff0;
    if (q < NMI)
      f.a[q] = *reinterpret_cast<const u32x4*>(smem + buf * STAGE + (wm * WM + q * 16) * ROWB + fo);
    else
      f.b[q - NMI] = *reinterpret_cast<const u32x4*>(smem + buf * STAGE + (BM + wn * WN + (q - NMI) * 16) * ROWB + fo);
  };

  Acc acc[NMI][NNI];
#pragma unroll
  for (int i = 0; i < NMI; ++i)
#pragma unroll
    for (int j = 0; j < NNI; ++j) acc[i][j] = Acc{0, 0, 0, 0};
  auto mma_one = [&](const Frag& f, int t) {
    const int i = t / NNI, j = t % NNI;
    acc[i][j] = Mfma<TIn>::mma(f.b[j], f.a[i], acc[i][j]);
  };

  // MFMAs of Fc, interleaved with the reads of (fbuf, fhalf) into Fn (if fhalf >= 0) and
  // with the DMA refill of k-step dk into stage dbuf (if dk >= 0)
  auto phase = [&](const Frag& Fc, Frag& Fn, int fbuf, int fhalf, int dk, int dbuf) {
    constexpr int G = LPS > (NF + 1) / 2 ? LPS : (NF + 1) / 2;
    constexpr int MPG = NMM / G;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (dk >= 0 && g < LPS) dload_one(dk, dbuf, g);
      if (fhalf >= 0 && 2 * g < NF) fload_one(Fn, fbuf, fhalf, 2 * g);
      if (fhalf >= 0 && 2 * g + 1 < NF) fload_one(Fn, fbuf, fhalf, 2 * g + 1);
#pragma unroll
      for (int t = g * MPG; t < (g + 1) * MPG; ++t) mma_one(Fc, t);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = G * MPG; t < NMM; ++t) mma_one(Fc, t);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Per-head epilogue.  The bf16-rounded tile goes to LDS (the stages are free once every
  // wavefront is past its last fragment read); each group of GP lanes then takes RPG token rows
  // of the tile and, row by row, its HPT heads: lane q holds elements 8q .. 8q+7 and
  // D/2+8q .. D/2+8q+7, the layout of the standalone per-head kernel, and the same arithmetic
  // (head_sumsq, group_sum, head_chunks) gives the same bits.  Value heads are stored as they
  // are.  The head gammas and the rows' angles are requested before the tile is staged, so
  // that no step of the loop waits for global memory.
  auto heads_epilogue = [&](const HeadArgs& h) {
    if constexpr (EPI == EPI_HEADS) {
      constexpr int HD = kHeadEpiD, GP = HD / 16, HPT = BN / HD, NG = NWV * (kWave / GP);
      constexpr int RPG = BM / NG;  // token rows per lane group
      constexpr int LDY = BN + 8;   // bf16 per LDS tile row (padded)
      static_assert(sizeof(TIn) == 2 && BN % HD == 0, "whole bf16 heads per tile");
      static_assert(BM * LDY * 2 <= NST * STAGE, "the output tile fits the stages");
      static_assert(RPG * NG == BM, "whole rows per lane group");
      const int grp = wave * (kWave / GP) + lane / GP, gl = lane & (GP - 1);
      const int c0 = gl * 8, c1 = c0 + HD / 2;
      const bool rope = h.cos_t != nullptr;
      const bool gq_on = h.gamma_q != nullptr, gk_on = h.gamma_k != nullptr;
      u32x4 gq0{}, gq1{}, gk0{}, gk1{};
      if (gq_on) {
        gq0 = *reinterpret_cast<const u32x4*>(h.gamma_q + c0);
        gq1 = *reinterpret_cast<const u32x4*>(h.gamma_q + c1);
      }
      if (gk_on) {
        gk0 = *reinterpret_cast<const u32x4*>(h.gamma_k + c0);
        gk1 = *reinterpret_cast<const u32x4*>(h.gamma_k + c1);
      }
      f32x4 cs[RPG][2], sn[RPG][2];
      if (rope) {
#pragma unroll
        for (int j = 0; j < RPG; ++j) {
          const int t = m0 + grp + j * NG;
          const size_t ab = (size_t)(t < M ? t : 0) * (HD / 2) + c0;  // a row that exists, for rows past M
          cs[j][0] = *reinterpret_cast<const f32x4*>(h.cos_t + ab);
          cs[j][1] = *reinterpret_cast<const f32x4*>(h.cos_t + ab + 4);
          sn[j][0] = *reinterpret_cast<const f32x4*>(h.sin_t + ab);
          sn[j][1] = *reinterpret_cast<const f32x4*>(h.sin_t + ab + 4);
        }
      }
      uint16_t* ty = reinterpret_cast<uint16_t*>(smem);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < NMI; ++i)
#pragma unroll
        for (int j = 0; j < NNI; ++j)
          *reinterpret_cast<u32x2*>(ty + (wm * WM + i * 16 + (lane & 15)) * LDY + wn * WN + j * 16 + 4 * (lane >> 4)) =
              u32x2{pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3])};
      __syncthreads();
      const int nqk = h.hq + h.hkv;
      uint16_t* y = static_cast<uint16_t*>(C);
#pragma unroll
      for (int j = 0; j < RPG; ++j) {
        const int r = grp + j * NG, t = m0 + r;
#pragma unroll
        for (int hh = 0; hh < HPT; ++hh) {
          const int col = n0 + hh * HD, hg = col / HD;
          const uint16_t* src = ty + r * LDY + hh * HD;
          const u32x4 v0 = *reinterpret_cast<const u32x4*>(src + c0);
          const u32x4 v1 = *reinterpret_cast<const u32x4*>(src + c1);
          const bool qk = hg < nqk, is_q = hg < h.hq;
          const float rstd = rstd_from_sumsq(group_sum<GP>(head_sumsq(v0, v1)), h.inv_d, h.eps);
          u32x4 o0 = v0, o1 = v1;
          if (qk) {
            const bool g_on = is_q ? gq_on : gk_on;
            const u32x4 g0 = is_q ? gq0 : gk0, g1 = is_q ? gq1 : gk1;
            if (rope) head_chunks<true>(v0, v1, g0, g1, g_on, cs[j], sn[j], rstd, o0, o1);
            else head_chunks<false>(v0, v1, g0, g1, g_on, cs[j], sn[j], rstd, o0, o1);
          }
          if (t < M && col < N) {
            uint16_t* dst = y + (size_t)t * (size_t)N + (size_t)col;
            *reinterpret_cast<u32x4*>(dst + c0) = o0;
            *reinterpret_cast<u32x4*>(dst + c1) = o1;
            if (qk && gl == 0 && h.rstd_out != nullptr) h.rstd_out[(size_t)t * (size_t)nqk + hg] = rstd;
          }
        }
      }
    }
  };

  // Dequant scales of this wavefront's rows and columns, requested before the first stages
  // so that they have long landed when the epilogue needs them (loading them per element in
  // the epilogue made it three times as long as the plain int32 one).  Out-of-range rows and
  // columns read as zero; their outputs are never stored.
  constexpr bool DEQ = EPI == EPI_DEQ_BF16 || EPI == EPI_DEQ_F32;
  float xs_r[DEQ ? NMI : 1], ws_r[DEQ ? NNI : 1][4];
  if constexpr (DEQ) {
    const __amdgpu_buffer_rsrc_t rxs = make_rsrc(xs, (uint32_t)M * 4u);
    const __amdgpu_buffer_rsrc_t rws = make_rsrc(ws, (uint32_t)N * 4u);
#pragma unroll
    for (int i = 0; i < NMI; ++i)
      xs_r[i] = __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(rxs, (uint32_t)(m0 + wm * WM + i * 16 + (lane & 15)) * 4u, 0, 0));
#pragma unroll
    for (int j = 0; j < NNI; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        ws_r[j][r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            rws, (uint32_t)(n0 + wn * WN + j * 16 + 4 * (lane >> 4) + r) * 4u, 0, 0));
  }

  // Every stage slot is always filled (k-steps past the range read as zero), so the
  // number of DMA loads in flight is the same at every wait.
#pragma unroll
  for (int st = 0; st < NST; ++st)
#pragma unroll
    for (int g = 0; g < LPS; ++g) dload_one(st, st, g);
  RNL_WAIT_VM_LGKM0((NST - 1) * LPS);
  __builtin_amdgcn_s_barrier();

  Frag F0, F1;
#pragma unroll
  for (int q = 0; q < NF; ++q) fload_one(F0, 0, 0, q);
  int slot = 0;
  for (int kt = 0; kt < nk - 1; ++kt) {
    const int nslot = (slot + 1 == NST) ? 0 : slot + 1;
    phase(F0, F1, slot, 1, -1, 0);  // first half: read the second half's fragments
    // k-step kt+1 has landed and this wave's reads of stage `slot` are complete
    RNL_WAIT_VM_LGKM0((NST - 2) * LPS);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    phase(F1, F0, nslot, 0, kt + NST, slot);  // second half: refill `slot`, read next first half
    slot = nslot;
  }
  // last k-step (an empty split range only ever loaded zero-filled stages, so these
  // MFMAs add nothing and need no guard)
  phase(F0, F1, slot, 1, -1, 0);
  phase(F1, F0, 0, -1, -1, 0);
  RNL_WAIT_VM_LGKM0(0);

  if constexpr (EPI == EPI_HEADS) {
    heads_epilogue(ha);
    return;
  }

  // epilogue: lane holds C[m][n .. n+3]
  const bool vec_ok = (N & 3) == 0;
#pragma unroll
  for (int i = 0; i < NMI; ++i) {
    const int m = m0 + wm * WM + i * 16 + (lane & 15);
    if (m >= M) continue;
    float xsm = 0.f;
    if constexpr (DEQ) xsm = xs_r[i];
#pragma unroll
    for (int j = 0; j < NNI; ++j) {
      const int n = n0 + wn * WN + j * 16 + 4 * (lane >> 4);
      if (n >= N) continue;
      const size_t off = (size_t)m * (size_t)N + (size_t)n;
      const bool full = vec_ok && (n + 3 < N);
      if constexpr (EPI == EPI_I32 || (EPI == EPI_PART && sizeof(TIn) == 1)) {
        int32_t* c = static_cast<int32_t*>(C) + off;
        if constexpr (EPI == EPI_PART) c += (size_t)z * (size_t)M * (size_t)N;
        if (full) {
          *reinterpret_cast<i32x4*>(c) = acc[i][j];
        } else {
          for (int r = 0; r < 4 && n + r < N; ++r) c[r] = acc[i][j][r];
        }
      } else {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (DEQ) {
            v[r] = __fmul_rn((float)acc[i][j][r], __fmul_rn(xsm, ws_r[j][r]));
          } else {
            v[r] = (float)acc[i][j][r];
          }
        }
        if constexpr (EPI == EPI_F32 || EPI == EPI_DEQ_F32 || EPI == EPI_PART) {
          float* c = static_cast<float*>(C) + off;
          if constexpr (EPI == EPI_PART) c += (size_t)z * (size_t)M * (size_t)N;
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
            for (int r = 0; r < 4 && n + r < N; ++r) c[r] = (uint16_t)(pack_bf16x2(v[r], 0.f) & 0xFFFFu);
          }
        }
      }
    }
  }
}

#undef RNL_WAIT_VM_LGKM0

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// GM: tiles per group along M (each XCD's run of tiles covers GM tile rows, so the wider the
// weight panel relative to the activation panel, the more tile rows a group should hold)
template <typename TIn, int BM, int BN, int NST, int EPI, int WPE = 1, int WNW = 2, int WMW = 2, int GM = 4>
hipError_t launch_tile(const TIn* A, const TIn* B, void* C, const float* xs, const float* ws, int64_t M,
                       int64_t N, int64_t K, int ksplit, hipStream_t s, const HeadArgs& ha = HeadArgs{}) {
  const int tiles_m = (int)cdiv(M, BM), tiles_n = (int)cdiv(N, BN);
  const int nk = (int)cdiv(K * (int64_t)sizeof(TIn), 128);
  const int sps = (int)cdiv(nk, ksplit);
  const int nwg = tiles_m * tiles_n * ksplit;
  hipLaunchKernelGGL((gemm_nt_kernel<TIn, BM, BN, NST, GM, EPI, WPE, WNW, WMW>), dim3(nwg), dim3(64 * WMW * WNW), 0, s, A, B, C,
                     xs, ws, (int)M, (int)N, (int)K, tiles_m, tiles_n, ksplit, sps, ha);
  return hipGetLastError();
}

// Tile shapes, largest first: 256x192 (2 LDS stages, 112 KiB), 256x128 and 128x256
// (3 stages, 144 KiB), 128x128 (4 stages, 128 KiB); and 128x128 with 2 stages
// (64 KiB), two workgroups per CU, so that one tile's prologue, barriers and
// output writes overlap the other's k-loop (used by the int8 GEMM); 128x96 (3
// stages, 84 KiB) for split-K stages whose 128x128 tiles would leave CUs idle.
enum Shape { S256x192, S256x128, S128x256, S128x128, S128x128_2PerCU, S128x96 };

inline Shape pick_shape(int64_t M, int64_t N) {
  // Largest tile that still gives every CU at least one workgroup.
  if (cdiv(M, 256) * cdiv(N, 192) >= 256) return S256x192;
  if (cdiv(M, 256) * cdiv(N, 128) >= 256) return S256x128;
  if (cdiv(M, 128) * cdiv(N, 256) >= 256) return S128x256;
  return S128x128;
}

template <typename TIn, int EPI>
hipError_t launch_shape(Shape sh, const TIn* A, const TIn* B, void* C, const float* xs, const float* ws,
                        int64_t M, int64_t N, int64_t K, int ksplit, hipStream_t s) {
  switch (sh) {
    case S256x192: return launch_tile<TIn, 256, 192, 2, EPI, 1, 2, 4>(A, B, C, xs, ws, M, N, K, ksplit, s);
    case S256x128: return launch_tile<TIn, 256, 128, 3, EPI>(A, B, C, xs, ws, M, N, K, ksplit, s);
    case S128x256: return launch_tile<TIn, 128, 256, 3, EPI>(A, B, C, xs, ws, M, N, K, ksplit, s);
    case S128x128_2PerCU: return launch_tile<TIn, 128, 128, 2, EPI, 2>(A, B, C, xs, ws, M, N, K, ksplit, s);
    case S128x96: return launch_tile<TIn, 128, 96, 3, EPI>(A, B, C, xs, ws, M, N, K, ksplit, s);
    default: return launch_tile<TIn, 128, 128, 4, EPI, 1, 2, 4>(A, B, C, xs, ws, M, N, K, ksplit, s);
  }
}

}  // namespace gemm_detail
}  // namespace rnl
