// Measurement probes, not steps of the method:
//   * a read-only HBM streaming probe, the practical ceiling the weight-bound
//     paths are measured against;
//   * a clock probe: one wavefront that spins for a fixed wall time and counts
//     shader clock ticks (s_memtime) against the 100 MHz real-time counter
//     (s_memrealtime), run beside a workload to record the clock it runs at;
//   * an MFMA rate probe: every wavefront issues a fixed number of matrix
//     instructions on register operands into eight independent accumulators,
//     no memory traffic, the practical ceiling the contractions are measured
//     against.
//
// The given number of workgroups of 256 threads read the buffer once with
// 16-byte loads (each load instruction of a wavefront covers 1 KiB contiguous),
// U loads in flight per thread, in a grid-stride loop; each workgroup folds what
// it read into one word (XOR) and stores it, so the loads cannot be dropped.
#include "common.hpp"
#include "launch.h"

namespace rnl {
namespace {

template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[4];
  const size_t stride = (size_t)gridDim.x * 256;
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = (i + u * stride < n16) ? src[i + u * stride] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, kWave);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// Spins until `ticks` periods of the 100 MHz real-time counter have passed (a
// bounded wait: it ends whatever else runs), then stores the elapsed shader
// clocks and real-time ticks.
// Workgroup b writes out[2b], out[2b + 1]; with 8 workgroups each XCD gets one
// (workgroups are dealt round-robin over the XCDs).  `delay` real-time ticks
// pass before counting starts.
__global__ __launch_bounds__(64) void clock_probe_kernel(uint64_t* __restrict__ out, uint64_t delay, uint64_t ticks) {
  const uint64_t s0 = __builtin_amdgcn_s_memrealtime();
  uint64_t r0 = s0;
  while (r0 - s0 < delay) {
    __builtin_amdgcn_s_sleep(2);
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  uint64_t r1 = r0;
  while (r1 - r0 < ticks) {
    __builtin_amdgcn_s_sleep(2);
    r1 = __builtin_amdgcn_s_memrealtime();
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = c1 - c0;
    out[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// MFMA rate probe.  KIND 0: v_mfma_f32_16x16x32_bf16 (16384 flop), 1:
// v_mfma_i32_16x16x64_i8 (32768 op), 2: v_mfma_scale_f32_16x16x128_f8f6f4 with
// E4M3 operands (65536 flop).  The operands are derived from the lane id so that
// nothing folds; each wavefront stores a fold of its accumulators to
// sink[global wavefront id], so the work is kept.
typedef int i32x8 __attribute__((ext_vector_type(8)));
constexpr int kProbeAcc = 8;

template <int KIND>
__global__ void mfma_probe_kernel(uint32_t* __restrict__ sink, int iters) {
  const uint32_t lane = threadIdx.x & 63;
  uint32_t fold = 0;
  if constexpr (KIND == 0) {
    // bf16 values near 2^-8: the sums stay finite over any iteration count used here
    const uint32_t w = 0x3B803B80u ^ (lane & 7u);
    const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{w, w ^ 1u, w ^ 2u, w ^ 3u});
    const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{w ^ 4u, w ^ 5u, w ^ 6u, w ^ 7u});
    f32x4 acc[kProbeAcc];
#pragma unroll
    for (int j = 0; j < kProbeAcc; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < kProbeAcc; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kProbeAcc; ++j) fold ^= __float_as_uint(acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3]);
  } else if constexpr (KIND == 1) {
    const i32x4 a = i32x4{(int)(0x01010101u ^ lane), 0x01010101, 0x01010101, 0x01010101};
    const i32x4 b = i32x4{0x01010101, (int)(0x01010101u ^ (lane << 8)), 0x01010101, 0x01010101};
    i32x4 acc[kProbeAcc];
#pragma unroll
    for (int j = 0; j < kProbeAcc; ++j) acc[j] = i32x4{0, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < kProbeAcc; ++j) acc[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < kProbeAcc; ++j) fold ^= (uint32_t)(acc[j][0] ^ acc[j][1] ^ acc[j][2] ^ acc[j][3]);
  } else {
    // E4M3 0x30 = 0.5; scales 127 = 2^0
    const int v = (int)(0x30303030u ^ (lane & 1u));
    const i32x8 a = i32x8{v, v, v, v, v, v, v, v};
    const i32x8 b = i32x8{v, v, v, v, v, v, v, 0x30303030};
    f32x4 acc[kProbeAcc];
#pragma unroll
    for (int j = 0; j < kProbeAcc; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int j = 0; j < kProbeAcc; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[j], 0, 0, 0, 127, 0, 127);
    }
#pragma unroll
    for (int j = 0; j < kProbeAcc; ++j) fold ^= __float_as_uint(acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) fold ^= __shfl_xor(fold, off, kWave);
  if (lane == 0) sink[blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = fold;
}

}  // namespace

hipError_t launch_mfma_probe(int kind, int workgroups, int waves, int iters, uint32_t* sink, hipStream_t s) {
  const dim3 grid((unsigned)workgroups), block((unsigned)(64 * waves));
  switch (kind) {
    case 0: hipLaunchKernelGGL((mfma_probe_kernel<0>), grid, block, 0, s, sink, iters); break;
    case 1: hipLaunchKernelGGL((mfma_probe_kernel<1>), grid, block, 0, s, sink, iters); break;
    default: hipLaunchKernelGGL((mfma_probe_kernel<2>), grid, block, 0, s, sink, iters); break;
  }
  return hipGetLastError();
}

hipError_t launch_clock_probe(uint64_t* out, uint64_t delay, uint64_t ticks, int workgroups, hipStream_t s) {
  hipLaunchKernelGGL(clock_probe_kernel, dim3((unsigned)workgroups), dim3(64), 0, s, out, delay, ticks);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, int unroll,
                              hipStream_t s) {
  const u32x4* p = static_cast<const u32x4*>(src);
  const dim3 grid((unsigned)workgroups), block(256);
  switch (unroll) {
    case 1: hipLaunchKernelGGL((stream_read_kernel<1>), grid, block, 0, s, p, bytes / 16, sink); break;
    case 2: hipLaunchKernelGGL((stream_read_kernel<2>), grid, block, 0, s, p, bytes / 16, sink); break;
    case 4: hipLaunchKernelGGL((stream_read_kernel<4>), grid, block, 0, s, p, bytes / 16, sink); break;
    case 8: hipLaunchKernelGGL((stream_read_kernel<8>), grid, block, 0, s, p, bytes / 16, sink); break;
    default: hipLaunchKernelGGL((stream_read_kernel<16>), grid, block, 0, s, p, bytes / 16, sink); break;
  }
  return hipGetLastError();
}

}  // namespace rnl
