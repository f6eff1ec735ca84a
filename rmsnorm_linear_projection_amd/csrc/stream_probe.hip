// Measurement probes, not steps of the method:
//   * a read-only HBM streaming probe, the practical ceiling the weight-bound
//     paths are measured against;
//   * a clock probe: one wavefront that spins for a fixed wall time and counts
//     shader clock ticks (s_memtime) against the 100 MHz real-time counter
//     (s_memrealtime), run beside a workload to record the clock it runs at.
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

}  // namespace

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
