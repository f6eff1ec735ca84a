// Device helpers shared by the gfx950 kernels of the fused RMSNorm -> Linear library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rnl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Buffer resource word 3 for gfx9-family raw buffers: 32-bit data format, no
// swizzle, no index stride; out-of-range loads return 0, stores are dropped.
constexpr int kBufWord3 = 0x00020000;
// An offset that is out of range for every resource we build (all are < 2 GiB).
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufWord3);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// bf16 <-> fp32.  Widening is exact; narrowing uses the hardware convert,
// which rounds to nearest even under the default mode register.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <class T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// rstd = 1 / sqrt(fl(fl(S * inv_k) + eps)) with IEEE-rounded multiply, add,
// square root and division (sqrtf and '/' are correctly rounded under the
// default HIP floating-point options; __fsqrt_rn is not).  The operators are
// written out under contract(off): under the default options __fmul_rn and
// __fadd_rn are plain '*' and '+' from a header where contraction into an FMA
// (one rounding instead of two) stays allowed.
__device__ __forceinline__ float rstd_from_sumsq(float S, float inv_k, float eps) {
#pragma clang fp contract(off)
  const float ms = S * inv_k;
  const float var = ms + eps;
  return 1.0f / sqrtf(var);
}

}  // namespace rnl
