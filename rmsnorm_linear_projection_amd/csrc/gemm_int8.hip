// int8 instantiations of the projection GEMM (kernel in gemm_kernel.hpp).  This unit
// is compiled with the MFMA accumulators in VGPRs (-amdgpu-mfma-vgpr-form): with
// AGPR accumulators the int32 MFMA loop gets its accumulators re-shuffled every
// iteration by the register allocator.
#include "gemm_kernel.hpp"

namespace rnl {
using namespace gemm_detail;

hipError_t launch_gemm_int8(const int8_t* A, const int8_t* B, void* C, int out_kind,
                            const float* xs, const float* ws, int64_t M, int64_t N, int64_t K,
                            hipStream_t s) {
  // When the largest tile cannot fill one round of CUs but 128x128 tiles give two
  // per CU, two co-resident 128x128 workgroups per CU are faster: an int8 k-step
  // carries twice the k of a bf16 one, so the fixed part of a tile weighs more
  // (2048 x 4096 x 4096: 37.2 us against 39.8 with 256x128).
  Shape sh = pick_shape(M, N);
  if (sh != S256x192 && cdiv(M, 128) * cdiv(N, 128) >= 512) sh = S128x128_2PerCU;
  if (out_kind == OUT_I32) return launch_shape<int8_t, EPI_I32>(sh, A, B, C, xs, ws, M, N, K, 1, s);
  if (out_kind == OUT_F32) return launch_shape<int8_t, EPI_DEQ_F32>(sh, A, B, C, xs, ws, M, N, K, 1, s);
  return launch_shape<int8_t, EPI_DEQ_BF16>(sh, A, B, C, xs, ws, M, N, K, 1, s);
}

}  // namespace rnl
