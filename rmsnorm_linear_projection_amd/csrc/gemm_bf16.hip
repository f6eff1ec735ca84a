// bf16 instantiations of the projection GEMM (kernel in gemm_kernel.hpp).
#include "gemm_kernel.hpp"

namespace rnl {
using namespace gemm_detail;

namespace {
int64_t split_tiles(Shape sh, int64_t M, int64_t N) {
  const int64_t bm = (sh == S256x192 || sh == S256x128) ? 256 : 128;
  const int64_t bn = sh == S256x192 ? 192 : (sh == S128x256 ? 256 : (sh == S128x96 ? 96 : 128));
  return cdiv(M, bm) * cdiv(N, bn);
}
// the largest power of two that keeps tiles x splits within one round of 256
// workgroups, with at least 8 k-steps per split
int64_t split_count(int64_t tiles, int64_t nk) {
  int64_t ks = 1;
  while (tiles * ks * 2 <= 256 && nk / (ks * 2) >= 8) ks *= 2;
  return ks;
}
}  // namespace

int gemm_split_plan(int64_t M, int64_t N, int64_t K, int elem_bytes, int* shape) {
  // For outputs too small to fill the chip, split K (a second, partial round of
  // workgroups and the extra fp32 partials cost more than the idle CUs:
  // 1024 x 1536 x 7168 runs 33 us with 2 splits, 41 us with 4).  When 128x128
  // tiles times the splits leave CUs idle and 128x96 tiles fill more of them,
  // take those: 1024 x 1536 gives 96 tiles x 2 = 192 workgroups against 128 x 2
  // = 256 (the split-K stage 28.3 against 30.1 us, identical partials).
  Shape sh = pick_shape(M, N);
  const int64_t nk = cdiv(K * elem_bytes, 128);
  int64_t ks = split_count(split_tiles(sh, M, N), nk);
  if (sh == S128x128 && ks > 1) {
    const int64_t t96 = split_tiles(S128x96, M, N), ks96 = split_count(t96, nk);
    if (t96 * ks96 > split_tiles(sh, M, N) * ks && ks96 > 1) {
      sh = S128x96;
      ks = ks96;
    }
  }
  if (shape != nullptr) *shape = (int)sh;
  return (int)ks;
}

hipError_t launch_gemm_bf16(const uint16_t* A, const uint16_t* B, void* C, int out_kind, int64_t M,
                            int64_t N, int64_t K, hipStream_t s) {
  const Shape sh = pick_shape(M, N);
  if (out_kind == OUT_F32) return launch_shape<uint16_t, EPI_F32>(sh, A, B, C, nullptr, nullptr, M, N, K, 1, s);
  return launch_shape<uint16_t, EPI_BF16>(sh, A, B, C, nullptr, nullptr, M, N, K, 1, s);
}

// The per-head epilogue needs whole heads in a tile: 128 x 384 (three heads of 128), eight
// wavefronts of 64 x 96 as in the 256 x 192 tile, two stages (128 KiB, which also hold the
// output tile).  At 4096 x 6144 it gives 512 tiles, two rounds of workgroups.  Groups of 8
// tile rows: with groups of 4, each XCD's round of 32 tiles spans 8 weight panels of 384
// rows, and the launch fetched 475 MB from HBM against 328 MB for the 256 x 192 GEMM.
hipError_t launch_gemm_bf16_heads(const uint16_t* A, const uint16_t* B, uint16_t* C, int64_t M, int64_t N,
                                  int64_t K, const HeadArgs& heads, hipStream_t s) {
  return launch_tile<uint16_t, 128, 384, 2, EPI_HEADS, 1, 4, 2, 8>(A, B, C, nullptr, nullptr, M, N, K, 1, s, heads);
}

hipError_t launch_gemm_bf16_splitk(const uint16_t* A, const uint16_t* B, float* partial, int64_t M,
                                   int64_t N, int64_t K, int ksplit, hipStream_t s) {
  // the tile shape of the split plan, whose split count the caller passes
  int sh = 0;
  gemm_split_plan(M, N, K, 2, &sh);
  return launch_shape<uint16_t, EPI_PART>((Shape)sh, A, B, partial, nullptr, nullptr, M, N, K, ksplit, s);
}

}  // namespace rnl
