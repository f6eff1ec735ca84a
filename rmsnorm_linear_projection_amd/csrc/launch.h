// Internal launchers of the gfx950 kernels.  Host code only; every launcher
// trusts its arguments (the C ABI validates them first) and returns the HIP
// status of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace rnl {

enum OutKind : int { OUT_BF16 = 1, OUT_F32 = 2, OUT_I32 = 4 };

// Row-wise RMSNorm pre-pass: one pass over each row computes the fp32 sum of
// squares, rstd, and writes the normed row either as bf16 (a_out) or as
// per-token symmetric int8 (q_out, x_scale_out).  rstd_out may be null.
hipError_t launch_norm_rows_bf16(const uint16_t* x, const uint16_t* gamma, float eps, int64_t T,
                                 int64_t K, uint16_t* a_out, float* rstd_out, hipStream_t s);
hipError_t launch_norm_rows_int8(const uint16_t* x, const uint16_t* gamma, float eps, int64_t T,
                                 int64_t K, int8_t* q_out, float* x_scale_out, float* rstd_out,
                                 hipStream_t s);
// The same, applied to x_add = bf16(x + residual) (sum in fp32), which is also
// written to x_add.
hipError_t launch_add_norm_rows_bf16(const uint16_t* x, const uint16_t* residual, uint16_t* x_add,
                                     const uint16_t* gamma, float eps, int64_t T, int64_t K, uint16_t* a_out,
                                     float* rstd_out, hipStream_t s);
hipError_t launch_add_norm_rows_int8(const uint16_t* x, const uint16_t* residual, uint16_t* x_add,
                                     const uint16_t* gamma, float eps, int64_t T, int64_t K, int8_t* q_out,
                                     float* x_scale_out, float* rstd_out, hipStream_t s);
// x_add = bf16(x + residual) alone.
hipError_t launch_add_rows(const uint16_t* x, const uint16_t* residual, uint16_t* x_add, int64_t T, int64_t K,
                           hipStream_t s);
// Same norm (bf16 out) applied to rows that are the bf16 rounding of the sum of S
// fp32 split-K partials, added in split order: row t of slice z starts at
// part + z * T * ld + t * ld (ld >= K, a multiple of 8); out is [T, K].  When
// sum_out is not null the bf16 row sums (the rows the norm reads) are also
// written, row t at sum_out + t * sum_ld (sum_ld a multiple of 8).
hipError_t launch_reduce_norm_bf16(const float* part, int S, int64_t ld, const uint16_t* gamma, float eps,
                                   int64_t T, int64_t K, uint16_t* out, float* rstd_out, uint16_t* sum_out,
                                   int64_t sum_ld, hipStream_t s);
// Two column ranges of the same rows normed on their own in one launch: the K
// columns from col0 (a multiple of 8) with their gamma, to out [T, K] and rstd_out.
struct NormCols {
  int64_t col0, K;
  const uint16_t* gamma;
  uint16_t* out;
  float* rstd_out;
};
// launch_reduce_norm_bf16 for two column ranges of the partial rows (sum_out, when
// not null, receives both ranges' bf16 sums at their columns, row stride ld).
hipError_t launch_reduce_norm_pair_bf16(const float* part, int S, int64_t ld, int64_t T, const NormCols& a,
                                        const NormCols& b, float eps, uint16_t* sum_out, hipStream_t s);
// The same for bf16 rows with stride ld (row t at x + t * ld; ld a multiple of 8).
hipError_t launch_norm_rows_pair_bf16_strided(const uint16_t* x, int64_t ld, int64_t T, const NormCols& a,
                                              const NormCols& b, float eps, hipStream_t s);

// Per-head RMSNorm (+ rotate-half RoPE when cos_t/sin_t are given) of the H
// heads of D columns that start at column col0 of y_in[T, ld] (bf16), written
// to the same places of y_out (which may be y_in).  Heads h < H1 take gamma1,
// the rest gamma2 (either may be null); cos_t/sin_t are [T, D/2] fp32;
// rstd_out [T, H] may be null.  D is a multiple of 16, at most 512.
hipError_t launch_head_norm_bf16(const uint16_t* y_in, uint16_t* y_out, int64_t T, int64_t ld, int64_t col0,
                                 int64_t H, int64_t D, int64_t H1, const uint16_t* gamma1, const uint16_t* gamma2,
                                 float eps, const float* cos_t, const float* sin_t, float* rstd_out,
                                 hipStream_t s);

// C[M,N] = A[M,K] . B[N,K]^T on bf16 MFMA, fp32 accumulation, C bf16 or fp32.
hipError_t launch_gemm_bf16(const uint16_t* A, const uint16_t* B, void* C, int out_kind, int64_t M,
                            int64_t N, int64_t K, hipStream_t s);

// Per-head stage applied inside the GEMM's epilogue (the pre-attention block):
// the columns of C are hq query heads, then hkv key heads, then value heads, of
// kHeadEpiD columns each; query and key heads are normed and rotated exactly as
// launch_head_norm_bf16 does (gamma_q for query heads, gamma_k for key heads,
// cos / sin both null for no rotation), value heads are the bf16 product.
constexpr int kHeadEpiD = 128;
struct HeadArgs {
  const uint16_t* gamma_q;  // [D] bf16 or null
  const uint16_t* gamma_k;  // [D] bf16 or null
  const float* cos_t;       // [M, D/2] fp32 or null
  const float* sin_t;       // [M, D/2] fp32 or null
  float* rstd_out;          // [M, hq + hkv] or null
  float eps;
  float inv_d;              // fl(1/D)
  int hq, hkv;
};
// C = bf16(A . B^T) with the per-head stage in the epilogue; N = (hq + 2 hkv) D.
hipError_t launch_gemm_bf16_heads(const uint16_t* A, const uint16_t* B, uint16_t* C, int64_t M, int64_t N,
                                  int64_t K, const HeadArgs& heads, hipStream_t s);

// Number of K splits the bf16/int8 GEMM would use for an output of M x N (1 when
// the tiles alone fill the chip); elem_bytes is the operand size.
int gemm_split_plan(int64_t M, int64_t N, int64_t K, int elem_bytes, int* shape);
// Split-K bf16 GEMM: partial[z, M, N] (fp32) for z < ksplit; sum over z is A . B^T.
hipError_t launch_gemm_bf16_splitk(const uint16_t* A, const uint16_t* B, float* partial, int64_t M,
                                   int64_t N, int64_t K, int ksplit, hipStream_t s);

// acc[M,N] = A[M,K] . B[N,K]^T on int8 MFMA (int32 accumulation).  With
// out_kind OUT_I32 C receives acc; otherwise C = fl(float(acc) * fl(xs[m] * ws[n]))
// as bf16 or fp32.
hipError_t launch_gemm_int8(const int8_t* A, const int8_t* B, void* C, int out_kind,
                            const float* xs, const float* ws, int64_t M, int64_t N, int64_t K,
                            hipStream_t s);

// RMSNorm, then MX quantisation of the fp32 normed rows: q_out [T, K] E4M3 codes,
// s_out [T, K/64] E8M0 scales (one per 64 consecutive values).  K % 64 == 0.
hipError_t launch_norm_rows_mx(const uint16_t* x, const uint16_t* gamma, float eps, int64_t T, int64_t K,
                               uint8_t* q_out, uint8_t* s_out, float* rstd_out, hipStream_t s);

// MXFP8 GEMM: C[M,N] = sum over 64-blocks of As * Bs * (A . B^T) with E4M3
// A[M,K], B[N,K] and E8M0 scales As[M,K/64], Bs[N,K/64]; C bf16 or fp32.
hipError_t launch_gemm_mx(const uint8_t* A, const uint8_t* As, const uint8_t* B, const uint8_t* Bs, void* C,
                          int out_kind, int64_t M, int64_t N, int64_t K, hipStream_t s);

// C[M,N] = A[M,K] . W[N,K]^T for M <= 16 (weight streaming), bf16 or fp32 out.
// R = weight rows per workgroup (a multiple of 4, at most 32), or 0 to let
// small_m_rows(N) spread the rows evenly over the compute units.
int small_m_rows(int64_t N);
// The same with the RMSNorm of the raw rows X[M,K] fused in (M <= 16): y = bf16(
// RMSNorm(X) * gamma) . W^T; rstd_out [M] may be null.  The normed rows live in
// LDS: small_m_norm_lds(M, K) bytes, which must not exceed kSmallNormLds.
constexpr size_t kSmallNormLds = 64 * 1024;
size_t small_m_norm_lds(int64_t M, int64_t K);
// Two prologues, both for normed rows within kSmallNormLds: up to
// kFusedNormRowsM rows normed one at a time, or kFusedNormRowsM < M <=
// kFusedNormAllM rows of at most kFusedNormAllK values, every row requested at
// once.  small_m_norm_fits tells whether either applies.
constexpr int64_t kFusedNormRowsM = 4;
constexpr int64_t kFusedNormAllM = 16;
constexpr int64_t kFusedNormAllK = 4096;
constexpr size_t kSmallNormLdsAllRows = kSmallNormLds;
bool small_m_norm_fits(int64_t M, int64_t K);
hipError_t launch_small_m_norm_bf16(const uint16_t* X, const uint16_t* gamma, float eps, const uint16_t* W,
                                    void* C, int out_kind, float* rstd_out, int64_t M, int64_t N, int64_t K,
                                    hipStream_t s);
// One or two tokens (M <= kRowGemvMaxM): y[M,N] = bf16(RMSNorm(X) * gamma) .
// W^T on the VALU, the norm shared by the four wavefronts of a workgroup through
// LDS, each wavefront streaming whole weight rows, 1 KiB per load instruction;
// K a multiple of 8 and at most kRowGemvMaxK; gamma and rstd_out may be null;
// residual and x_add (given together or not at all) add the residual first and
// write x_add out.
constexpr int64_t kRowGemvMaxK = 8192;
constexpr int64_t kRowGemvMaxM = 2;
bool row_gemv_fits(int64_t M, int64_t K);
// weight rows per wavefront for N rows of kc = ceil(K / 512) chunks per lane:
// about kRowGemvWaves wavefronts, at most 4 rows (3 past 6 chunks, 2 past 8, 1
// past 12)
constexpr int64_t kRowGemvWaves = 1024;
int row_gemv_rows(int64_t N, int kc);
hipError_t launch_row_gemv_norm_bf16(const uint16_t* X, const uint16_t* residual, uint16_t* x_add,
                                     const uint16_t* gamma, float eps, const uint16_t* W, void* C, int out_kind,
                                     float* rstd_out, int64_t M, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_small_m_bf16(const uint16_t* A, const uint16_t* W, void* C, int out_kind, int64_t M,
                               int64_t N, int64_t K, int R, hipStream_t s);

// fp32-weight projection of the fp32 normed rows, split over K.
size_t skinny_workspace_bytes(int64_t T, int64_t K, int64_t N);
hipError_t launch_skinny_fp32w(const uint16_t* x, const uint16_t* gamma, float eps, const float* W,
                               void* y, int out_kind, float* rstd_out, int64_t T, int64_t K,
                               int64_t N, void* workspace, hipStream_t s);

// Read-only streaming probe (not a step of the method): `workgroups` workgroups of
// 256 threads read `bytes` (a multiple of 16) from src once, `unroll` (1, 2, 4, 8
// or 16) loads in flight per thread; sink receives one word per workgroup.
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, int unroll,
                              hipStream_t s);
// Clock probe (not a step of the method): `workgroups` wavefronts each wait `delay`
// periods of the 100 MHz real-time counter, then spin for `ticks` periods;
// out[2b] = shader clocks elapsed in that span, out[2b + 1] = real-time ticks.
hipError_t launch_clock_probe(uint64_t* out, uint64_t delay, uint64_t ticks, int workgroups, hipStream_t s);
// MFMA rate probe: `workgroups` x `waves` wavefronts, each `iters` x 8 matrix
// instructions of the given kind (0 bf16, 1 int8, 2 scaled E4M3); one word per
// wavefront to sink.
hipError_t launch_mfma_probe(int kind, int workgroups, int waves, int iters, uint32_t* sink, hipStream_t s);

}  // namespace rnl
