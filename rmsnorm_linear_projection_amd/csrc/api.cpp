// C ABI of the fused RMSNorm -> Linear library: argument validation, workspace
// sizing, kernel-family dispatch and launches.  Declarations and the contract
// of every entry point are in include/rnl.h.
#include "rnl.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "launch.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_last_error[0] = '\0';
  return RNL_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(RNL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxK = int64_t(1) << 20;
constexpr int64_t kMaxK_int8 = 133144;  // K * 127 * 127 <= 2^31 - 1
constexpr int64_t kMaxDim = int64_t(1) << 24;  // N: keeps grid sizes and 32-bit tile offsets in range
// T: below 2^24, because the long-row norm, the split-K reduce and the fp32-weight
// finalize launch one workgroup of 256 threads per row, and a dispatch counts its
// work-items along one grid axis in 32 bits
constexpr int64_t kMaxT = kMaxDim - 1;
constexpr int64_t kMaxHeads = (int64_t(1) << 31) - 1;  // T * heads: the per-head kernel divides in 32 bits
constexpr int64_t kMaxN_fp32w = int64_t(1) << 20;  // fp32 weights: column blocks of 32 fit one grid axis
constexpr int64_t kSmallM = 16;  // at most this many activation rows: weight-streaming kernel

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

enum Variant { V_AUTO, V_GEMM, V_PREPASS };

Variant forced_variant() {
  const char* v = std::getenv("RNL_VARIANT");
  if (v != nullptr && std::strcmp(v, "gemm") == 0) return V_GEMM;
  if (v != nullptr && std::strcmp(v, "prepass") == 0) return V_PREPASS;
  return V_AUTO;
}

// bf16 projections with at most 16 activation rows stream the weight with the
// small-M kernel; larger ones use the tiled GEMM.  RNL_VARIANT=gemm forces the
// tiled GEMM for any M.
bool use_small_m(int64_t M) { return M <= kSmallM && forced_variant() != V_GEMM; }

hipError_t project_bf16(const uint16_t* A, const uint16_t* W, void* C, int kind, int64_t M, int64_t N,
                        int64_t K, hipStream_t s) {
  if (use_small_m(M)) return rnl::launch_small_m_bf16(A, W, C, kind, M, N, K, 0, s);
  return rnl::launch_gemm_bf16(A, W, C, kind, M, N, K, s);
}

// K splits of the chain's first projection (1 = none)
int chain_splits(int64_t T, int64_t R, int64_t K) {
  return use_small_m(T) ? 1 : rnl::gemm_split_plan(T, R, K, 2, nullptr);
}

int check_dims(int64_t T, int64_t K, int64_t N, int64_t maxK) {
  if (T <= 0 || K <= 0 || N <= 0) return fail(RNL_ERR_SHAPE, "sizes must be >= 1 (T=%lld K=%lld N=%lld)", (long long)T, (long long)K, (long long)N);
  if (K % 8 != 0) return fail(RNL_ERR_SHAPE, "K=%lld is not a multiple of 8", (long long)K);
  if (K > maxK) return fail(RNL_ERR_SHAPE, "K=%lld exceeds the limit %lld", (long long)K, (long long)maxK);
  if (T > kMaxT || N > kMaxDim) return fail(RNL_ERR_SHAPE, "T must be < 2^24 and N <= 2^24");
  return RNL_OK;
}

int check_eps(float eps) {
  if (!std::isfinite(eps) || eps < 0.f) return fail(RNL_ERR_ARG, "eps must be finite and >= 0");
  return RNL_OK;
}

#define RNL_TRY(expr)              \
  do {                             \
    int _rc = (expr);              \
    if (_rc != RNL_OK) return _rc; \
  } while (0)

#define RNL_ALIGN(p, a, name)                                                          \
  do {                                                                                 \
    if ((p) != nullptr && !aligned((p), (a)))                                          \
      return fail(RNL_ERR_ALIGN, "%s is not %d-byte aligned", name, (int)(a));          \
  } while (0)

size_t bf16_ws(int64_t T, int64_t K, int64_t N, int w_dtype) {
  if (w_dtype == RNL_FP32) return rnl::skinny_workspace_bytes(T, K, N);
  return align256((size_t)T * (size_t)K * 2);  // the normed bf16 activations
}

// x_add_out must not share a byte with x or the residual: the kernels read
// both after writing parts of x_add.
bool add_overlaps(const void* x, const void* residual, const void* x_add, int64_t T, int64_t K) {
  const uintptr_t n = (uintptr_t)T * (uintptr_t)K * 2u;
  auto hit = [n](const void* a, const void* b) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + n && pb < pa + n;
  };
  return hit(x_add, x) || hit(x_add, residual);
}

// The bf16 / fp32-weight path, with an optional residual added before the norm
// (residual and x_add both non-null) -- shared by rmsnorm_linear_bf16 and
// add_rmsnorm_linear_bf16.  With `heads`, a call that reaches the tiled GEMM runs the
// per-head stage in its epilogue (bf16 weights and output only), and *heads_done is set.
int bf16_path(const void* x, const void* residual, void* x_add, const void* gamma, float eps, const void* W,
              int w_dtype, void* y, int out_dtype, float* rstd_out, int64_t T, int64_t K, int64_t N,
              void* workspace, size_t workspace_bytes, void* stream, const rnl::HeadArgs* heads = nullptr,
              bool* heads_done = nullptr) {
  if (x == nullptr || W == nullptr || y == nullptr) return fail(RNL_ERR_NULL, "x, W and y are required");
  RNL_TRY(check_dims(T, K, N, kMaxK));
  if (w_dtype != RNL_BF16 && w_dtype != RNL_FP32) return fail(RNL_ERR_DTYPE, "w_dtype must be RNL_BF16 or RNL_FP32");
  if (out_dtype != RNL_BF16 && out_dtype != RNL_FP32) return fail(RNL_ERR_DTYPE, "out_dtype must be RNL_BF16 or RNL_FP32");
  if (w_dtype == RNL_FP32 && N > kMaxN_fp32w) return fail(RNL_ERR_SHAPE, "fp32 weights need N <= 2^20");
  RNL_TRY(check_eps(eps));
  RNL_ALIGN(x, 16, "x");
  RNL_ALIGN(residual, 16, "residual");
  RNL_ALIGN(x_add, 16, "x_add_out");
  RNL_ALIGN(gamma, 16, "gamma");
  RNL_ALIGN(W, 16, "W");
  RNL_ALIGN(y, 16, "y");
  RNL_ALIGN(rstd_out, 4, "rstd_out");
  RNL_ALIGN(workspace, 256, "workspace");
  if (residual != nullptr && add_overlaps(x, residual, x_add, T, K))
    return fail(RNL_ERR_ARG, "x_add_out overlaps x or residual");
  const size_t need = bf16_ws(T, K, N, w_dtype);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(RNL_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace == nullptr ? (size_t)0 : workspace_bytes);

  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* rb = static_cast<const uint16_t*>(residual);
  uint16_t* xab = static_cast<uint16_t*>(x_add);
  const uint16_t* gb = static_cast<const uint16_t*>(gamma);
  const int ok_kind = out_dtype == RNL_BF16 ? rnl::OUT_BF16 : rnl::OUT_F32;
  if (w_dtype == RNL_FP32) {
    if (rb != nullptr) {
      // the split-K kernel reads x itself: form x_add first and project that
      const hipError_t e = rnl::launch_add_rows(xb, rb, xab, T, K, s);
      if (e != hipSuccess) return hip_status(e, "residual add launch");
      xb = xab;
    }
    return hip_status(rnl::launch_skinny_fp32w(xb, gb, eps, static_cast<const float*>(W), y, ok_kind,
                                               rstd_out, T, K, N, workspace, s),
                      "skinny split-K launch");
  }
  const uint16_t* wb = static_cast<const uint16_t*>(W);
  // one or two tokens: the workgroup adds the residual (if any) and norms the rows once, and each
  // wavefront streams whole weight rows
  const bool fuse_ok = forced_variant() != V_PREPASS;
  if (fuse_ok && use_small_m(T) && rnl::row_gemv_fits(T, K))
    return hip_status(rnl::launch_row_gemv_norm_bf16(xb, rb, xab, gb, eps, wb, y, ok_kind, rstd_out, T, N, K, s),
                      "whole-row norm + projection launch (one or two tokens)");
  // a few tokens whose normed rows fit LDS, no residual: the norm runs inside the weight-streaming kernel
  if (fuse_ok && rb == nullptr && use_small_m(T) && rnl::small_m_norm_fits(T, K))
    return hip_status(rnl::launch_small_m_norm_bf16(xb, gb, eps, wb, y, ok_kind, rstd_out, T, N, K, s),
                      "fused norm + projection launch");
  uint16_t* a = static_cast<uint16_t*>(workspace);
  const hipError_t e = rb != nullptr ? rnl::launch_add_norm_rows_bf16(xb, rb, xab, gb, eps, T, K, a, rstd_out, s)
                                     : rnl::launch_norm_rows_bf16(xb, gb, eps, T, K, a, rstd_out, s);
  if (e != hipSuccess) return hip_status(e, "norm pre-pass launch");
  if (heads != nullptr && ok_kind == rnl::OUT_BF16 && !use_small_m(T)) {
    *heads_done = true;
    return hip_status(rnl::launch_gemm_bf16_heads(a, wb, static_cast<uint16_t*>(y), T, N, K, *heads, s),
                      "bf16 projection launch with the per-head epilogue");
  }
  return hip_status(project_bf16(a, wb, y, ok_kind, T, N, K, s), "bf16 projection launch");
}

// The int8 path, with an optional residual added before the norm.
int int8_path(const void* x, const void* residual, void* x_add, const void* gamma, float eps, const int8_t* Wq,
              const float* w_scale, void* y, int out_dtype, int8_t* xq_out, float* x_scale_out, float* rstd_out,
              int64_t T, int64_t K, int64_t N, void* workspace, size_t workspace_bytes, void* stream) {
  if (x == nullptr || Wq == nullptr || w_scale == nullptr || y == nullptr)
    return fail(RNL_ERR_NULL, "x, Wq, w_scale and y are required");
  RNL_TRY(check_dims(T, K, N, kMaxK_int8));
  if (K % 16 != 0) return fail(RNL_ERR_SHAPE, "int8 path needs K %% 16 == 0 (K=%lld)", (long long)K);
  if (out_dtype != RNL_BF16 && out_dtype != RNL_FP32 && out_dtype != RNL_INT32)
    return fail(RNL_ERR_DTYPE, "out_dtype must be RNL_BF16, RNL_FP32 or RNL_INT32");
  RNL_TRY(check_eps(eps));
  RNL_ALIGN(x, 16, "x");
  RNL_ALIGN(residual, 16, "residual");
  RNL_ALIGN(x_add, 16, "x_add_out");
  RNL_ALIGN(gamma, 16, "gamma");
  RNL_ALIGN(Wq, 16, "Wq");
  RNL_ALIGN(w_scale, 4, "w_scale");
  RNL_ALIGN(y, 16, "y");
  RNL_ALIGN(xq_out, 16, "xq_out");
  RNL_ALIGN(x_scale_out, 4, "x_scale_out");
  RNL_ALIGN(rstd_out, 4, "rstd_out");
  RNL_ALIGN(workspace, 256, "workspace");
  if (residual != nullptr && add_overlaps(x, residual, x_add, T, K))
    return fail(RNL_ERR_ARG, "x_add_out overlaps x or residual");
  const size_t q_bytes = xq_out ? 0 : align256((size_t)T * (size_t)K);
  const size_t s_bytes = x_scale_out ? 0 : align256((size_t)T * 4);
  const size_t need = q_bytes + s_bytes;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(RNL_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace == nullptr ? (size_t)0 : workspace_bytes);

  hipStream_t s = static_cast<hipStream_t>(stream);
  int8_t* q = xq_out ? xq_out : static_cast<int8_t*>(workspace);
  float* xs = x_scale_out ? x_scale_out
                          : reinterpret_cast<float*>(static_cast<char*>(workspace) + q_bytes);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* gb = static_cast<const uint16_t*>(gamma);
  const hipError_t e =
      residual != nullptr
          ? rnl::launch_add_norm_rows_int8(xb, static_cast<const uint16_t*>(residual), static_cast<uint16_t*>(x_add),
                                           gb, eps, T, K, q, xs, rstd_out, s)
          : rnl::launch_norm_rows_int8(xb, gb, eps, T, K, q, xs, rstd_out, s);
  if (e != hipSuccess) return hip_status(e, "norm+quant pre-pass launch");
  const int kind = out_dtype == RNL_INT32 ? rnl::OUT_I32 : (out_dtype == RNL_FP32 ? rnl::OUT_F32 : rnl::OUT_BF16);
  return hip_status(rnl::launch_gemm_int8(q, Wq, y, kind, xs, w_scale, T, N, K, s), "int8 GEMM launch");
}

constexpr int64_t kMaxHeadDim = 512;  // a head fits one wavefront (64 lanes x 8 values)

int check_head_dim(int64_t D) {
  if (D < 16 || D > kMaxHeadDim || D % 16 != 0)
    return fail(RNL_ERR_SHAPE, "head size D=%lld must be a multiple of 16 in [16, 512]", (long long)D);
  return RNL_OK;
}

// y_out either is y_in (in place) or shares no byte with rows [0, T) of it
bool partial_overlap(const void* a, const void* b, int64_t T, int64_t ld) {
  if (a == b) return false;
  const uintptr_t n = (uintptr_t)T * (uintptr_t)ld * 2u;
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + n && pb < pa + n;
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point (rmsnorm_linear_bf16_noalloc).
// The array lives in the library's code object: every GPU the library runs on
// holds its own copy from the first use until the process ends.  In host code
// `scratch` names a host-side stand-in, not device memory, so it is never
// passed to a kernel: the device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address is used.
// The kernels fully write every scratch byte they later read, so nothing in it
// has to start at zero.
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;
__attribute__((used)) static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of this device's scratch for work on stream s (the stream's
// device; the current device for the null stream).
int scratch_for(hipStream_t s, void** out) {
  int dev = 0;
  hipError_t e = s != nullptr ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "device of the stream");
  if (dev < 0 || dev >= kMaxDevices) return fail(RNL_ERR_ARG, "device %d outside the supported range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e, "hipSetDevice");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (e2 != hipSuccess) return hip_status(e2, "hipSetDevice");
    if (p == nullptr) return fail(RNL_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return RNL_OK;
}

}  // namespace

extern "C" {

size_t rnl_noalloc_scratch_bytes(void) { return kScratchBytes; }

int rmsnorm_linear_bf16_noalloc(const void* x, const void* gamma, float eps, const void* W, int w_dtype, void* y,
                                int out_dtype, float* rstd_out, int64_t T, int64_t K, int64_t N, void* stream) {
  // the size check runs before any HIP call, like every other validation
  if (x == nullptr || W == nullptr || y == nullptr) return fail(RNL_ERR_NULL, "x, W and y are required");
  RNL_TRY(check_dims(T, K, N, kMaxK));
  if (w_dtype != RNL_BF16 && w_dtype != RNL_FP32) return fail(RNL_ERR_DTYPE, "w_dtype must be RNL_BF16 or RNL_FP32");
  if (w_dtype == RNL_FP32 && N > kMaxN_fp32w) return fail(RNL_ERR_SHAPE, "fp32 weights need N <= 2^20");
  const size_t need = bf16_ws(T, K, N, w_dtype);
  if (need > kScratchBytes)
    return fail(RNL_ERR_WORKSPACE, "these sizes need %zu bytes of scratch; the allocation-free entry point has %zu",
                need, kScratchBytes);
  void* ws = nullptr;
  RNL_TRY(scratch_for(static_cast<hipStream_t>(stream), &ws));
  return bf16_path(x, nullptr, nullptr, gamma, eps, W, w_dtype, y, out_dtype, rstd_out, T, K, N, ws, kScratchBytes,
                   stream);
}

const char* rnl_status_str(int status) {
  switch (status) {
    case RNL_OK: return "ok";
    case RNL_ERR_NULL: return "a required pointer is NULL";
    case RNL_ERR_SHAPE: return "invalid or unsupported shape";
    case RNL_ERR_DTYPE: return "unsupported dtype";
    case RNL_ERR_ARG: return "invalid scalar argument";
    case RNL_ERR_ALIGN: return "misaligned pointer";
    case RNL_ERR_WORKSPACE: return "workspace missing or too small";
    case RNL_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* rnl_last_error(void) { return g_last_error; }

int rnl_clock_probe(uint64_t* out, int64_t delay_us, int64_t microseconds, int workgroups, void* stream) {
  if (out == nullptr) return fail(RNL_ERR_NULL, "out is required");
  if (microseconds < 1 || microseconds > 10000000 || delay_us < 0 || delay_us > 10000000)
    return fail(RNL_ERR_SHAPE, "microseconds must be in [1, 10^7] and delay_us in [0, 10^7]");
  if (workgroups < 1 || workgroups > 1024) return fail(RNL_ERR_SHAPE, "workgroups must be in [1, 1024]");
  RNL_ALIGN(out, 8, "out");
  return hip_status(rnl::launch_clock_probe(out, (uint64_t)delay_us * 100u, (uint64_t)microseconds * 100u, workgroups,
                                            static_cast<hipStream_t>(stream)),
                    "clock probe launch");
}

int rnl_mfma_probe(int kind, int workgroups, int waves_per_group, int64_t iterations, uint32_t* sink, void* stream) {
  if (sink == nullptr) return fail(RNL_ERR_NULL, "sink is required");
  if (kind < 0 || kind > 2) return fail(RNL_ERR_ARG, "kind must be 0 (bf16), 1 (int8) or 2 (scaled E4M3)");
  if (workgroups < 1 || workgroups > 65536) return fail(RNL_ERR_SHAPE, "workgroups must be in [1, 65536]");
  if (waves_per_group < 1 || waves_per_group > 16) return fail(RNL_ERR_SHAPE, "waves_per_group must be in [1, 16]");
  if (iterations < 1 || iterations > (int64_t(1) << 24)) return fail(RNL_ERR_SHAPE, "iterations must be in [1, 2^24]");
  RNL_ALIGN(sink, 4, "sink");
  return hip_status(rnl::launch_mfma_probe(kind, workgroups, waves_per_group, (int)iterations, sink,
                                           static_cast<hipStream_t>(stream)),
                    "MFMA probe launch");
}

int rnl_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, int unroll, void* stream) {
  if (src == nullptr || sink == nullptr) return fail(RNL_ERR_NULL, "src and sink are required");
  if (bytes == 0 || bytes % 16 != 0) return fail(RNL_ERR_SHAPE, "bytes must be a positive multiple of 16");
  if (workgroups < 1 || workgroups > 65536) return fail(RNL_ERR_SHAPE, "workgroups must be in [1, 65536]");
  if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8 && unroll != 16)
    return fail(RNL_ERR_ARG, "unroll must be 1, 2, 4, 8 or 16");
  RNL_ALIGN(src, 16, "src");
  RNL_ALIGN(sink, 4, "sink");
  return hip_status(rnl::launch_stream_read(src, bytes, sink, workgroups, unroll, static_cast<hipStream_t>(stream)),
                    "stream probe launch");
}

size_t rmsnorm_linear_bf16_workspace_bytes(int64_t T, int64_t K, int64_t N, int w_dtype,
                                           int out_dtype) {
  (void)out_dtype;
  if (T <= 0 || K <= 0 || N <= 0) return 0;
  return bf16_ws(T, K, N, w_dtype);
}

int rmsnorm_linear_bf16(const void* x, const void* gamma, float eps, const void* W, int w_dtype,
                        void* y, int out_dtype, float* rstd_out, int64_t T, int64_t K, int64_t N,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return bf16_path(x, nullptr, nullptr, gamma, eps, W, w_dtype, y, out_dtype, rstd_out, T, K, N, workspace,
                   workspace_bytes, stream);
}

size_t add_rmsnorm_linear_bf16_workspace_bytes(int64_t T, int64_t K, int64_t N, int w_dtype, int out_dtype) {
  return rmsnorm_linear_bf16_workspace_bytes(T, K, N, w_dtype, out_dtype);
}

int add_rmsnorm_linear_bf16(const void* x, const void* residual, void* x_add_out, const void* gamma, float eps,
                            const void* W, int w_dtype, void* y, int out_dtype, float* rstd_out, int64_t T,
                            int64_t K, int64_t N, void* workspace, size_t workspace_bytes, void* stream) {
  if (residual == nullptr || x_add_out == nullptr) return fail(RNL_ERR_NULL, "residual and x_add_out are required");
  return bf16_path(x, residual, x_add_out, gamma, eps, W, w_dtype, y, out_dtype, rstd_out, T, K, N, workspace,
                   workspace_bytes, stream);
}

size_t rmsnorm_linear_int8_workspace_bytes(int64_t T, int64_t K, int64_t N, int out_dtype) {
  (void)N;
  (void)out_dtype;
  if (T <= 0 || K <= 0) return 0;
  return align256((size_t)T * (size_t)K) + align256((size_t)T * 4);
}

int rmsnorm_linear_int8(const void* x, const void* gamma, float eps, const int8_t* Wq,
                        const float* w_scale, void* y, int out_dtype, int8_t* xq_out,
                        float* x_scale_out, float* rstd_out, int64_t T, int64_t K, int64_t N,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return int8_path(x, nullptr, nullptr, gamma, eps, Wq, w_scale, y, out_dtype, xq_out, x_scale_out, rstd_out, T,
                   K, N, workspace, workspace_bytes, stream);
}

size_t add_rmsnorm_linear_int8_workspace_bytes(int64_t T, int64_t K, int64_t N, int out_dtype) {
  return rmsnorm_linear_int8_workspace_bytes(T, K, N, out_dtype);
}

int add_rmsnorm_linear_int8(const void* x, const void* residual, void* x_add_out, const void* gamma, float eps,
                            const int8_t* Wq, const float* w_scale, void* y, int out_dtype, int8_t* xq_out,
                            float* x_scale_out, float* rstd_out, int64_t T, int64_t K, int64_t N,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (residual == nullptr || x_add_out == nullptr) return fail(RNL_ERR_NULL, "residual and x_add_out are required");
  return int8_path(x, residual, x_add_out, gamma, eps, Wq, w_scale, y, out_dtype, xq_out, x_scale_out, rstd_out, T,
                   K, N, workspace, workspace_bytes, stream);
}

size_t norm_proj_chain_workspace_bytes(int64_t T, int64_t K, int64_t R, int64_t N) {
  (void)N;
  if (T <= 0 || R <= 0 || K <= 0) return 0;
  const int ks = chain_splits(T, R, K);
  if (ks > 1) return align256((size_t)ks * (size_t)T * (size_t)R * 4);  // fp32 split-K partials of q_a
  return align256((size_t)T * (size_t)R * 2);                           // bf16 q_a
}

int norm_proj_chain(const void* x, const void* W_a, const void* gamma, float eps, const void* W_b,
                    void* qr_out, void* y, float* rstd_out, void* qa_out, int64_t T, int64_t K, int64_t R,
                    int64_t N, void* workspace, size_t workspace_bytes, void* stream) {
  if (x == nullptr || W_a == nullptr || W_b == nullptr || qr_out == nullptr || y == nullptr)
    return fail(RNL_ERR_NULL, "x, W_a, W_b, qr_out and y are required");
  RNL_TRY(check_dims(T, K, N, kMaxK));
  RNL_TRY(check_dims(T, R, N, kMaxK));
  RNL_TRY(check_eps(eps));
  RNL_ALIGN(x, 16, "x");
  RNL_ALIGN(W_a, 16, "W_a");
  RNL_ALIGN(gamma, 16, "gamma");
  RNL_ALIGN(W_b, 16, "W_b");
  RNL_ALIGN(qr_out, 16, "qr_out");
  RNL_ALIGN(y, 16, "y");
  RNL_ALIGN(rstd_out, 4, "rstd_out");
  RNL_ALIGN(qa_out, 16, "qa_out");
  RNL_ALIGN(workspace, 256, "workspace");
  const size_t need = norm_proj_chain_workspace_bytes(T, K, R, N);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(RNL_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace == nullptr ? (size_t)0 : workspace_bytes);

  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* wa = static_cast<const uint16_t*>(W_a);
  const uint16_t* gb = static_cast<const uint16_t*>(gamma);
  uint16_t* qr = static_cast<uint16_t*>(qr_out);
  uint16_t* qa_keep = static_cast<uint16_t*>(qa_out);
  const int ks = chain_splits(T, R, K);
  hipError_t e;
  if (ks > 1) {
    // q_a is too small to fill the chip: split its K, then add the partials in split
    // order inside the norm pre-pass (q_a = bf16 of the sum)
    float* part = static_cast<float*>(workspace);
    e = rnl::launch_gemm_bf16_splitk(xb, wa, part, T, R, K, ks, s);
    if (e != hipSuccess) return hip_status(e, "chain stage-1 split-K GEMM launch");
    e = rnl::launch_reduce_norm_bf16(part, ks, R, gb, eps, T, R, qr, rstd_out, qa_keep, R, s);
    if (e != hipSuccess) return hip_status(e, "chain reduce+norm launch");
  } else {
    // the stage-1 rows go to qa_out when the caller asks for them
    uint16_t* qa = qa_keep != nullptr ? qa_keep : static_cast<uint16_t*>(workspace);
    e = project_bf16(xb, wa, qa, rnl::OUT_BF16, T, R, K, s);
    if (e != hipSuccess) return hip_status(e, "chain stage-1 projection launch");
    e = rnl::launch_norm_rows_bf16(qa, gb, eps, T, R, qr, rstd_out, s);
    if (e != hipSuccess) return hip_status(e, "chain norm launch");
  }
  return hip_status(project_bf16(static_cast<const uint16_t*>(qr_out), static_cast<const uint16_t*>(W_b), y,
                                 rnl::OUT_BF16, T, N, R, s),
                    "chain stage-2 projection launch");
}

size_t rmsnorm_linear_mxfp8_workspace_bytes(int64_t T, int64_t K, int64_t N, int out_dtype) {
  (void)N;
  (void)out_dtype;
  if (T <= 0 || K <= 0) return 0;
  return align256((size_t)T * (size_t)K) + align256((size_t)T * (size_t)(K / 64));
}

int rmsnorm_linear_mxfp8(const void* x, const void* gamma, float eps, const uint8_t* Wq, const uint8_t* w_scale,
                         void* y, int out_dtype, uint8_t* xq_out, uint8_t* x_scale_out, float* rstd_out, int64_t T,
                         int64_t K, int64_t N, void* workspace, size_t workspace_bytes, void* stream) {
  if (x == nullptr || Wq == nullptr || w_scale == nullptr || y == nullptr)
    return fail(RNL_ERR_NULL, "x, Wq, w_scale and y are required");
  RNL_TRY(check_dims(T, K, N, kMaxK));
  if (K % 64 != 0) return fail(RNL_ERR_SHAPE, "MXFP8 needs K %% 64 == 0 (K=%lld)", (long long)K);
  if (out_dtype != RNL_BF16 && out_dtype != RNL_FP32) return fail(RNL_ERR_DTYPE, "out_dtype must be RNL_BF16 or RNL_FP32");
  RNL_TRY(check_eps(eps));
  RNL_ALIGN(x, 16, "x");
  RNL_ALIGN(gamma, 16, "gamma");
  RNL_ALIGN(Wq, 16, "Wq");
  RNL_ALIGN(y, 16, "y");
  RNL_ALIGN(xq_out, 16, "xq_out");
  RNL_ALIGN(rstd_out, 4, "rstd_out");
  RNL_ALIGN(workspace, 256, "workspace");
  const size_t q_bytes = xq_out ? 0 : align256((size_t)T * (size_t)K);
  const size_t s_bytes = x_scale_out ? 0 : align256((size_t)T * (size_t)(K / 64));
  const size_t need = q_bytes + s_bytes;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(RNL_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace == nullptr ? (size_t)0 : workspace_bytes);

  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* q = xq_out ? xq_out : static_cast<uint8_t*>(workspace);
  uint8_t* xs = x_scale_out ? x_scale_out : static_cast<uint8_t*>(workspace) + q_bytes;
  const hipError_t e = rnl::launch_norm_rows_mx(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(gamma),
                                                eps, T, K, q, xs, rstd_out, s);
  if (e != hipSuccess) return hip_status(e, "norm+MX quant launch");
  return hip_status(rnl::launch_gemm_mx(q, xs, Wq, w_scale, y, out_dtype == RNL_FP32 ? rnl::OUT_F32 : rnl::OUT_BF16,
                                        T, N, K, s),
                    "MXFP8 GEMM launch");
}

size_t mla_prolog_bf16_workspace_bytes(int64_t T, int64_t K, int64_t R, int64_t Rkv, int64_t N) {
  (void)N;
  if (T <= 0 || R <= 0 || Rkv <= 0 || K <= 0) return 0;
  const int64_t Rt = R + Rkv;
  const int ks = chain_splits(T, Rt, K);
  if (ks > 1) return align256((size_t)ks * (size_t)T * (size_t)Rt * 4);  // fp32 split-K partials of [q_a | kv]
  return align256((size_t)T * (size_t)Rt * 2);                           // bf16 [q_a | kv]
}

int mla_prolog_bf16(const void* x, const void* W_akv, const void* gamma_cq, const void* gamma_ckv, float eps,
                    const void* W_b, void* qr_out, void* kv_out, void* y, float* rstd_q_out, float* rstd_kv_out,
                    void* qakv_out, int64_t T, int64_t K, int64_t R, int64_t Rkv, int64_t N, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (x == nullptr || W_akv == nullptr || W_b == nullptr || qr_out == nullptr || kv_out == nullptr || y == nullptr)
    return fail(RNL_ERR_NULL, "x, W_akv, W_b, qr_out, kv_out and y are required");
  RNL_TRY(check_dims(T, K, N, kMaxK));
  RNL_TRY(check_dims(T, R, N, kMaxK));
  RNL_TRY(check_dims(T, Rkv, N, kMaxK));
  RNL_TRY(check_dims(T, K, R + Rkv, kMaxK));
  RNL_TRY(check_eps(eps));
  RNL_ALIGN(x, 16, "x");
  RNL_ALIGN(W_akv, 16, "W_akv");
  RNL_ALIGN(gamma_cq, 16, "gamma_cq");
  RNL_ALIGN(gamma_ckv, 16, "gamma_ckv");
  RNL_ALIGN(W_b, 16, "W_b");
  RNL_ALIGN(qr_out, 16, "qr_out");
  RNL_ALIGN(kv_out, 16, "kv_out");
  RNL_ALIGN(y, 16, "y");
  RNL_ALIGN(rstd_q_out, 4, "rstd_q_out");
  RNL_ALIGN(rstd_kv_out, 4, "rstd_kv_out");
  RNL_ALIGN(qakv_out, 16, "qakv_out");
  RNL_ALIGN(workspace, 256, "workspace");
  const size_t need = mla_prolog_bf16_workspace_bytes(T, K, R, Rkv, N);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(RNL_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace == nullptr ? (size_t)0 : workspace_bytes);

  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* w = static_cast<const uint16_t*>(W_akv);
  const uint16_t* gq = static_cast<const uint16_t*>(gamma_cq);
  const uint16_t* gkv = static_cast<const uint16_t*>(gamma_ckv);
  uint16_t* qr = static_cast<uint16_t*>(qr_out);
  uint16_t* kvo = static_cast<uint16_t*>(kv_out);
  const int64_t Rt = R + Rkv;
  uint16_t* keep = static_cast<uint16_t*>(qakv_out);
  const int ks = chain_splits(T, Rt, K);
  hipError_t e;
  // one pass over x for both branches: [q_a | kv] = x . [W_a; W_kv]^T, then each
  // part of the row is normed with its own gamma
  // the query and the kv columns are normed on their own, in one launch
  const rnl::NormCols cq{0, R, gq, qr, rstd_q_out}, ckv{R, Rkv, gkv, kvo, rstd_kv_out};
  if (ks > 1) {
    float* part = static_cast<float*>(workspace);
    e = rnl::launch_gemm_bf16_splitk(xb, w, part, T, Rt, K, ks, s);
    if (e != hipSuccess) return hip_status(e, "stage-1 split-K GEMM launch");
    e = rnl::launch_reduce_norm_pair_bf16(part, ks, Rt, T, cq, ckv, eps, keep, s);
    if (e != hipSuccess) return hip_status(e, "query and kv reduce+norm launch");
  } else {
    // the stage-1 rows go to qakv_out when the caller asks for them
    uint16_t* qakv = keep != nullptr ? keep : static_cast<uint16_t*>(workspace);
    e = project_bf16(xb, w, qakv, rnl::OUT_BF16, T, Rt, K, s);
    if (e != hipSuccess) return hip_status(e, "stage-1 projection launch");
    e = rnl::launch_norm_rows_pair_bf16_strided(qakv, Rt, T, cq, ckv, eps, s);
    if (e != hipSuccess) return hip_status(e, "query and kv norm launch");
  }
  return hip_status(project_bf16(qr, static_cast<const uint16_t*>(W_b), y, rnl::OUT_BF16, T, N, R, s),
                    "stage-2 projection launch");
}

size_t preattn_qkv_bf16_workspace_bytes(int64_t T, int64_t K, int64_t Hq, int64_t Hkv, int64_t D) {
  if (T <= 0 || K <= 0 || Hq <= 0 || Hkv < 0 || D <= 0) return 0;
  return bf16_ws(T, K, (Hq + 2 * Hkv) * D, RNL_BF16);
}

int preattn_qkv_bf16(const void* x, const void* residual, void* x_add_out, const void* gamma, float eps,
                     const void* W, void* y, float* rstd_out, const void* gamma_q, const void* gamma_k,
                     float head_eps, const float* cos_t, const float* sin_t, float* head_rstd_out, int64_t T,
                     int64_t K, int64_t Hq, int64_t Hkv, int64_t D, void* workspace, size_t workspace_bytes,
                     void* stream) {
  if ((residual == nullptr) != (x_add_out == nullptr))
    return fail(RNL_ERR_NULL, "residual and x_add_out are given together or not at all");
  if ((cos_t == nullptr) != (sin_t == nullptr)) return fail(RNL_ERR_NULL, "cos and sin are given together or not at all");
  if (T <= 0 || K <= 0 || Hq <= 0 || Hkv < 0)
    return fail(RNL_ERR_SHAPE, "need T, K, Hq >= 1 and Hkv >= 0 (T=%lld K=%lld Hq=%lld Hkv=%lld)", (long long)T,
                (long long)K, (long long)Hq, (long long)Hkv);
  RNL_TRY(check_head_dim(D));
  if (Hq + 2 * Hkv > kMaxDim / D) return fail(RNL_ERR_SHAPE, "(Hq + 2 Hkv) * D must be <= 2^24");
  if (T > kMaxHeads / (Hq + Hkv)) return fail(RNL_ERR_SHAPE, "T * (Hq + Hkv) must be < 2^31");
  RNL_TRY(check_eps(head_eps));
  RNL_ALIGN(gamma_q, 16, "gamma_q");
  RNL_ALIGN(gamma_k, 16, "gamma_k");
  RNL_ALIGN(cos_t, 16, "cos");
  RNL_ALIGN(sin_t, 16, "sin");
  RNL_ALIGN(head_rstd_out, 4, "head_rstd_out");
  const int64_t N = (Hq + 2 * Hkv) * D;
  // Heads of 128 on the tiled GEMM: the per-head stage runs in the GEMM's epilogue
  // (RNL_VARIANT=prepass keeps it a separate pass, as for other head sizes and few tokens).
  const rnl::HeadArgs ha{static_cast<const uint16_t*>(gamma_q), static_cast<const uint16_t*>(gamma_k), cos_t, sin_t,
                         head_rstd_out, head_eps, 1.0f / (float)D, (int)Hq, (int)Hkv};
  const bool epi = D == rnl::kHeadEpiD && forced_variant() != V_PREPASS;
  bool heads_done = false;
  RNL_TRY(bf16_path(x, residual, x_add_out, gamma, eps, W, RNL_BF16, y, RNL_BF16, rstd_out, T, K, N, workspace,
                    workspace_bytes, stream, epi ? &ha : nullptr, &heads_done));
  if (heads_done) return ok();
  uint16_t* yb = static_cast<uint16_t*>(y);
  return hip_status(rnl::launch_head_norm_bf16(yb, yb, T, N, 0, Hq + Hkv, D, Hq,
                                               static_cast<const uint16_t*>(gamma_q),
                                               static_cast<const uint16_t*>(gamma_k), head_eps, cos_t, sin_t,
                                               head_rstd_out, static_cast<hipStream_t>(stream)),
                    "per-head norm launch");
}

int head_rms_norm_bf16(const void* y_in, void* y_out, const void* gamma, float eps, const float* cos_t,
                       const float* sin_t, float* rstd_out, int64_t T, int64_t ld, int64_t col0, int64_t H,
                       int64_t D, void* stream) {
  if (y_in == nullptr || y_out == nullptr) return fail(RNL_ERR_NULL, "y_in and y_out are required");
  if ((cos_t == nullptr) != (sin_t == nullptr)) return fail(RNL_ERR_NULL, "cos and sin are given together or not at all");
  if (T <= 0 || H <= 0 || col0 < 0 || ld <= 0)
    return fail(RNL_ERR_SHAPE, "need T, H, ld >= 1 and col0 >= 0");
  RNL_TRY(check_head_dim(D));
  if (T > kMaxT || ld > kMaxDim) return fail(RNL_ERR_SHAPE, "T must be < 2^24 and ld <= 2^24");
  if (ld % 8 != 0 || col0 % 8 != 0) return fail(RNL_ERR_SHAPE, "ld and col0 must be multiples of 8");
  if (H > (ld - col0) / D) return fail(RNL_ERR_SHAPE, "col0 + H * D exceeds the row length ld");
  if (T > kMaxHeads / H) return fail(RNL_ERR_SHAPE, "T * H must be < 2^31");
  RNL_TRY(check_eps(eps));
  RNL_ALIGN(y_in, 16, "y_in");
  RNL_ALIGN(y_out, 16, "y_out");
  RNL_ALIGN(gamma, 16, "gamma");
  RNL_ALIGN(cos_t, 16, "cos");
  RNL_ALIGN(sin_t, 16, "sin");
  RNL_ALIGN(rstd_out, 4, "rstd_out");
  if (partial_overlap(y_in, y_out, T, ld)) return fail(RNL_ERR_ARG, "y_out overlaps y_in without being y_in");
  const uint16_t* gb = static_cast<const uint16_t*>(gamma);
  return hip_status(rnl::launch_head_norm_bf16(static_cast<const uint16_t*>(y_in), static_cast<uint16_t*>(y_out),
                                               T, ld, col0, H, D, H, gb, gb, eps, cos_t, sin_t, rstd_out,
                                               static_cast<hipStream_t>(stream)),
                    "per-head norm launch");
}

int rms_norm_bf16(const void* x, const void* gamma, float eps, void* y, float* rstd_out, int64_t T,
                  int64_t K, void* stream) {
  if (x == nullptr || y == nullptr) return fail(RNL_ERR_NULL, "x and y are required");
  RNL_TRY(check_dims(T, K, 1, kMaxK));
  RNL_TRY(check_eps(eps));
  RNL_ALIGN(x, 16, "x");
  RNL_ALIGN(gamma, 16, "gamma");
  RNL_ALIGN(y, 16, "y");
  RNL_ALIGN(rstd_out, 4, "rstd_out");
  return hip_status(rnl::launch_norm_rows_bf16(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(gamma),
                                               eps, T, K, static_cast<uint16_t*>(y), rstd_out,
                                               static_cast<hipStream_t>(stream)),
                    "norm launch");
}

int rms_norm_quant_int8(const void* x, const void* gamma, float eps, int8_t* xq, float* x_scale,
                        float* rstd_out, int64_t T, int64_t K, void* stream) {
  if (x == nullptr || xq == nullptr || x_scale == nullptr) return fail(RNL_ERR_NULL, "x, xq and x_scale are required");
  RNL_TRY(check_dims(T, K, 1, kMaxK_int8));
  if (K % 16 != 0) return fail(RNL_ERR_SHAPE, "int8 path needs K %% 16 == 0 (K=%lld)", (long long)K);
  RNL_TRY(check_eps(eps));
  RNL_ALIGN(x, 16, "x");
  RNL_ALIGN(gamma, 16, "gamma");
  RNL_ALIGN(xq, 16, "xq");
  RNL_ALIGN(x_scale, 4, "x_scale");
  RNL_ALIGN(rstd_out, 4, "rstd_out");
  return hip_status(rnl::launch_norm_rows_int8(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(gamma),
                                               eps, T, K, xq, x_scale, rstd_out,
                                               static_cast<hipStream_t>(stream)),
                    "norm+quant launch");
}

int linear_heads_bf16(const void* a, const void* W, void* y, const void* gamma_q, const void* gamma_k,
                      float head_eps, const float* cos_t, const float* sin_t, float* head_rstd_out, int64_t M,
                      int64_t K, int64_t Hq, int64_t Hkv, int64_t D, void* stream) {
  if (a == nullptr || W == nullptr || y == nullptr) return fail(RNL_ERR_NULL, "a, W and y are required");
  if ((cos_t == nullptr) != (sin_t == nullptr)) return fail(RNL_ERR_NULL, "cos and sin are given together or not at all");
  if (M <= 0 || K <= 0 || Hq <= 0 || Hkv < 0)
    return fail(RNL_ERR_SHAPE, "need M, K, Hq >= 1 and Hkv >= 0 (M=%lld K=%lld Hq=%lld Hkv=%lld)", (long long)M,
                (long long)K, (long long)Hq, (long long)Hkv);
  RNL_TRY(check_head_dim(D));
  if (Hq + 2 * Hkv > kMaxDim / D) return fail(RNL_ERR_SHAPE, "(Hq + 2 Hkv) * D must be <= 2^24");
  const int64_t N = (Hq + 2 * Hkv) * D;
  RNL_TRY(check_dims(M, K, N, kMaxK));
  if (M > kMaxHeads / (Hq + Hkv)) return fail(RNL_ERR_SHAPE, "M * (Hq + Hkv) must be < 2^31");
  RNL_TRY(check_eps(head_eps));
  RNL_ALIGN(a, 16, "a");
  RNL_ALIGN(W, 16, "W");
  RNL_ALIGN(y, 16, "y");
  RNL_ALIGN(gamma_q, 16, "gamma_q");
  RNL_ALIGN(gamma_k, 16, "gamma_k");
  RNL_ALIGN(cos_t, 16, "cos");
  RNL_ALIGN(sin_t, 16, "sin");
  RNL_ALIGN(head_rstd_out, 4, "head_rstd_out");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint16_t* ab = static_cast<const uint16_t*>(a);
  const uint16_t* wb = static_cast<const uint16_t*>(W);
  uint16_t* yb = static_cast<uint16_t*>(y);
  const uint16_t* gq = static_cast<const uint16_t*>(gamma_q);
  const uint16_t* gk = static_cast<const uint16_t*>(gamma_k);
  if (D == rnl::kHeadEpiD && !use_small_m(M) && forced_variant() != V_PREPASS) {
    const rnl::HeadArgs ha{gq, gk, cos_t, sin_t, head_rstd_out, head_eps, 1.0f / (float)D, (int)Hq, (int)Hkv};
    return hip_status(rnl::launch_gemm_bf16_heads(ab, wb, yb, M, N, K, ha, s),
                      "bf16 projection launch with the per-head epilogue");
  }
  const hipError_t e = project_bf16(ab, wb, yb, rnl::OUT_BF16, M, N, K, s);
  if (e != hipSuccess) return hip_status(e, "bf16 projection launch");
  return hip_status(rnl::launch_head_norm_bf16(yb, yb, M, N, 0, Hq + Hkv, D, Hq, gq, gk, head_eps, cos_t, sin_t,
                                               head_rstd_out, s),
                    "per-head norm launch");
}

int linear_bf16(const void* a, const void* W, void* y, int out_dtype, int64_t M, int64_t K, int64_t N,
                void* stream) {
  if (a == nullptr || W == nullptr || y == nullptr) return fail(RNL_ERR_NULL, "a, W and y are required");
  RNL_TRY(check_dims(M, K, N, kMaxK));
  if (out_dtype != RNL_BF16 && out_dtype != RNL_FP32) return fail(RNL_ERR_DTYPE, "out_dtype must be RNL_BF16 or RNL_FP32");
  RNL_ALIGN(a, 16, "a");
  RNL_ALIGN(W, 16, "W");
  RNL_ALIGN(y, 16, "y");
  return hip_status(project_bf16(static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(W), y,
                                 out_dtype == RNL_BF16 ? rnl::OUT_BF16 : rnl::OUT_F32, M, N, K,
                                 static_cast<hipStream_t>(stream)),
                    "bf16 projection launch");
}

int rms_norm_quant_mxfp8(const void* x, const void* gamma, float eps, uint8_t* xq, uint8_t* x_scale,
                         float* rstd_out, int64_t T, int64_t K, void* stream) {
  if (x == nullptr || xq == nullptr || x_scale == nullptr) return fail(RNL_ERR_NULL, "x, xq and x_scale are required");
  RNL_TRY(check_dims(T, K, 1, kMaxK));
  if (K % 64 != 0) return fail(RNL_ERR_SHAPE, "MXFP8 needs K %% 64 == 0 (K=%lld)", (long long)K);
  RNL_TRY(check_eps(eps));
  RNL_ALIGN(x, 16, "x");
  RNL_ALIGN(gamma, 16, "gamma");
  RNL_ALIGN(xq, 16, "xq");
  RNL_ALIGN(rstd_out, 4, "rstd_out");
  return hip_status(rnl::launch_norm_rows_mx(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(gamma), eps,
                                             T, K, xq, x_scale, rstd_out, static_cast<hipStream_t>(stream)),
                    "norm+MX quant launch");
}

int linear_mxfp8(const uint8_t* xq, const uint8_t* x_scale, const uint8_t* Wq, const uint8_t* w_scale, void* y,
                 int out_dtype, int64_t M, int64_t K, int64_t N, void* stream) {
  if (xq == nullptr || x_scale == nullptr || Wq == nullptr || w_scale == nullptr || y == nullptr)
    return fail(RNL_ERR_NULL, "xq, x_scale, Wq, w_scale and y are required");
  RNL_TRY(check_dims(M, K, N, kMaxK));
  if (K % 64 != 0) return fail(RNL_ERR_SHAPE, "MXFP8 needs K %% 64 == 0 (K=%lld)", (long long)K);
  if (out_dtype != RNL_BF16 && out_dtype != RNL_FP32) return fail(RNL_ERR_DTYPE, "out_dtype must be RNL_BF16 or RNL_FP32");
  RNL_ALIGN(xq, 16, "xq");
  RNL_ALIGN(Wq, 16, "Wq");
  RNL_ALIGN(y, 16, "y");
  return hip_status(rnl::launch_gemm_mx(xq, x_scale, Wq, w_scale, y, out_dtype == RNL_FP32 ? rnl::OUT_F32 : rnl::OUT_BF16,
                                        M, N, K, static_cast<hipStream_t>(stream)),
                    "MXFP8 GEMM launch");
}

int linear_int8(const int8_t* xq, const float* x_scale, const int8_t* Wq, const float* w_scale, void* y,
                int out_dtype, int64_t M, int64_t K, int64_t N, void* stream) {
  if (xq == nullptr || Wq == nullptr || y == nullptr) return fail(RNL_ERR_NULL, "xq, Wq and y are required");
  if (out_dtype != RNL_INT32 && (x_scale == nullptr || w_scale == nullptr))
    return fail(RNL_ERR_NULL, "x_scale and w_scale are required to dequantise");
  RNL_TRY(check_dims(M, K, N, kMaxK_int8));
  if (K % 16 != 0) return fail(RNL_ERR_SHAPE, "int8 path needs K %% 16 == 0 (K=%lld)", (long long)K);
  if (out_dtype != RNL_BF16 && out_dtype != RNL_FP32 && out_dtype != RNL_INT32)
    return fail(RNL_ERR_DTYPE, "out_dtype must be RNL_BF16, RNL_FP32 or RNL_INT32");
  RNL_ALIGN(xq, 16, "xq");
  RNL_ALIGN(Wq, 16, "Wq");
  RNL_ALIGN(x_scale, 4, "x_scale");
  RNL_ALIGN(w_scale, 4, "w_scale");
  RNL_ALIGN(y, 16, "y");
  const int kind = out_dtype == RNL_INT32 ? rnl::OUT_I32 : (out_dtype == RNL_FP32 ? rnl::OUT_F32 : rnl::OUT_BF16);
  return hip_status(rnl::launch_gemm_int8(xq, Wq, y, kind, x_scale, w_scale, M, N, K, static_cast<hipStream_t>(stream)),
                    "int8 GEMM launch");
}

}  // extern "C"
