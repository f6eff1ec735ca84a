/*
 * rnl.h -- C ABI of the MI355X (gfx950) fused RMSNorm -> Linear projection library.
 *
 * The operation (AT-10 page "PyPTO-Gym operator design pattern AT-10: RMSNorm +
 * Linear fused (V->C layout)", section 2 "CV layout and standard compute flow"):
 * per token t,
 *     xf     = float(x[t, :])
 *     ms     = fl( fl(sum_k xf^2) * fl(1/K) )         (fp32 reduction)
 *     rstd   = 1 / sqrt(ms + eps)                      (section 3, variant B)
 *     n[k]   = fl( fl(xf[k] * rstd) * float(gamma[k]) ) (gamma optional)
 *     y[t,:] = bf16(n) . W^T                          (W stored [N, K])
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is DEVICE memory, row-major and contiguous, owned by
 *     the caller; outputs are preallocated by the caller (SK-14 page, the host
 *     wrapper preallocates outputs).  Outputs must not alias inputs.
 *   - Calls are asynchronous: they enqueue kernels on `stream` (a hipStream_t;
 *     NULL means the default stream) and return.  Nothing is allocated and no
 *     host synchronisation happens inside a call.
 *   - Return value: RNL_OK (0) when the work was enqueued, else a negative
 *     RNL_ERR_* code.  Arguments are validated before any HIP call, so an
 *     invalid call touches no memory.  rnl_last_error() gives a detail string
 *     for the calling thread.  No exception or abort crosses the ABI.
 *   - Sizes are int64_t and must be >= 1.  K must be a multiple of 8 (16-byte
 *     vectors of bf16) and at most 2^20; T below 2^24 (some stages launch a
 *     workgroup of 256 threads per row, and a grid axis counts its work-items
 *     in 32 bits) and N at most 2^24.  Any T and N in range are accepted:
 *     partial tiles are masked (the pages' valid_shape tails).  Buffers may be
 *     larger than 4 GiB: rows and tiles are addressed from 64-bit bases.
 *   - Alignment: x, gamma, W, Wq, W_a, W_b, y, qr_out, xq_out must be 16-byte
 *     aligned; rstd_out, x_scale_out, w_scale 4-byte; workspace 256-byte.
 *   - eps must be finite and >= 0; it is used as the fp32 value fl(eps).
 *   - `workspace` is scratch device memory of at least the size the matching
 *     *_workspace_bytes() query returns for the same arguments (0 means none
 *     is needed and the pointer may be NULL).  Its contents on entry do not
 *     matter and are undefined afterwards.
 *   - bf16 projections with at most 16 activation rows run a weight-streaming
 *     kernel (one or two rows with K <= 8192: a kernel that adds the residual
 *     if any, norms the rows, streams whole weight rows and multiplies on the
 *     vector units), larger ones the
 *     tiled GEMM.  Environment variable RNL_VARIANT
 *     (read at every call) set to "gemm" forces the tiled GEMM for any size,
 *     "prepass" forces the separate norm pre-pass (no norm fused into the
 *     weight-streaming kernels) and the separate per-head pass of
 *     preattn_qkv_bf16, for testing; anything else, or unset, lets the shape
 *     decide.
 */
#ifndef RNL_H
#define RNL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every entry point below is exported from librnl.so; nothing else is. */
#define RNL_API __attribute__((visibility("default")))

/* dtype codes */
#define RNL_BF16 1
#define RNL_FP32 2
#define RNL_INT8 3
#define RNL_INT32 4

/* status codes */
#define RNL_OK 0
#define RNL_ERR_NULL (-1)      /* a required pointer is NULL                    */
#define RNL_ERR_SHAPE (-2)     /* size <= 0, K % 8 != 0, or a size limit exceeded */
#define RNL_ERR_DTYPE (-3)     /* unsupported dtype code or combination          */
#define RNL_ERR_ARG (-4)       /* eps negative or not finite                     */
#define RNL_ERR_ALIGN (-5)     /* a pointer is not aligned as required           */
#define RNL_ERR_WORKSPACE (-6) /* workspace NULL or smaller than required        */
#define RNL_ERR_HIP (-7)       /* a HIP runtime call or kernel launch failed     */

/*
 * rmsnorm_linear_bf16 -- fused RMSNorm -> Linear (AT-10).
 *
 * AT-10 page, section 2 (compute flow), section 3 (AT-03 RMSNorm: fp32 inside,
 * optional gamma, optional rstd output), section 4 (AT-09 BF16 mode: bf16
 * operands, the weight transposed).  With w_dtype == RNL_FP32 this is the
 * SK-03 page's mhc_pre variant (a very long reduction into a handful of
 * output columns, computed in fp32): the normed rows stay fp32 and are
 * multiplied by an fp32 weight.
 *
 *   x         [T, K] bf16 activations.
 *   gamma     [K] bf16 scale, or NULL for no gamma (has_gamma = false).
 *   eps       added to the mean square before the root.
 *   W         [N, K] weight, row n holds output column n (b_trans = True);
 *             bf16 when w_dtype == RNL_BF16, fp32 when w_dtype == RNL_FP32.
 *   y         [T, N] output, bf16 (out_dtype RNL_BF16) or fp32 (RNL_FP32).
 *             bf16 weights: y = round_bf16(fp32 accumulation of
 *             bf16(n) * W).  fp32 weights: y = fp32 accumulation of n * W.
 *   rstd_out  [T] fp32 per-token rstd (AT-03 output_rstd), or NULL.
 *   With fp32 weights the normed rows are not rounded to bf16, and the
 *   reduction over K is split across workgroups and added in a fixed order,
 *   so repeated calls give identical results.
 *
 * Errors: RNL_ERR_NULL (x, W or y NULL), RNL_ERR_SHAPE (also N > 2^20 with
 * fp32 weights), RNL_ERR_DTYPE (w_dtype not BF16/FP32, out_dtype not
 * BF16/FP32), RNL_ERR_ARG,
 * RNL_ERR_ALIGN, RNL_ERR_WORKSPACE, RNL_ERR_HIP.
 */
RNL_API int rmsnorm_linear_bf16(const void* x, const void* gamma, float eps, const void* W, int w_dtype,
                        void* y, int out_dtype, float* rstd_out, int64_t T, int64_t K, int64_t N,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes rmsnorm_linear_bf16 needs for these arguments (0 = none). */
RNL_API size_t rmsnorm_linear_bf16_workspace_bytes(int64_t T, int64_t K, int64_t N, int w_dtype,
                                           int out_dtype);

/*
 * rmsnorm_linear_bf16_noalloc -- rmsnorm_linear_bf16 for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).
 *
 * Same arguments, results and errors as rmsnorm_linear_bf16, without the
 * workspace: the kernels use a fixed scratch array that the library holds on
 * each GPU it runs on (allocated with the library's code, on that GPU, and
 * kept until the process ends).  The call itself allocates nothing.
 *   - Sizes whose rmsnorm_linear_bf16_workspace_bytes() exceeds
 *     rnl_noalloc_scratch_bytes() (32 MiB; e.g. T * K <= 16 Mi with bf16
 *     weights) are rejected with RNL_ERR_WORKSPACE before any HIP call.
 *   - Every call on one GPU uses that GPU's one scratch array: calls that may
 *     overlap on a GPU (different streams without ordering, or several host
 *     threads) race and must be serialised by the caller.  Calls in one
 *     stream are ordered and safe.
 *   - The scratch's device is the device of `stream` (the current device for
 *     the NULL stream); its address is looked up once per device, with the
 *     runtime's symbol lookup, on the first call there.
 */
RNL_API int rmsnorm_linear_bf16_noalloc(const void* x, const void* gamma, float eps, const void* W, int w_dtype,
                                        void* y, int out_dtype, float* rstd_out, int64_t T, int64_t K, int64_t N,
                                        void* stream);

/* Bytes of the scratch array behind rmsnorm_linear_bf16_noalloc (per GPU). */
RNL_API size_t rnl_noalloc_scratch_bytes(void);

/*
 * rmsnorm_linear_int8 -- fused RMSNorm -> per-token int8 quant -> int8 GEMM ->
 * dequant (AT-11 = AT-10 with AT-09's INT8 W8A8 mode).
 *
 * AT-10 page, section 4: the fp32 normed rows are quantised per token
 * (AT-05), multiplied by the int8 weight with int32 accumulation, and the
 * accumulators are dequantised with both scales (AT-06).
 * AT-05 (AT-10 page section 4; SK-03 page quant variant, common.py quant):
 * amax[t] = max_k |n[t,k]|, s = fl(127 / amax), q = saturate_+-127(rint(fl(n*s)))
 * with round-half-to-even, x_scale = fl(amax / 127); an all-zero row gives
 * q = 0 and x_scale = 0.  AT-06 in the order of the SK-14 page's
 * QuantMatMulReduceSum: y = fl(float(acc) * fl(x_scale[t] * w_scale[n])).
 *
 *   x, gamma, eps  as in rmsnorm_linear_bf16 (normed rows are fp32, not bf16).
 *   Wq        [N, K] int8 weight, values in [-127, 127].
 *   w_scale   [N] fp32 per-output-channel weight scale.
 *   y         [T, N]: bf16 or fp32 dequantised output, or, with out_dtype ==
 *             RNL_INT32, the raw int32 accumulators acc[t, n].
 *   xq_out    [T, K] int8 quantised activations, or NULL.
 *   x_scale_out [T] fp32 dequant scale amax/127, or NULL.
 *   rstd_out  [T] fp32, or NULL.
 *   K must be a multiple of 16 (16-byte int8 vectors) and at most 133144, so
 *   that |acc| <= K * 127 * 127 fits int32.
 *
 * Errors: as rmsnorm_linear_bf16 (w_scale and Wq are required).
 */
RNL_API int rmsnorm_linear_int8(const void* x, const void* gamma, float eps, const int8_t* Wq,
                        const float* w_scale, void* y, int out_dtype, int8_t* xq_out,
                        float* x_scale_out, float* rstd_out, int64_t T, int64_t K, int64_t N,
                        void* workspace, size_t workspace_bytes, void* stream);

RNL_API size_t rmsnorm_linear_int8_workspace_bytes(int64_t T, int64_t K, int64_t N, int out_dtype);

/*
 * add_rmsnorm_linear_bf16 / add_rmsnorm_linear_int8 -- residual add in front
 * of the fused norm and projection.
 *
 * AT-10 page, section 6: in the pre-attention operator the layer input is
 * first added to the residual stream and the norm reads that sum; the atom
 * table of section 3 lists the add-then-norm variant among those that also
 * give rstd.  Each call first forms
 *   x_add[t, k] = round_bf16(float(x[t, k]) + float(residual[t, k]))
 * (one fp32 addition, round to nearest even), writes it to x_add_out (the
 * new residual stream), and then computes exactly what rmsnorm_linear_bf16
 * (resp. rmsnorm_linear_int8) computes with x_add in place of x.
 *
 *   x, residual  [T, K] bf16, both required.
 *   x_add_out    [T, K] bf16 output, required; must not overlap any input
 *                or output buffer (an overlap with x or residual is
 *                rejected with RNL_ERR_ARG).
 *   all other arguments, limits and errors as in the call without the add;
 *   RNL_ERR_NULL also when residual or x_add_out is NULL.
 */
RNL_API int add_rmsnorm_linear_bf16(const void* x, const void* residual, void* x_add_out, const void* gamma,
                                    float eps, const void* W, int w_dtype, void* y, int out_dtype,
                                    float* rstd_out, int64_t T, int64_t K, int64_t N, void* workspace,
                                    size_t workspace_bytes, void* stream);

RNL_API size_t add_rmsnorm_linear_bf16_workspace_bytes(int64_t T, int64_t K, int64_t N, int w_dtype,
                                                       int out_dtype);

RNL_API int add_rmsnorm_linear_int8(const void* x, const void* residual, void* x_add_out, const void* gamma,
                                    float eps, const int8_t* Wq, const float* w_scale, void* y, int out_dtype,
                                    int8_t* xq_out, float* x_scale_out, float* rstd_out, int64_t T, int64_t K,
                                    int64_t N, void* workspace, size_t workspace_bytes, void* stream);

RNL_API size_t add_rmsnorm_linear_int8_workspace_bytes(int64_t T, int64_t K, int64_t N, int out_dtype);

/*
 * rmsnorm_linear_mxfp8 -- fused RMSNorm -> MX quantisation -> MXFP8 scaled GEMM
 * (AT-10 with AT-09's MXFP8 mode).
 *
 * AT-10 page, section 4: in MXFP8 mode the projection is one scaled matmul of
 * fp8 operands with their scales, accumulating in FP32; the SK-14 page gives
 * the MXFP8 layout: E4M3FN data, E8M0 scales, one scale per 64 elements.  The
 * fp32 normed rows (as in rmsnorm_linear_int8) are quantised per block of 64
 * consecutive k: scale X = 2^e, e = floor(log2(amax)) - 8 clamped to
 * [-127, 127] (-127 for an all-zero block), element = the E4M3 value nearest
 * to n / X (ties to even, clamped to +-448, zero as +0).  Then
 *   y[t, n] = sum over blocks b of X[t, b] * Xw[n, b] * sum_{k in b} q[t, k] * Wq[n, k]
 * accumulated in fp32, written as bf16 (RNL_BF16) or fp32 (RNL_FP32).
 *
 *   x, gamma, eps  as in rmsnorm_linear_bf16.
 *   Wq        [N, K] E4M3 bytes; w_scale [N, K/64] E8M0 bytes (2^(code - 127)).
 *   xq_out    [T, K] E4M3 bytes, or NULL; x_scale_out [T, K/64] E8M0, or NULL.
 *   rstd_out  [T] fp32, or NULL.
 *   K must be a multiple of 64.  Codes 0x7F / 0xFF (E4M3) and 255 (E8M0) are
 *   NaN and make the affected outputs NaN.
 *
 * Errors: as rmsnorm_linear_bf16 (Wq and w_scale are required).
 */
RNL_API int rmsnorm_linear_mxfp8(const void* x, const void* gamma, float eps, const uint8_t* Wq,
                                 const uint8_t* w_scale, void* y, int out_dtype, uint8_t* xq_out,
                                 uint8_t* x_scale_out, float* rstd_out, int64_t T, int64_t K, int64_t N,
                                 void* workspace, size_t workspace_bytes, void* stream);

RNL_API size_t rmsnorm_linear_mxfp8_workspace_bytes(int64_t T, int64_t K, int64_t N, int out_dtype);

/*
 * norm_proj_chain -- two-stage low-rank projection q_a_proj -> RMSNorm -> q_b_proj.
 *
 * AT-10 page, section 5 (MLAProlog query branch: bf16 product with the
 * down-projection weight, RMSNorm with gamma, bf16 cast, the normed rows
 * written out, then the bf16 product with the up-projection weight) and
 * SK-14 page section 5, orchestration mode 1 (serial pipeline).
 *
 *   x       [T, K] bf16.
 *   W_a     [R, K] bf16 (b_trans).   q_a = round_bf16(x . W_a^T)   [T, R]
 *   gamma   [R] bf16 or NULL; eps.   qr  = round_bf16(RMSNorm(q_a) * gamma)
 *   W_b     [N, R] bf16 (b_trans).   y   = round_bf16(qr . W_b^T)  [T, N]
 *   qr_out  [T, R] bf16, required (the normed low-rank query).
 *   y       [T, N] bf16.
 *   rstd_out [T] fp32 rstd of the q_a rows, or NULL.
 *   qa_out  [T, R] bf16 q_a, the rows the norm reads, or NULL.
 *   R must be a multiple of 8.  Outputs must not overlap inputs or each other.
 */
RNL_API int norm_proj_chain(const void* x, const void* W_a, const void* gamma, float eps, const void* W_b,
                    void* qr_out, void* y, float* rstd_out, void* qa_out, int64_t T, int64_t K, int64_t R,
                    int64_t N, void* workspace, size_t workspace_bytes, void* stream);

RNL_API size_t norm_proj_chain_workspace_bytes(int64_t T, int64_t K, int64_t R, int64_t N);

/*
 * mla_prolog_bf16 -- the query chain of norm_proj_chain and the KV branch of the
 * MLA prolog, with one pass over x for both first projections.
 *
 * AT-10 page, section 5: beside q_a_proj -> norm -> q_b_proj, the KV path
 * projects the same x with the KV weight (bf16 out), applies RMSNorm, multiplies
 * by gamma_ckv and casts to bf16: a second AT-10 instance sharing x.
 *
 *   x         [T, K] bf16.
 *   W_akv     [R + Rkv, K] bf16: rows [0, R) the query down-projection W_a,
 *             rows [R, R + Rkv) the KV projection W_kv (stacked by the caller).
 *   [q_a | kv] = round_bf16(x . W_akv^T)                       [T, R + Rkv]
 *   qr_out    [T, R]   = round_bf16(RMSNorm(q_a) * gamma_cq)     (required)
 *   kv_out    [T, Rkv] = round_bf16(RMSNorm(kv) * gamma_ckv)     (required)
 *   y         [T, N]   = round_bf16(qr . W_b^T), W_b [N, R] bf16.
 *   gamma_cq [R], gamma_ckv [Rkv] bf16 or NULL; one eps for both norms.
 *   rstd_q_out, rstd_kv_out [T] fp32 or NULL.
 *   qakv_out  [T, R + Rkv] bf16 [q_a | kv], the rows the two norms read, or NULL.
 *   R and Rkv must be multiples of 8.  Outputs must not overlap inputs.
 *
 * Errors: as norm_proj_chain.
 */
RNL_API int mla_prolog_bf16(const void* x, const void* W_akv, const void* gamma_cq, const void* gamma_ckv, float eps,
                            const void* W_b, void* qr_out, void* kv_out, void* y, float* rstd_q_out,
                            float* rstd_kv_out, void* qakv_out, int64_t T, int64_t K, int64_t R, int64_t Rkv,
                            int64_t N, void* workspace, size_t workspace_bytes, void* stream);

RNL_API size_t mla_prolog_bf16_workspace_bytes(int64_t T, int64_t K, int64_t R, int64_t Rkv, int64_t N);

/*
 * preattn_qkv_bf16 -- the pre-attention block around the fused norm and
 * projection: optional residual add, input RMSNorm, fused QKV projection,
 * split into heads, per-head RMSNorm of the query and key heads, optional
 * rotary embedding of both.
 *
 * AT-10 page, section 6: in the non-quantised Qwen3 pre-attention the norm of
 * x_add is followed by the bf16 product with the fused QKV weight, whose output
 * is split into Q, K and V, and Q and K get a per-head norm and RoPE.  The
 * steps, in order:
 *   x_add = round_bf16(float(x) + float(residual))   (only with a residual)
 *   p     = rmsnorm_linear_bf16(x_add or x, gamma, eps, W)       [T, N] bf16
 *   heads: columns [0, Hq D) are Hq query heads, [Hq D, (Hq+Hkv) D) Hkv key
 *          heads, the last Hkv D columns value heads, D columns each;
 *   each query / key head: n = fl(fl(float(p) * rstd_h) * gamma_q / gamma_k)
 *          with rstd_h the AT-03 rstd of its D values (head_eps);
 *   RoPE (cos, sin given): element i < D/2 of a head and element i + D/2 are
 *          rotated together by the angle of (t, i):
 *          out[i]       = fl(fl(n[i] c) - fl(n[i+D/2] s)),
 *          out[i + D/2] = fl(fl(n[i+D/2] c) + fl(n[i] s)),  c, s = cos[t,i], sin[t,i];
 *   y     = round_bf16 of that; value heads are p unchanged.
 * With D = 128 on the tiled GEMM (more than 16 tokens) the per-head stage runs
 * in the GEMM's epilogue; otherwise it is a separate pass over y.  The results
 * are the same bits either way.
 *
 *   x, residual, x_add_out, gamma, eps, rstd_out  as in add_rmsnorm_linear_bf16
 *             (residual and x_add_out together, or both NULL for no add).
 *   W         [(Hq + 2 Hkv) D, K] bf16 fused QKV weight (b_trans).
 *   y         [T, (Hq + 2 Hkv) D] bf16 output, columns Q | K | V.
 *   gamma_q, gamma_k  [D] bf16 head-norm scales, or NULL; head_eps.
 *   cos, sin  [T, D/2] fp32 rotation tables, both or neither (no RoPE).
 *   head_rstd_out [T, Hq + Hkv] fp32 rstd of every normed head, or NULL.
 *   D must be a multiple of 16 and at most 512; T (Hq + Hkv) < 2^31.
 *
 * Errors: as rmsnorm_linear_bf16; RNL_ERR_NULL also when only one of
 * residual / x_add_out or of cos / sin is given; RNL_ERR_SHAPE for D and for
 * T (Hq + Hkv).
 */
RNL_API int preattn_qkv_bf16(const void* x, const void* residual, void* x_add_out, const void* gamma, float eps,
                             const void* W, void* y, float* rstd_out, const void* gamma_q, const void* gamma_k,
                             float head_eps, const float* cos, const float* sin, float* head_rstd_out, int64_t T,
                             int64_t K, int64_t Hq, int64_t Hkv, int64_t D, void* workspace,
                             size_t workspace_bytes, void* stream);

RNL_API size_t preattn_qkv_bf16_workspace_bytes(int64_t T, int64_t K, int64_t Hq, int64_t Hkv, int64_t D);

/*
 * The atoms the fused entry points are built from.  They run the same kernels
 * and follow the same conventions (device pointers, asynchronous on `stream`,
 * validation before any HIP call, status codes); none needs a workspace.
 *
 * rms_norm_bf16 -- AT-03 RMSNorm (AT-10 page, section 3: fp32 inside, variant B
 * rstd, optional gamma, bf16 output, optional rstd output):
 *   y[t,k] = round_bf16(fl(fl(float(x[t,k]) * rstd[t]) * float(gamma[k]))).
 *   x [T,K] bf16; gamma [K] bf16 or NULL; y [T,K] bf16; rstd_out [T] or NULL.
 */
RNL_API int rms_norm_bf16(const void* x, const void* gamma, float eps, void* y, float* rstd_out,
                          int64_t T, int64_t K, void* stream);

/*
 * rms_norm_quant_int8 -- AT-03 followed by AT-05 per-token symmetric int8
 * quantisation of the fp32 normed rows (AT-10 page section 4; SK-03 page quant
 * variant).  xq [T,K] int8 and x_scale [T] fp32 (amax/127) are required;
 * rstd_out may be NULL.  K must be a multiple of 16.
 */
RNL_API int rms_norm_quant_int8(const void* x, const void* gamma, float eps, int8_t* xq,
                                float* x_scale, float* rstd_out, int64_t T, int64_t K,
                                void* stream);

/*
 * head_rms_norm_bf16 -- the per-head stage alone (AT-10 page section 6; the
 * section 9 golden chain re-norms the q_b output per head the same way):
 * the H heads of D columns starting at column col0 of every row of
 * y_in [T, ld] are normed (gamma [D] or NULL, eps) and, with cos/sin
 * [T, D/2] fp32, rotated as in preattn_qkv_bf16; the results go to the same
 * places of y_out, the other columns of y_out are not written.  y_out may be
 * y_in (in place) but may not overlap it otherwise (RNL_ERR_ARG).
 * rstd_out [T, H] or NULL.  ld and col0 multiples of 8; D a multiple of 16,
 * at most 512; col0 + H D <= ld; T H < 2^31 (RNL_ERR_SHAPE otherwise).
 */
RNL_API int head_rms_norm_bf16(const void* y_in, void* y_out, const void* gamma, float eps, const float* cos,
                               const float* sin, float* rstd_out, int64_t T, int64_t ld, int64_t col0, int64_t H,
                               int64_t D, void* stream);

/*
 * linear_heads_bf16 -- the projection of already-normed rows followed by the
 * per-head stage of preattn_qkv_bf16 (AT-10 page section 6): y = bf16(a . W^T)
 * with W [(Hq + 2 Hkv) D, K], then every query head (gamma_q) and key head
 * (gamma_k) of y normed and, with cos / sin [M, D/2] fp32, rotated exactly as
 * preattn_qkv_bf16 does; the Hkv value heads are the bf16 product.
 *   a [M, K] bf16, y [M, (Hq + 2 Hkv) D] bf16, head_rstd_out [M, Hq + Hkv] or
 *   NULL.  K a multiple of 8; D a multiple of 16, at most 512; M (Hq + Hkv) < 2^31.
 * With D = 128 and more than 16 rows the stage runs in the GEMM's epilogue
 * (one launch); otherwise the projection and a per-head pass over y (two
 * launches).  The results are the same bits either way.
 * Errors: RNL_ERR_NULL (a, W, y; cos without sin or the reverse),
 * RNL_ERR_SHAPE, RNL_ERR_ARG (head_eps), RNL_ERR_ALIGN (16 bytes; 4 for
 * head_rstd_out), RNL_ERR_HIP.
 */
RNL_API int linear_heads_bf16(const void* a, const void* W, void* y, const void* gamma_q, const void* gamma_k,
                              float head_eps, const float* cos, const float* sin, float* head_rstd_out, int64_t M,
                              int64_t K, int64_t Hq, int64_t Hkv, int64_t D, void* stream);

/*
 * linear_bf16 -- AT-09 Linear Projection, BF16 mode (AT-10 page section 4):
 * y[M,N] = a[M,K] . W[N,K]^T (b_trans), bf16 operands, fp32 accumulation,
 * y bf16 (out_dtype RNL_BF16, rounded once) or fp32 (RNL_FP32).
 */
RNL_API int linear_bf16(const void* a, const void* W, void* y, int out_dtype, int64_t M, int64_t K,
                        int64_t N, void* stream);

/*
 * linear_int8 -- AT-09 Linear Projection, INT8 W8A8 mode, with the AT-06
 * dequant: acc = xq[M,K] . Wq[N,K]^T in int32; y = fl(float(acc) *
 * fl(x_scale[m] * w_scale[n])) as bf16 or fp32, or acc itself for RNL_INT32.
 * K must be a multiple of 16 and at most 133144.
 */
RNL_API int linear_int8(const int8_t* xq, const float* x_scale, const int8_t* Wq,
                        const float* w_scale, void* y, int out_dtype, int64_t M, int64_t K,
                        int64_t N, void* stream);

/*
 * rms_norm_quant_mxfp8 -- AT-03 followed by the MX quantisation of
 * rmsnorm_linear_mxfp8: xq [T, K] E4M3 and x_scale [T, K/64] E8M0 (required),
 * rstd_out [T] or NULL.  K must be a multiple of 64.
 */
RNL_API int rms_norm_quant_mxfp8(const void* x, const void* gamma, float eps, uint8_t* xq, uint8_t* x_scale,
                                 float* rstd_out, int64_t T, int64_t K, void* stream);

/*
 * linear_mxfp8 -- AT-09 Linear Projection, MXFP8 mode: the scaled product of
 * rmsnorm_linear_mxfp8 on given MX operands, xq [M, K] / x_scale [M, K/64] and
 * Wq [N, K] / w_scale [N, K/64]; y [M, N] bf16 or fp32.
 */
RNL_API int linear_mxfp8(const uint8_t* xq, const uint8_t* x_scale, const uint8_t* Wq, const uint8_t* w_scale,
                         void* y, int out_dtype, int64_t M, int64_t K, int64_t N, void* stream);

/*
 * rnl_stream_read -- HBM streaming probe; not a step of the method.  Reads
 * `bytes` (a positive multiple of 16) of device memory at src once with
 * `workgroups` workgroups (1 to 65536) of 256 threads: 16-byte loads, 1 KiB
 * contiguous per wavefront load instruction, `unroll` (1, 2, 4, 8 or 16) loads
 * in flight per lane, grid-stride.  Each workgroup writes one word, a fold of
 * what it read, to sink[workgroup] (so the reads cannot be elided).  Its
 * duration gives the practical read bandwidth that the weight-bound paths are
 * compared with.
 * Errors: RNL_ERR_NULL, RNL_ERR_SHAPE (bytes, workgroups), RNL_ERR_ARG
 * (unroll), RNL_ERR_ALIGN (src 16-byte, sink 4-byte), RNL_ERR_HIP.
 */
RNL_API int rnl_stream_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, int unroll, void* stream);

/*
 * rnl_clock_probe -- clock probe; not a step of the method.  `workgroups`
 * (1 to 1024) wavefronts each wait `delay_us` (0 to 10^7) microseconds, then
 * spin for `microseconds` (1 to 10^7) of the 100 MHz real-time counter, and
 * wavefront b writes out[2b] = shader clock cycles elapsed over the spin
 * (s_memtime), out[2b + 1] = real-time ticks elapsed (s_memrealtime):
 * 100 * out[2b] / out[2b + 1] is the shader clock in MHz on its compute unit.
 * With 8 wavefronts each XCD gets one.  Run on a second stream beside a
 * workload, it records the clock the workload runs at.  Every wait is bounded
 * by the real-time counter, so it ends whatever else runs.
 * Errors: RNL_ERR_NULL, RNL_ERR_SHAPE, RNL_ERR_ALIGN (out 8-byte), RNL_ERR_HIP.
 */
RNL_API int rnl_clock_probe(uint64_t* out, int64_t delay_us, int64_t microseconds, int workgroups, void* stream);

/*
 * rnl_mfma_probe -- MFMA rate probe; not a step of the method.
 * `workgroups` (1 to 65536) workgroups of `waves_per_group` (1 to 16) wavefronts
 * each issue `iterations` (1 to 2^24) x 8 matrix instructions into eight
 * independent accumulators held in registers, no memory traffic:
 *   kind 0: v_mfma_f32_16x16x32_bf16            (16384 flop each)
 *   kind 1: v_mfma_i32_16x16x64_i8              (32768 op each)
 *   kind 2: v_mfma_scale_f32_16x16x128_f8f6f4   (E4M3 operands, 65536 flop each)
 * Wavefront w of workgroup b writes one word (a fold of its accumulators) to
 * sink[b * waves_per_group + w]; sink holds workgroups * waves_per_group words.
 * Its duration gives the practical matrix-core rate the contractions are
 * compared with.
 * Errors: RNL_ERR_NULL, RNL_ERR_ARG (kind), RNL_ERR_SHAPE, RNL_ERR_ALIGN (sink
 * 4-byte), RNL_ERR_HIP.
 */
RNL_API int rnl_mfma_probe(int kind, int workgroups, int waves_per_group, int64_t iterations, uint32_t* sink,
                           void* stream);

/* Static description of a status code. */
RNL_API const char* rnl_status_str(int status);

/* Detail of the last error on the calling thread ("" if none). */
RNL_API const char* rnl_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RNL_H */
