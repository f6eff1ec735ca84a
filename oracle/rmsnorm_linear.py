"""numpy reference of the fused RMSNorm -> Linear projection: the same
definitions as the C oracle (oracle/c/rnl_oracle.c), written independently in
numpy and kept as its cross-check; every pin runs against both.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
``cpu_baseline`` leg of the benchmark; never by the product path.

Pages this follows (cited by title and section):

* AT-10 page -- "PyPTO-Gym operator design pattern AT-10: RMSNorm + Linear
  fused (V->C layout), principle and MLAProlog practice":
  section 2 (CV layout and the standard compute flow),
  section 3 (V stage: RMSNorm variant A "rsqrt", variant B "sqrt + div",
  the MLA ``rms_norm`` code, the AT-03 instantiation-parameter table),
  section 4 (C stage: AT-09 BF16 mode, INT8 W8A8 mode, AT-05 / AT-06),
  section 5 (MLAProlog: q_a_proj -> norm -> q_b_proj),
  section 9 (golden reference: ``rms_norm_new`` divides x by sqrt).
* SK-03 page -- "SK-03 Linear Projection (Norm->MatMul)": the skeleton
  template, the quant variant (its per-tensor quant helper)
  and the mhc_pre variant (large reduction x tiny width, FP32 compute).
* SK-14 page -- "SK-14 General Multi-MatMul skeleton": section 5 mode 1
  (serial pipeline, MLA q_a_proj -> norm -> q_b_proj) and the
  QuantMatMulReduceSum example (dequant as acc_fp32 * (x1_scale * x2_scale)).
* Patterns page -- "PyPTO common coding patterns": section 9.17 table
  (eps is added before the reciprocal square root) and section 9.18 point 5
  (a transposed second operand multiplies by the weight's rows).

Conventions.  bf16 tensors are passed as ``uint16`` bit patterns, fp32 as
``float32``, int8 as ``int8``.  Every fp32 step is one numpy float32 operation,
which IEEE-754 rounds to nearest even; numpy never contracts a multiply and an
add.  Where the pages leave a point open, the docstring of the function that
takes it says READING and gives the choice and its reason.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
F64 = np.float64


# ----------------------------------------------------------------------------
# bf16 <-> fp32
# ----------------------------------------------------------------------------
def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact: bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even.

    AT-10 page section 2 casts the fp32 normed values to BF16 before the
    matmul; the rounding rule is not stated.  READING: IEEE round to nearest
    even on the 16 discarded bits; a NaN stays a (quiet) NaN.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        quiet = ((u >> np.uint64(16)) | np.uint64(0x0040)).astype(np.uint16)
        rounded = np.where(nan, quiet, rounded)
    return rounded


def _bf16_round_f32(x) -> np.ndarray:
    """fp32 values rounded to bf16 and widened back to fp32 (exact widening)."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# ----------------------------------------------------------------------------
# RMSNorm (AT-03 as used by AT-10)
# ----------------------------------------------------------------------------
def _row_mean_square(xf: np.ndarray) -> np.ndarray:
    """ms[t] = fl( fl(sum_k xf^2) * fl(1/K) ).

    AT-10 page section 3, variant A: square in fp32, sum along the last axis,
    multiply by 1/D.  The pages ask for fp32 reductions (the C-API-05
    constraint quoted there) but give no summation order.  READING: the
    squares (exact in fp64) are summed in fp64 and the sum is rounded to fp32
    once, so the oracle's sum is the correctly rounded value up to fp64
    round-off; 1/D is the fp32 constant fl(1/K).
    """
    K = xf.shape[-1]
    x64 = xf.astype(F64)
    S = F32(np.sum(x64 * x64, axis=-1))  # fp64 sum, one rounding to fp32
    c = F32(1.0) / F32(K)
    return (S * c).astype(F32)


def rstd_variant_b(ms: np.ndarray, eps: float) -> np.ndarray:
    """rstd = fl(1 / fl(sqrt(fl(ms + eps)))) -- AT-10 page section 3 variant B
    (sqrt then divide ones by std), the form the MLA ``rms_norm`` code uses.
    eps is added to the mean square, before the root (patterns page 9.17)."""
    var = (ms.astype(F32) + F32(eps)).astype(F32)
    std = np.sqrt(var).astype(F32)
    return (F32(1.0) / std).astype(F32)


def rstd_variant_a(ms: np.ndarray, eps: float) -> np.ndarray:
    """rstd = rsqrt(fl(ms + eps)) -- AT-10 page section 3 variant A.

    The hardware rsqrt instruction has its own error; the oracle takes the
    ideal value: 1/sqrt(var) in fp64, rounded once to fp32.
    """
    var = (ms.astype(F32) + F32(eps)).astype(F32)
    return (1.0 / np.sqrt(var.astype(F64))).astype(F32)


def rms_norm_rows(x_bits, gamma_bits, eps: float, rstd=None, variant: str = "B"):
    """Per-row RMSNorm in fp32.  Returns (n [T,K] fp32, rstd [T] fp32).

    AT-10 page section 3: xf = float(x); ms = (sum of xf^2) * (1/D);
    var = ms + eps; rstd = 1/sqrt(var); n = xf * rstd, then n * float(gamma)
    when gamma is given (gamma applied after the rstd product, as the MLA
    caller does in section 5).  If ``rstd`` is given (for instance the device's own), it is
    used instead of recomputing it, so that the normed values can be compared
    bit for bit downstream.
    """
    xf = bf16_bits_to_f32(x_bits)
    if xf.ndim != 2:
        raise ValueError("x must be [T, K]")
    if rstd is None:
        ms = _row_mean_square(xf)
        rstd = rstd_variant_b(ms, eps) if variant == "B" else rstd_variant_a(ms, eps)
    rstd = np.asarray(rstd, dtype=F32).reshape(-1)
    n = (xf * rstd[:, None]).astype(F32)
    if gamma_bits is not None:
        g = bf16_bits_to_f32(gamma_bits).reshape(1, -1)
        n = (n * g).astype(F32)
    return n, rstd


def rms_norm_rows_mla_order(x_bits, eps: float):
    """Alternative ordering of the MLA ``rms_norm`` code (AT-10 page section 3):
    each square is multiplied by 1/D before the sum.  Returns (n, rstd); no
    gamma (the caller applies it).  Used only to cross-check the ordering."""
    xf = bf16_bits_to_f32(x_bits)
    K = xf.shape[-1]
    c = F32(1.0) / F32(K)
    sq = (xf * xf).astype(F32)
    scaled = (sq * c).astype(F32)
    ms = F32(np.sum(scaled.astype(F64), axis=-1))
    rstd = rstd_variant_b(np.asarray(ms, dtype=F32), eps)
    return (xf * rstd[:, None]).astype(F32), rstd


def rms_norm_rows_golden_div(x_bits, eps: float):
    """The golden reference form of AT-10 page section 9 (``rms_norm_new``):
    x / sqrt(mean_sq + eps), a division instead of a product with rstd."""
    xf = bf16_bits_to_f32(x_bits)
    ms = _row_mean_square(xf)
    std = np.sqrt((ms + F32(eps)).astype(F32)).astype(F32)
    return (xf / std[:, None]).astype(F32)


# ----------------------------------------------------------------------------
# Projections
# ----------------------------------------------------------------------------
def project_bf16(n: np.ndarray, W_bits) -> np.ndarray:
    """y = bf16(n) . W^T as fp32 [T, N].

    AT-10 page section 2 and 4: the normed rows are cast to BF16 and
    multiplied by the weight stored [N, K], whose rows are the output columns
    (patterns page 9.18 point 5).  READING: the products of two bf16 values are
    exact in fp64; they are accumulated in fp64 and the result is rounded once
    to fp32.  A bf16 output is that fp32 value rounded to bf16.
    """
    a = _bf16_round_f32(n).astype(F64)
    w = bf16_bits_to_f32(W_bits).astype(F64)
    return (a @ w.T).astype(F32)


def project_fp32(n: np.ndarray, W: np.ndarray) -> np.ndarray:
    """FP32 compute of the SK-03 page's mhc_pre variant: normed rows stay fp32,
    W is fp32 [N, K]; fp32 x fp32 products are exact in fp64, summed in fp64,
    rounded once to fp32."""
    return (n.astype(F64) @ np.asarray(W, dtype=F32).astype(F64).T).astype(F32)


# ----------------------------------------------------------------------------
# INT8 W8A8 (AT-09 INT8 mode, AT-05 quant, AT-06 dequant)
# ----------------------------------------------------------------------------
def quant_values(n: np.ndarray, s: np.ndarray) -> np.ndarray:
    """q = saturate_int8(round_half_even(fl(n * s))), saturating at +-127.

    SK-03 page, quant variant: ``common.py quant`` casts with RINT, then
    ROUND, then TRUNC with saturation to INT8.  READING: one round-to-nearest-
    even to an integer; the later casts leave an in-range integer unchanged;
    saturation is symmetric at +-127 (the symmetric scale never needs -128).
    """
    v = (n.astype(F32) * np.asarray(s, dtype=F32)).astype(F32)
    r = np.rint(v)  # numpy rint rounds half to even
    return np.clip(r, -127.0, 127.0).astype(np.int8)


def quant_rows(n: np.ndarray):
    """Per-token symmetric dynamic quant (AT-05; SK-03 page quant variant).

    amax[t] = max_k |n[t,k]|; s = fl(127 / amax) (AT-10 page section 4: 127.0 /
    max gives the scale); q = quant_values(n, s); dequant scale x_scale =
    fl(amax / 127) (SK-03 page: the symmetric scale is max/127.0 and is
    returned for dequant).  READING for an all-zero row (amax = 0, which the
    pages leave open): q = 0 and x_scale = 0.
    Returns (q int8 [T,K], x_scale fp32 [T], s fp32 [T]).
    """
    n = n.astype(F32)
    amax = np.max(np.abs(n), axis=-1).astype(F32)
    zero = amax == 0
    safe = np.where(zero, F32(1.0), amax).astype(F32)
    s = (F32(127.0) / safe).astype(F32)
    s = np.where(zero, F32(0.0), s).astype(F32)
    q = quant_values(n, s[:, None])
    x_scale = (amax / F32(127.0)).astype(F32)
    return q, x_scale, s


def int8_gemm(q: np.ndarray, Wq: np.ndarray) -> np.ndarray:
    """acc[t, j] = sum_k q[t,k] * Wq[j,k], exact (AT-09 INT8 mode: int8 x int8
    -> INT32 matmul with b_trans).  Raises if a sum leaves int32.

    Every product is an integer of magnitude at most 128^2, so every partial
    sum is an integer of magnitude at most K * 128^2.  While that bound is
    below 2^53 each partial sum is exactly representable in fp64, so an fp64
    accumulation gives the exact integer in any summation order; that form is
    used then (numpy has no fast integer product).  Beyond it the sum is formed
    in int64 (int8_gemm_int64)."""
    Wq = np.asarray(Wq, dtype=np.int8)
    K = q.shape[-1]
    if K * 128 * 128 < 2**53:
        acc = (q.astype(F64) @ Wq.astype(F64).T).astype(np.int64)
    else:
        acc = int8_gemm_int64(q, Wq)
    if acc.size and (acc.max() > 2**31 - 1 or acc.min() < -(2**31)):
        raise OverflowError("int8 GEMM result does not fit int32")
    return acc


def int8_gemm_int64(q: np.ndarray, Wq: np.ndarray) -> np.ndarray:
    """The same sum in int64 arithmetic (slow; the reference for the fp64 form)."""
    return q.astype(np.int64) @ np.asarray(Wq, dtype=np.int8).astype(np.int64).T


def dequant(acc: np.ndarray, x_scale: np.ndarray, w_scale: np.ndarray) -> np.ndarray:
    """y = fl( fl(float(acc)) * fl(x_scale[t] * w_scale[j]) ) as fp32.

    AT-06 multiplies the int32 result by the activation and weight scales; the
    SK-14 page's QuantMatMulReduceSum fixes the order: cast the int32 result to
    fp32, form scale_mul = x1_scale * x2_scale, multiply.  The int -> fp32
    cast rounds to nearest even.
    """
    accf = acc.astype(F32)
    sm = (np.asarray(x_scale, dtype=F32)[:, None] * np.asarray(w_scale, dtype=F32)[None, :]).astype(F32)
    return (accf * sm).astype(F32)


# ----------------------------------------------------------------------------
# Residual add before the norm (pre-attention input norm)
# ----------------------------------------------------------------------------
def add_residual(x_bits, r_bits) -> np.ndarray:
    """x_add = x + residual, as bf16 bits [T, K].

    AT-10 page section 6: in the pre-attention operator the input is usually
    first added to the residual stream and the norm is applied to that sum;
    the atom table of section 3 lists the in-place add-then-norm variant
    among the ones that also output rstd.  READING: the two bf16 operands are
    added in fp32 (one rounding) and the sum is rounded to bf16 (nearest
    even), which is the bf16 tensor the norm then reads and the new residual
    stream the caller keeps.
    """
    xf = bf16_bits_to_f32(x_bits)
    rf = bf16_bits_to_f32(r_bits)
    return f32_to_bf16_bits((xf + rf).astype(F32))


# ----------------------------------------------------------------------------
# MXFP8 (AT-09 MXFP8 mode): E4M3 elements, one E8M0 scale per 64 elements
# ----------------------------------------------------------------------------
MX_BLOCK = 64
E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 (FN: no infinities) bytes -> fp32 values.  Sign bit, 4 exponent bits
    with bias 7, 3 mantissa bits; exponent field 0 is subnormal (m * 2^-9);
    exponent 15 with mantissa 7 is NaN.  The SK-14 page names the data format of
    its MXFP8 grouped matmul as E4M3FN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return (sign * mag).astype(F32)


def e4m3_encode(v) -> np.ndarray:
    """fp32 -> E4M3 bytes, round to nearest even, saturating to +-448.

    READING: the pages fix the format but not the conversion; the OCP MX rule
    is taken -- the nearest representable value (ties to the even mantissa),
    and magnitudes beyond the largest normal 448 are clamped to it.  A zero
    (of either sign) encodes as +0.
    """
    v = np.asarray(v, dtype=F64)
    a = np.abs(v)
    _, e = np.frexp(a)                          # a = f * 2^e, f in [0.5, 1)
    q = np.maximum(e - 1, -6) - 3               # exponent of the spacing at a
    r = np.rint(a * np.exp2(-q)) * np.exp2(q)   # exact scaling, RNE to the spacing
    r = np.minimum(r, E4M3_MAX)
    _, e2 = np.frexp(r)
    E = e2 - 1
    normal = r >= 2.0 ** -6
    exp_field = np.where(normal, E + 7, 0)
    mant = np.where(normal, r * np.exp2(-E.astype(F64)) * 8 - 8, r * 2.0 ** 9)
    code = (exp_field.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    code = np.where(r == 0, 0, code | np.where(v < 0, 0x80, 0))
    return code.astype(np.uint8)


def e8m0_decode(codes) -> np.ndarray:
    """E8M0 scale bytes -> 2^(code - 127) (fp64; code 255 is NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def mx_quant_rows(n: np.ndarray, block: int = MX_BLOCK):
    """MX quantisation of fp32 rows n [T, K] (K a multiple of ``block``).
    Returns (codes [T, K] E4M3 bytes, scales [T, K/block] E8M0 bytes).

    AT-09 page text (AT-10 page section 4): MXFP8 mode multiplies fp8 operands
    with their scales inside one scaled matmul; the SK-14 page gives the layout
    (E4M3FN data, E8M0 scale, one scale shared by 64 elements).  READING (how
    the activations get their scale, not stated): the OCP MX rule -- per block
    of 64 consecutive k, X = 2^(floor(log2(amax)) - 8) with 8 the largest
    exponent of E4M3, the exponent clamped to E8M0's [-127, 127]; an all-zero
    block takes X = 2^-127; each element is e4m3_encode(n / X).
    """
    n = np.asarray(n, dtype=F32)
    T, K = n.shape
    nb = n.reshape(T, K // block, block).astype(F64)
    amax = np.max(np.abs(nb), axis=-1)
    _, e = np.frexp(amax)
    shared = np.where(amax > 0, e - 1 - 8, -127)
    shared = np.clip(shared, -127, 127)
    codes = e4m3_encode(nb * np.exp2(-shared.astype(F64))[..., None]).reshape(T, K)
    return codes, (shared + 127).astype(np.uint8)


def mx_scaled_mm(qx, sx, qw, sw, block: int = MX_BLOCK) -> np.ndarray:
    """scaled_mm(x_fp8, w_fp8, FP32, x_scale, w_scale) with W stored [N, K]:
    y[t, n] = sum over blocks b of X_x[t, b] X_w[n, b] sum_{k in b} x[t, k] w[n, k].

    The E4M3 products are exact and every scale is a power of two, so the oracle
    forms the exact sum in fp64 and rounds once to fp32 (AT-10 page section 4:
    the MXFP8 product accumulates into FP32).
    """
    xf = e4m3_decode(qx).astype(F64)
    wf = e4m3_decode(qw).astype(F64)
    T, K = xf.shape
    N = wf.shape[0]
    xs = e8m0_decode(sx)
    ws = e8m0_decode(sw)
    xb = (xf.reshape(T, K // block, block) * xs[..., None]).reshape(T, K)
    wb = (wf.reshape(N, K // block, block) * ws[..., None]).reshape(N, K)
    return (xb @ wb.T).astype(F32)


# ----------------------------------------------------------------------------
# Post-projection V stage: per-head RMSNorm and rotary embedding
# ----------------------------------------------------------------------------
def rope_rotate_half(n: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotary embedding of fp32 head vectors n [R, D] by the angles whose
    cosines and sines are cos, sin [R, D/2] (fp32).

    AT-10 page section 6 and the SK-03 page (key features: the optional V
    stage after the projection) name RoPE after the per-head norm but do not
    define it.  READING: the rotate-half pairing of the Qwen3 family the AT-10
    page names -- element i is rotated together with element i + D/2 -- with
    the angles supplied per row and pair by the caller, in fp32 on the normed
    values before the bf16 cast, every product and sum rounded once:
        out[i]       = fl( fl(n[i] c[i])       - fl(n[i + D/2] s[i]) )
        out[i + D/2] = fl( fl(n[i + D/2] c[i]) + fl(n[i] s[i]) )
    """
    n = np.asarray(n, dtype=F32)
    h = n.shape[-1] // 2
    c = np.asarray(cos, dtype=F32)
    s = np.asarray(sin, dtype=F32)
    lo, hi = n[..., :h], n[..., h:]
    out = np.empty_like(n)
    out[..., :h] = ((lo * c).astype(F32) - (hi * s).astype(F32)).astype(F32)
    out[..., h:] = ((hi * c).astype(F32) + (lo * s).astype(F32)).astype(F32)
    return out


def head_rms_norm(y_bits, col0: int, H: int, D: int, gamma_bits, eps: float, cos=None, sin=None, rstd=None):
    """Per-head RMSNorm of the H heads of D columns that start at column col0
    of y [T, N] (bf16 bits), optionally followed by RoPE; columns outside the
    heads are returned unchanged.  Returns (out bits [T, N], rstd [T, H]).

    AT-10 page section 6: after the fused QKV projection the output is split
    into Q, K and V and a norm is applied per head; section 9's golden chain
    likewise reshapes the q_b output to (heads, head_dim) and applies RMSNorm
    again.  READING: each head is one AT-03 row of D values read from the
    bf16 projection output (the tensor the split takes apart), normed as in
    rms_norm_rows with gamma [D] shared by the heads, rotated by RoPE when
    cos/sin [T, D/2] are given (the same angles for every head of a token),
    and rounded to bf16.
    """
    y = np.asarray(y_bits, dtype=np.uint16)
    T = y.shape[0]
    seg = y[:, col0:col0 + H * D].reshape(T * H, D)
    n, r = rms_norm_rows(seg, gamma_bits, eps, None if rstd is None else np.asarray(rstd, dtype=F32).reshape(-1))
    if cos is not None:
        c = np.repeat(np.asarray(cos, dtype=F32), H, axis=0)  # row t*H + h takes the angles of token t
        sn = np.repeat(np.asarray(sin, dtype=F32), H, axis=0)
        n = rope_rotate_half(n, c, sn)
    out = y.copy()
    out[:, col0:col0 + H * D] = f32_to_bf16_bits(n).reshape(T, H * D)
    return out, r.reshape(T, H)


def preattn_qkv(x_bits, r_bits, gamma_bits, eps, W_bits, Hq, Hkv, D, gq_bits, gk_bits, head_eps,
                cos=None, sin=None, rstd=None, head_rstd=None):
    """Pre-attention block of the AT-10 page section 6: optional residual add,
    input RMSNorm, fused QKV projection (W [(Hq + 2 Hkv) D, K], columns Q | K |
    V), split into Hq query heads, Hkv key heads and Hkv value heads of D
    columns, per-head RMSNorm of Q (gamma_q) and K (gamma_k) with RoPE on both,
    V as projected.

    Returns a dict: x_add (bits or None), y_proj (bf16 bits of the projection),
    y32 (the projection in fp32), y (bf16 bits after the head stage), rstd [T],
    head_rstd [T, Hq + Hkv].
    ``rstd`` / ``head_rstd`` replace the computed values when given (the
    device's own), so that downstream values can be compared bit for bit.
    """
    xa = None
    if r_bits is not None:
        xa = add_residual(x_bits, r_bits)
        x_bits = xa
    y32, yb, rstd = rmsnorm_linear_bf16(x_bits, gamma_bits, eps, W_bits, rstd)
    hr = None if head_rstd is None else np.asarray(head_rstd, dtype=F32)
    y, rq = head_rms_norm(yb, 0, Hq, D, gq_bits, head_eps, cos, sin, None if hr is None else hr[:, :Hq])
    y, rk = head_rms_norm(y, Hq * D, Hkv, D, gk_bits, head_eps, cos, sin, None if hr is None else hr[:, Hq:])
    return {"x_add": xa, "y_proj": yb, "y32": y32, "y": y, "rstd": rstd,
            "head_rstd": np.concatenate([rq, rk], axis=1)}


# ----------------------------------------------------------------------------
# Entry points (same names and argument meanings as the C-ABI library)
# ----------------------------------------------------------------------------
def rmsnorm_linear_bf16(x_bits, gamma_bits, eps, W_bits, rstd=None):
    """AT-10: RMSNorm (fp32) -> bf16 cast -> product with W[N,K] transposed.

    Returns (y32 fp32 [T,N], y_bf16 bits [T,N], rstd [T]).
    """
    n, rstd = rms_norm_rows(x_bits, gamma_bits, eps, rstd)
    y32 = project_bf16(n, W_bits)
    return y32, f32_to_bf16_bits(y32), rstd


def rmsnorm_linear_fp32w(x_bits, gamma_bits, eps, W, rstd=None):
    """SK-03 page mhc_pre variant: normed rows kept fp32 (no bf16 cast), fp32
    weight [N, K], fp32 output.  Returns (y32 [T,N], rstd [T])."""
    n, rstd = rms_norm_rows(x_bits, gamma_bits, eps, rstd)
    return project_fp32(n, W), rstd


def rmsnorm_linear_int8(x_bits, gamma_bits, eps, Wq, w_scale, rstd=None):
    """AT-11 = AT-10 with the INT8 W8A8 projection (AT-05 -> INT32 matmul ->
    AT-06).  The fp32 normed rows are quantized (AT-10 page section 6: the
    Phase-1 sketch quantizes ``normed``).  Returns a dict with q, x_scale,
    acc (int64), y32 (fp32), y_bf16 (bits), rstd."""
    n, rstd = rms_norm_rows(x_bits, gamma_bits, eps, rstd)
    q, x_scale, _ = quant_rows(n)
    acc = int8_gemm(q, Wq)
    y32 = dequant(acc, x_scale, w_scale)
    return {"q": q, "x_scale": x_scale, "acc": acc, "y32": y32,
            "y_bf16": f32_to_bf16_bits(y32), "rstd": rstd}


def norm_proj_chain(x_bits, Wa_bits, gamma_bits, eps, Wb_bits, rstd=None, qa_bits=None):
    """MLA q_a_proj -> RMSNorm -> q_b_proj (AT-10 page section 5; SK-14 page
    section 5 mode 1).

    q_a = bf16(x . W_a^T); qr = bf16(RMSNorm(q_a) * gamma) is the second
    output; y = bf16(qr . W_b^T).  If ``qa_bits``
    is given (the device's q_a) the norm starts from it, and if ``rstd`` is
    given it replaces the recomputed one.  Returns a dict with qa (bits),
    qr (bits), y32 (fp32), y_bf16 (bits), rstd.
    """
    if qa_bits is None:
        qa_bits = f32_to_bf16_bits(project_bf16(bf16_bits_to_f32(x_bits), Wa_bits))
    n, rstd = rms_norm_rows(qa_bits, gamma_bits, eps, rstd)
    qr_bits = f32_to_bf16_bits(n)
    y32 = project_bf16(bf16_bits_to_f32(qr_bits), Wb_bits)
    return {"qa": qa_bits, "qr": qr_bits, "y32": y32, "y_bf16": f32_to_bf16_bits(y32), "rstd": rstd}


def rmsnorm_linear_mxfp8(x_bits, gamma_bits, eps, qw, sw, rstd=None):
    """AT-10 with AT-09's MXFP8 mode: the fp32 normed rows are MX-quantised
    (64-element blocks) and multiplied by the MXFP8 weight (E4M3 [N, K] with
    E8M0 scales [N, K/64]) in one scaled product accumulating in fp32.
    Returns a dict with q (E4M3 bytes), x_scale (E8M0 bytes), y32, y_bf16 (bits),
    rstd."""
    n, rstd = rms_norm_rows(x_bits, gamma_bits, eps, rstd)
    q, xs = mx_quant_rows(n)
    y32 = mx_scaled_mm(q, xs, qw, sw)
    return {"q": q, "x_scale": xs, "y32": y32, "y_bf16": f32_to_bf16_bits(y32), "rstd": rstd}


def mla_prolog(x_bits, Wa_bits, gq_bits, eps, Wb_bits, Wkv_bits, gkv_bits, rstd=None, rstd_kv=None):
    """The query chain and the KV branch of the MLA prolog on one x (AT-10 page
    section 5: besides q_a_proj -> norm -> q_b_proj, the KV path projects the
    same x with the KV weight in BF16, applies RMSNorm, multiplies by
    gamma_ckv and casts to BF16 -- a second AT-10 instance in parallel).

    kv = bf16(x . W_kv^T); kv_out = bf16(RMSNorm(kv) * gamma_ckv).  READING: the
    whole kv row is normed (the pages norm the KV projection as one row; a
    rotary slice of it is not part of this step).  Returns norm_proj_chain's
    dict plus kv (bits), kv_out (bits) and rstd_kv; ``rstd`` / ``rstd_kv``
    replace the computed values when given.
    """
    out = norm_proj_chain(x_bits, Wa_bits, gq_bits, eps, Wb_bits, rstd)
    kv = f32_to_bf16_bits(project_bf16(bf16_bits_to_f32(x_bits), Wkv_bits))
    n, rkv = rms_norm_rows(kv, gkv_bits, eps, rstd_kv)
    out.update(kv=kv, kv_out=f32_to_bf16_bits(n), rstd_kv=rkv)
    return out


def add_rmsnorm_linear_bf16(x_bits, r_bits, gamma_bits, eps, W_bits, rstd=None):
    """Residual add, then AT-10 on the sum.  Returns (x_add bits, y32, y_bf16
    bits, rstd)."""
    xa = add_residual(x_bits, r_bits)
    y32, ybf, rstd = rmsnorm_linear_bf16(xa, gamma_bits, eps, W_bits, rstd)
    return xa, y32, ybf, rstd


def add_rmsnorm_linear_fp32w(x_bits, r_bits, gamma_bits, eps, W, rstd=None):
    """Residual add, then the fp32-weight variant.  Returns (x_add bits, y32, rstd)."""
    xa = add_residual(x_bits, r_bits)
    y32, rstd = rmsnorm_linear_fp32w(xa, gamma_bits, eps, W, rstd)
    return xa, y32, rstd


def add_rmsnorm_linear_int8(x_bits, r_bits, gamma_bits, eps, Wq, w_scale, rstd=None):
    """Residual add, then AT-11 on the sum.  Returns the dict of
    rmsnorm_linear_int8 with the x_add bits under "x_add"."""
    xa = add_residual(x_bits, r_bits)
    out = rmsnorm_linear_int8(xa, gamma_bits, eps, Wq, w_scale, rstd)
    out["x_add"] = xa
    return out
