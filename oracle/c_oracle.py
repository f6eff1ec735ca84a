"""The C oracle (oracle/c/rnl_oracle.c) behind the same function names and
arguments as the numpy reference (oracle/rmsnorm_linear.py).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
``cpu_baseline`` leg of the benchmark; never by the product path.

Every arithmetic step runs in the C library; this module only passes numpy
buffers through ctypes and chains the C steps in the order the pages give
(each function cites them).  bf16 tensors are ``uint16`` bit patterns, fp32
``float32``, int8 ``int8``, as in the numpy reference.

Rows are split over ``threads()`` POSIX threads inside the library (at most 16
by default, the CPU share a GPU gets; ``set_threads`` changes it).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

F32 = np.float32
_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librnl_oracle.so")

_lib = None
_threads = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)))


def set_threads(n: int) -> None:
    """Threads the row loops use (1: the calling thread only)."""
    global _threads
    _threads = max(1, int(n))


def threads() -> int:
    return _threads


def cpu_count() -> int:
    """Online host CPUs as the C library sees them (sysconf)."""
    return int(_load().orc_cpu_count())


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build_oracle

        build_oracle.build()
    lib = ctypes.CDLL(LIB_PATH)
    p, i64, f, i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    sig = {
        "orc_cpu_count": ([], i),
        "orc_f32_to_bf16": ([p, i64, p], None),
        "orc_bf16_to_f32": ([p, i64, p], None),
        "orc_rms_norm_rows": ([p, p, f, i64, i64, p, i, p, p, i], None),
        "orc_rms_norm_rows_mla_order": ([p, f, i64, i64, p, p], None),
        "orc_rms_norm_rows_golden_div": ([p, f, i64, i64, p], None),
        "orc_project_bf16": ([p, p, i64, i64, i64, p, i], None),
        "orc_project_fp32": ([p, p, i64, i64, i64, p, i], None),
        "orc_quant_rows": ([p, i64, i64, p, p, p], None),
        "orc_quant_values": ([p, p, i64, i64, p], None),
        "orc_int8_gemm": ([p, p, i64, i64, i64, p, i], i),
        "orc_dequant": ([p, p, p, i64, i64, p], None),
        "orc_add_residual": ([p, p, i64, p], None),
        "orc_rope_rotate_half": ([p, i64, i64, p, p, p], None),
        "orc_head_rms_norm": ([p, i64, i64, i64, i64, i64, p, f, p, p, p, p, p], None),
        "orc_e4m3_decode": ([p, i64, p], None),
        "orc_e8m0_decode": ([p, i64, p], None),
        "orc_e4m3_encode": ([p, i64, p], None),
        "orc_mx_quant_rows": ([p, i64, i64, p, p], None),
        "orc_mx_scaled_mm": ([p, p, p, p, i64, i64, i64, p, i], None),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _c(a, dtype):
    """A C-contiguous array of dtype, at least 1-D (a copy only when needed)."""
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ----------------------------------------------------------------------------
# bf16 <-> fp32
# ----------------------------------------------------------------------------
def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, dtype=F32)
    _load().orc_bf16_to_f32(_p(b), b.size, _p(out))
    return out


def f32_to_bf16_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns, nearest even (AT-10 page section 2's BF16 cast;
    the rounding is a READING)."""
    a = _c(x, F32)
    out = np.empty(a.shape, dtype=np.uint16)
    _load().orc_f32_to_bf16(_p(a), a.size, _p(out))
    return out


# ----------------------------------------------------------------------------
# RMSNorm (AT-10 page section 3)
# ----------------------------------------------------------------------------
def rms_norm_rows(x_bits, gamma_bits, eps: float, rstd=None, variant: str = "B"):
    """Per-row RMSNorm in fp32: (n [T,K] fp32, rstd [T] fp32).  Variant B (sqrt
    then divide) or A (ideal rsqrt); a given ``rstd`` (the device's) replaces the
    computed one."""
    x = _c(x_bits, np.uint16)
    if x.ndim != 2:
        raise ValueError("x must be [T, K]")
    T, K = x.shape
    g = None if gamma_bits is None else _c(gamma_bits, np.uint16).reshape(-1)
    rin = None if rstd is None else _c(rstd, F32).reshape(-1)
    n = np.empty((T, K), dtype=F32)
    r = np.empty(T, dtype=F32)
    _load().orc_rms_norm_rows(_p(x), _p(g), float(eps), T, K, _p(rin), 1 if variant == "A" else 0, _p(n), _p(r),
                              _threads)
    return n, r


def rms_norm_rows_mla_order(x_bits, eps: float):
    """The MLA rms_norm code's ordering (section 3): (n, rstd), no gamma."""
    x = _c(x_bits, np.uint16)
    T, K = x.shape
    n = np.empty((T, K), dtype=F32)
    r = np.empty(T, dtype=F32)
    _load().orc_rms_norm_rows_mla_order(_p(x), float(eps), T, K, _p(n), _p(r))
    return n, r


def rms_norm_rows_golden_div(x_bits, eps: float):
    """Section 9's golden form: x / sqrt(ms + eps)."""
    x = _c(x_bits, np.uint16)
    T, K = x.shape
    n = np.empty((T, K), dtype=F32)
    _load().orc_rms_norm_rows_golden_div(_p(x), float(eps), T, K, _p(n))
    return n


# ----------------------------------------------------------------------------
# Projections (AT-09; AT-10 page sections 2, 4; SK-03 page mhc_pre)
# ----------------------------------------------------------------------------
def project_bf16(n, W_bits) -> np.ndarray:
    """y = bf16(n) . W^T as fp32 [T, N], W [N, K] bf16 bits."""
    a = _c(n, F32)
    w = _c(W_bits, np.uint16)
    T, K = a.shape
    N = w.shape[0]
    assert w.shape[1] == K
    y = np.empty((T, N), dtype=F32)
    _load().orc_project_bf16(_p(a), _p(w), T, K, N, _p(y), _threads)
    return y


def project_fp32(n, W) -> np.ndarray:
    """FP32 compute (mhc_pre): y = n . W^T, W [N, K] fp32, no bf16 cast."""
    a = _c(n, F32)
    w = _c(W, F32)
    T, K = a.shape
    N = w.shape[0]
    assert w.shape[1] == K
    y = np.empty((T, N), dtype=F32)
    _load().orc_project_fp32(_p(a), _p(w), T, K, N, _p(y), _threads)
    return y


# ----------------------------------------------------------------------------
# INT8 W8A8 (AT-09 INT8 mode, AT-05, AT-06)
# ----------------------------------------------------------------------------
def quant_values(n, s) -> np.ndarray:
    """q = saturate_+-127(rint(fl(n * s))) with s [T] (or [T, 1])."""
    a = _c(n, F32)
    T, K = a.shape
    sv = _c(np.broadcast_to(np.asarray(s, dtype=F32).reshape(-1, 1), (T, 1)), F32).reshape(-1)
    q = np.empty((T, K), dtype=np.int8)
    _load().orc_quant_values(_p(a), _p(sv), T, K, _p(q))
    return q


def quant_rows(n):
    """Per-token symmetric quant: (q int8 [T,K], x_scale fp32 [T], s fp32 [T])."""
    a = _c(n, F32)
    T, K = a.shape
    q = np.empty((T, K), dtype=np.int8)
    xs = np.empty(T, dtype=F32)
    s = np.empty(T, dtype=F32)
    _load().orc_quant_rows(_p(a), T, K, _p(q), _p(xs), _p(s))
    return q, xs, s


def int8_gemm(q, Wq) -> np.ndarray:
    """acc[t, j] = sum_k q[t,k] Wq[j,k] in int64; raises if a sum leaves int32."""
    a = _c(q, np.int8)
    w = _c(Wq, np.int8)
    T, K = a.shape
    N = w.shape[0]
    assert w.shape[1] == K
    acc = np.empty((T, N), dtype=np.int64)
    if _load().orc_int8_gemm(_p(a), _p(w), T, K, N, _p(acc), _threads):
        raise OverflowError("int8 GEMM result does not fit int32")
    return acc


int8_gemm_int64 = int8_gemm  # the C sum is int64 already


def dequant(acc, x_scale, w_scale) -> np.ndarray:
    """y = fl(fl(float(acc)) * fl(x_scale[t] * w_scale[j])) (SK-14 page order)."""
    a = _c(acc, np.int64)
    T, N = a.shape
    xs = _c(x_scale, F32).reshape(-1)
    ws = _c(w_scale, F32).reshape(-1)
    y = np.empty((T, N), dtype=F32)
    _load().orc_dequant(_p(a), _p(xs), _p(ws), T, N, _p(y))
    return y


# ----------------------------------------------------------------------------
# Residual add (AT-10 page section 6)
# ----------------------------------------------------------------------------
def add_residual(x_bits, r_bits) -> np.ndarray:
    """x_add = bf16(fl(x + residual)) as bf16 bits."""
    x = _c(x_bits, np.uint16)
    r = _c(r_bits, np.uint16)
    assert x.shape == r.shape
    out = np.empty(x.shape, dtype=np.uint16)
    _load().orc_add_residual(_p(x), _p(r), x.size, _p(out))
    return out


# ----------------------------------------------------------------------------
# Per-head norm + RoPE (AT-10 page section 6)
# ----------------------------------------------------------------------------
def rope_rotate_half(n, cos, sin) -> np.ndarray:
    """Rotate-half RoPE of fp32 rows n [R, D] by cos, sin [R, D/2]."""
    a = _c(n, F32)
    shape = a.shape
    D = shape[-1]
    a = a.reshape(-1, D)
    R = a.shape[0]
    c = _c(np.broadcast_to(np.asarray(cos, dtype=F32), shape[:-1] + (D // 2,)), F32).reshape(R, D // 2)
    s = _c(np.broadcast_to(np.asarray(sin, dtype=F32), shape[:-1] + (D // 2,)), F32).reshape(R, D // 2)
    out = np.empty_like(a)
    _load().orc_rope_rotate_half(_p(a), R, D, _p(c), _p(s), _p(out))
    return out.reshape(shape)


def head_rms_norm(y_bits, col0: int, H: int, D: int, gamma_bits, eps: float, cos=None, sin=None, rstd=None):
    """Per-head RMSNorm (+ RoPE) of the H heads of D columns from col0 of y [T, N]
    (bf16 bits): (out bits [T, N], rstd [T, H])."""
    y = _c(y_bits, np.uint16)
    T, ld = y.shape
    g = None if gamma_bits is None else _c(gamma_bits, np.uint16).reshape(-1)
    c = None if cos is None else _c(cos, F32).reshape(T, D // 2)
    s = None if sin is None else _c(sin, F32).reshape(T, D // 2)
    rin = None if rstd is None else _c(rstd, F32).reshape(T, H)
    out = np.empty_like(y)
    r = np.empty((T, H), dtype=F32)
    _load().orc_head_rms_norm(_p(y), T, ld, col0, H, D, _p(g), float(eps), _p(c), _p(s), _p(rin), _p(out), _p(r))
    return out, r


# ----------------------------------------------------------------------------
# MXFP8 (AT-09 MXFP8 mode)
# ----------------------------------------------------------------------------
MX_BLOCK = 64


def e4m3_decode(codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, dtype=F32)
    _load().orc_e4m3_decode(_p(c), c.size, _p(out))
    return out


def e4m3_encode(v) -> np.ndarray:
    a = _c(v, np.float64)
    out = np.empty(a.shape, dtype=np.uint8)
    _load().orc_e4m3_encode(_p(a), a.size, _p(out))
    return out


def e8m0_decode(codes) -> np.ndarray:
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    _load().orc_e8m0_decode(_p(c), c.size, _p(out))
    return out


def mx_quant_rows(n, block: int = MX_BLOCK):
    """MX quant of fp32 rows: (E4M3 codes [T, K], E8M0 scales [T, K/64])."""
    assert block == MX_BLOCK
    a = _c(n, F32)
    T, K = a.shape
    codes = np.empty((T, K), dtype=np.uint8)
    scales = np.empty((T, K // MX_BLOCK), dtype=np.uint8)
    _load().orc_mx_quant_rows(_p(a), T, K, _p(codes), _p(scales))
    return codes, scales


def mx_scaled_mm(qx, sx, qw, sw, block: int = MX_BLOCK) -> np.ndarray:
    """scaled_mm of MX operands with W [N, K]: fp32 [T, N]."""
    assert block == MX_BLOCK
    a, b = _c(qx, np.uint8), _c(qw, np.uint8)
    xs, ws = _c(sx, np.uint8), _c(sw, np.uint8)
    T, K = a.shape
    N = b.shape[0]
    y = np.empty((T, N), dtype=F32)
    _load().orc_mx_scaled_mm(_p(a), _p(xs), _p(b), _p(ws), T, K, N, _p(y), _threads)
    return y


# ----------------------------------------------------------------------------
# Entry points: the C steps chained in the pages' order
# ----------------------------------------------------------------------------
def rmsnorm_linear_bf16(x_bits, gamma_bits, eps, W_bits, rstd=None):
    """AT-10: RMSNorm -> bf16 cast -> product with W[N,K]^T: (y32, y_bf16 bits, rstd)."""
    n, rstd = rms_norm_rows(x_bits, gamma_bits, eps, rstd)
    y32 = project_bf16(n, W_bits)
    return y32, f32_to_bf16_bits(y32), rstd


def rmsnorm_linear_fp32w(x_bits, gamma_bits, eps, W, rstd=None):
    """SK-03 mhc_pre: fp32 normed rows times fp32 W: (y32, rstd)."""
    n, rstd = rms_norm_rows(x_bits, gamma_bits, eps, rstd)
    return project_fp32(n, W), rstd


def rmsnorm_linear_int8(x_bits, gamma_bits, eps, Wq, w_scale, rstd=None):
    """AT-11: norm -> per-token quant -> int8 GEMM -> dequant (dict)."""
    n, rstd = rms_norm_rows(x_bits, gamma_bits, eps, rstd)
    q, x_scale, _ = quant_rows(n)
    acc = int8_gemm(q, Wq)
    y32 = dequant(acc, x_scale, w_scale)
    return {"q": q, "x_scale": x_scale, "acc": acc, "y32": y32, "y_bf16": f32_to_bf16_bits(y32), "rstd": rstd}


def norm_proj_chain(x_bits, Wa_bits, gamma_bits, eps, Wb_bits, rstd=None, qa_bits=None):
    """MLA q_a_proj -> RMSNorm -> q_b_proj (AT-10 page section 5): dict with qa,
    qr (bits), y32, y_bf16, rstd; a given qa_bits / rstd (the device's) replaces
    the computed ones."""
    if qa_bits is None:
        qa_bits = f32_to_bf16_bits(project_bf16(bf16_bits_to_f32(x_bits), Wa_bits))
    n, rstd = rms_norm_rows(qa_bits, gamma_bits, eps, rstd)
    qr_bits = f32_to_bf16_bits(n)
    y32 = project_bf16(bf16_bits_to_f32(qr_bits), Wb_bits)
    return {"qa": qa_bits, "qr": qr_bits, "y32": y32, "y_bf16": f32_to_bf16_bits(y32), "rstd": rstd}


def mla_prolog(x_bits, Wa_bits, gq_bits, eps, Wb_bits, Wkv_bits, gkv_bits, rstd=None, rstd_kv=None):
    """The chain plus the KV branch on one x (AT-10 page section 5)."""
    out = norm_proj_chain(x_bits, Wa_bits, gq_bits, eps, Wb_bits, rstd)
    kv = f32_to_bf16_bits(project_bf16(bf16_bits_to_f32(x_bits), Wkv_bits))
    n, rkv = rms_norm_rows(kv, gkv_bits, eps, rstd_kv)
    out.update(kv=kv, kv_out=f32_to_bf16_bits(n), rstd_kv=rkv)
    return out


def rmsnorm_linear_mxfp8(x_bits, gamma_bits, eps, qw, sw, rstd=None):
    """AT-10 with the MXFP8 mode: dict with q, x_scale, y32, y_bf16, rstd."""
    n, rstd = rms_norm_rows(x_bits, gamma_bits, eps, rstd)
    q, xs = mx_quant_rows(n)
    y32 = mx_scaled_mm(q, xs, qw, sw)
    return {"q": q, "x_scale": xs, "y32": y32, "y_bf16": f32_to_bf16_bits(y32), "rstd": rstd}


def preattn_qkv(x_bits, r_bits, gamma_bits, eps, W_bits, Hq, Hkv, D, gq_bits, gk_bits, head_eps,
                cos=None, sin=None, rstd=None, head_rstd=None):
    """Pre-attention block (AT-10 page section 6): dict with x_add, y_proj, y32
    (the projection in fp32), y, rstd, head_rstd."""
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


def add_rmsnorm_linear_bf16(x_bits, r_bits, gamma_bits, eps, W_bits, rstd=None):
    """Residual add, then AT-10 on the sum: (x_add bits, y32, y_bf16 bits, rstd)."""
    xa = add_residual(x_bits, r_bits)
    y32, ybf, rstd = rmsnorm_linear_bf16(xa, gamma_bits, eps, W_bits, rstd)
    return xa, y32, ybf, rstd


def add_rmsnorm_linear_fp32w(x_bits, r_bits, gamma_bits, eps, W, rstd=None):
    """Residual add, then the fp32-weight variant: (x_add bits, y32, rstd)."""
    xa = add_residual(x_bits, r_bits)
    y32, rstd = rmsnorm_linear_fp32w(xa, gamma_bits, eps, W, rstd)
    return xa, y32, rstd


def add_rmsnorm_linear_int8(x_bits, r_bits, gamma_bits, eps, Wq, w_scale, rstd=None):
    """Residual add, then AT-11 on the sum (dict, with "x_add")."""
    xa = add_residual(x_bits, r_bits)
    out = rmsnorm_linear_int8(xa, gamma_bits, eps, Wq, w_scale, rstd)
    out["x_add"] = xa
    return out
