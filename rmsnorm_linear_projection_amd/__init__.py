"""Fused RMSNorm -> Linear projection on MI355X (gfx950).

Thin Python binding of ``librnl.so`` (the C ABI declared in include/rnl.h).
It only marshals arguments: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.
There is no fallback: if the library is missing or cannot be loaded, every
call raises.

Entry points (same names as the C ABI):

* :func:`rmsnorm_linear_bf16` -- RMSNorm -> bf16 cast -> product with W[N,K]^T
  (fp32 weights: the normed rows stay fp32, the large-reduction split-K path);
* :func:`rmsnorm_linear_int8` -- RMSNorm -> per-token int8 quant -> int8 GEMM ->
  dequant;
* :func:`rmsnorm_linear_mxfp8` -- RMSNorm -> MX quantisation (E4M3, one E8M0 scale
  per 64 values) -> MXFP8 scaled GEMM;
* :func:`add_rmsnorm_linear_bf16`, :func:`add_rmsnorm_linear_int8` -- the same
  with the residual add in front (x_add = x + residual, also returned);
* :func:`preattn_qkv_bf16` -- (residual add ->) RMSNorm -> fused QKV projection ->
  per-head RMSNorm of the query and key heads (-> RoPE);
* :func:`mla_prolog_bf16` -- the chain plus the KV branch (kv = x W_kv^T -> RMSNorm),
  one pass over x for both first projections;
* :func:`norm_proj_chain` -- q_a = x W_a^T -> RMSNorm -> qr -> y = qr W_b^T.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "rmsnorm_linear_bf16",
    "rmsnorm_linear_bf16_noalloc",
    "noalloc_scratch_bytes",
    "stream_read",
    "clock_probe",
    "mfma_probe",
    "MFMA_PROBE_KINDS",
    "rmsnorm_linear_int8",
    "add_rmsnorm_linear_bf16",
    "add_rmsnorm_linear_int8",
    "norm_proj_chain",
    "mla_prolog_bf16",
    "preattn_qkv_bf16",
    "head_rms_norm_bf16",
    "rms_norm_bf16",
    "rms_norm_quant_int8",
    "rmsnorm_linear_mxfp8",
    "rms_norm_quant_mxfp8",
    "linear_mxfp8",
    "linear_bf16",
    "linear_heads_bf16",
    "linear_int8",
    "workspace_bytes",
    "load_library",
    "RnlError",
    "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librnl.so")

# codes from include/rnl.h
RNL_BF16, RNL_FP32, RNL_INT8, RNL_INT32 = 1, 2, 3, 4
_DTYPE_CODE = {torch.bfloat16: RNL_BF16, torch.float32: RNL_FP32, torch.int8: RNL_INT8, torch.int32: RNL_INT32}

_c_i64 = ctypes.c_int64
_c_p = ctypes.c_void_p


class RnlError(RuntimeError):
    """A non-zero status returned by the C ABI."""

    def __init__(self, status: int, detail: str):
        super().__init__(f"rnl status {status}: {detail}")
        self.status = status


_lib = None


def load_library() -> ctypes.CDLL:
    """Load librnl.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m rmsnorm_linear_projection_amd.build_lib` "
            "or __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    lib.rmsnorm_linear_bf16.argtypes = [_c_p, _c_p, ctypes.c_float, _c_p, ctypes.c_int, _c_p, ctypes.c_int,
                                        _c_p, _c_i64, _c_i64, _c_i64, _c_p, ctypes.c_size_t, _c_p]
    lib.rmsnorm_linear_bf16.restype = ctypes.c_int
    lib.rmsnorm_linear_bf16_workspace_bytes.argtypes = [_c_i64, _c_i64, _c_i64, ctypes.c_int, ctypes.c_int]
    lib.rmsnorm_linear_bf16_workspace_bytes.restype = ctypes.c_size_t
    lib.rmsnorm_linear_int8.argtypes = [_c_p, _c_p, ctypes.c_float, _c_p, _c_p, _c_p, ctypes.c_int, _c_p, _c_p,
                                        _c_p, _c_i64, _c_i64, _c_i64, _c_p, ctypes.c_size_t, _c_p]
    lib.rmsnorm_linear_int8.restype = ctypes.c_int
    lib.rmsnorm_linear_int8_workspace_bytes.argtypes = [_c_i64, _c_i64, _c_i64, ctypes.c_int]
    lib.rmsnorm_linear_int8_workspace_bytes.restype = ctypes.c_size_t
    lib.norm_proj_chain.argtypes = [_c_p, _c_p, _c_p, ctypes.c_float, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64,
                                    _c_i64, _c_i64, _c_i64, _c_p, ctypes.c_size_t, _c_p]
    lib.norm_proj_chain.restype = ctypes.c_int
    lib.norm_proj_chain_workspace_bytes.argtypes = [_c_i64, _c_i64, _c_i64, _c_i64]
    lib.norm_proj_chain_workspace_bytes.restype = ctypes.c_size_t
    lib.rms_norm_bf16.argtypes = [_c_p, _c_p, ctypes.c_float, _c_p, _c_p, _c_i64, _c_i64, _c_p]
    lib.rms_norm_bf16.restype = ctypes.c_int
    lib.rms_norm_quant_int8.argtypes = [_c_p, _c_p, ctypes.c_float, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_p]
    lib.rms_norm_quant_int8.restype = ctypes.c_int
    lib.linear_bf16.argtypes = [_c_p, _c_p, _c_p, ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_p]
    lib.linear_bf16.restype = ctypes.c_int
    lib.linear_heads_bf16.argtypes = [_c_p, _c_p, _c_p, _c_p, _c_p, ctypes.c_float, _c_p, _c_p, _c_p, _c_i64, _c_i64,
                                      _c_i64, _c_i64, _c_i64, _c_p]
    lib.linear_heads_bf16.restype = ctypes.c_int
    lib.linear_int8.argtypes = [_c_p, _c_p, _c_p, _c_p, _c_p, ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_p]
    lib.linear_int8.restype = ctypes.c_int
    lib.add_rmsnorm_linear_bf16.argtypes = [_c_p, _c_p, _c_p] + lib.rmsnorm_linear_bf16.argtypes[1:]
    lib.add_rmsnorm_linear_bf16.restype = ctypes.c_int
    lib.add_rmsnorm_linear_bf16_workspace_bytes.argtypes = lib.rmsnorm_linear_bf16_workspace_bytes.argtypes
    lib.add_rmsnorm_linear_bf16_workspace_bytes.restype = ctypes.c_size_t
    lib.add_rmsnorm_linear_int8.argtypes = [_c_p, _c_p, _c_p] + lib.rmsnorm_linear_int8.argtypes[1:]
    lib.add_rmsnorm_linear_int8.restype = ctypes.c_int
    lib.add_rmsnorm_linear_int8_workspace_bytes.argtypes = lib.rmsnorm_linear_int8_workspace_bytes.argtypes
    lib.add_rmsnorm_linear_int8_workspace_bytes.restype = ctypes.c_size_t
    lib.preattn_qkv_bf16.argtypes = [_c_p, _c_p, _c_p, _c_p, ctypes.c_float, _c_p, _c_p, _c_p, _c_p, _c_p,
                                     ctypes.c_float, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                     _c_p, ctypes.c_size_t, _c_p]
    lib.preattn_qkv_bf16.restype = ctypes.c_int
    lib.preattn_qkv_bf16_workspace_bytes.argtypes = [_c_i64] * 5
    lib.preattn_qkv_bf16_workspace_bytes.restype = ctypes.c_size_t
    lib.head_rms_norm_bf16.argtypes = [_c_p, _c_p, _c_p, ctypes.c_float, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64,
                                       _c_i64, _c_i64, _c_p]
    lib.head_rms_norm_bf16.restype = ctypes.c_int
    lib.mla_prolog_bf16.argtypes = [_c_p, _c_p, _c_p, _c_p, ctypes.c_float, _c_p, _c_p, _c_p, _c_p, _c_p, _c_p,
                                    _c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, ctypes.c_size_t, _c_p]
    lib.mla_prolog_bf16.restype = ctypes.c_int
    lib.mla_prolog_bf16_workspace_bytes.argtypes = [_c_i64] * 5
    lib.mla_prolog_bf16_workspace_bytes.restype = ctypes.c_size_t
    lib.rmsnorm_linear_mxfp8.argtypes = lib.rmsnorm_linear_int8.argtypes
    lib.rmsnorm_linear_mxfp8.restype = ctypes.c_int
    lib.rmsnorm_linear_mxfp8_workspace_bytes.argtypes = [_c_i64, _c_i64, _c_i64, ctypes.c_int]
    lib.rmsnorm_linear_mxfp8_workspace_bytes.restype = ctypes.c_size_t
    lib.rms_norm_quant_mxfp8.argtypes = [_c_p, _c_p, ctypes.c_float, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_p]
    lib.rms_norm_quant_mxfp8.restype = ctypes.c_int
    lib.linear_mxfp8.argtypes = [_c_p, _c_p, _c_p, _c_p, _c_p, ctypes.c_int, _c_i64, _c_i64, _c_i64, _c_p]
    lib.linear_mxfp8.restype = ctypes.c_int
    lib.rmsnorm_linear_bf16_noalloc.argtypes = [_c_p, _c_p, ctypes.c_float, _c_p, ctypes.c_int, _c_p, ctypes.c_int,
                                                _c_p, _c_i64, _c_i64, _c_i64, _c_p]
    lib.rmsnorm_linear_bf16_noalloc.restype = ctypes.c_int
    lib.rnl_noalloc_scratch_bytes.argtypes = []
    lib.rnl_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.rnl_clock_probe.argtypes = [_c_p, _c_i64, _c_i64, ctypes.c_int, _c_p]
    lib.rnl_clock_probe.restype = ctypes.c_int
    lib.rnl_stream_read.argtypes = [_c_p, ctypes.c_size_t, _c_p, ctypes.c_int, ctypes.c_int, _c_p]
    lib.rnl_stream_read.restype = ctypes.c_int
    lib.rnl_mfma_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _c_i64, _c_p, _c_p]
    lib.rnl_mfma_probe.restype = ctypes.c_int
    lib.rnl_status_str.argtypes = [ctypes.c_int]
    lib.rnl_status_str.restype = ctypes.c_char_p
    lib.rnl_last_error.argtypes = []
    lib.rnl_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(rc: int):
    if rc != 0:
        lib = load_library()
        raise RnlError(rc, f"{lib.rnl_status_str(rc).decode()}: {lib.rnl_last_error().decode()}")


def _dev_tensor(t, name, dtype=None, ndim=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D")


def _shape(cond: bool, what: str):
    if not cond:
        raise ValueError(what)


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _workspace(nbytes: int, dev, given):
    if nbytes == 0:
        return None, 0
    if given is not None:
        _dev_tensor(given, "workspace")
        return given, given.numel() * given.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=dev), nbytes


def workspace_bytes(kind: str, *shape, w_dtype=torch.bfloat16, out_dtype=torch.bfloat16) -> int:
    """Workspace a call needs: kind 'bf16', 'int8', 'add_bf16', 'add_int8' (T, K, N), 'chain' (T, K, R, N)
    'preattn' (T, K, Hq, Hkv, D) or 'mla' (T, K, R, Rkv, N)."""
    lib = load_library()
    if kind == "bf16":
        return int(lib.rmsnorm_linear_bf16_workspace_bytes(*shape, _DTYPE_CODE[w_dtype], _DTYPE_CODE[out_dtype]))
    if kind == "add_bf16":
        return int(lib.add_rmsnorm_linear_bf16_workspace_bytes(*shape, _DTYPE_CODE[w_dtype], _DTYPE_CODE[out_dtype]))
    if kind == "int8":
        return int(lib.rmsnorm_linear_int8_workspace_bytes(*shape, _DTYPE_CODE[out_dtype]))
    if kind == "mxfp8":
        return int(lib.rmsnorm_linear_mxfp8_workspace_bytes(*shape, _DTYPE_CODE[out_dtype]))
    if kind == "add_int8":
        return int(lib.add_rmsnorm_linear_int8_workspace_bytes(*shape, _DTYPE_CODE[out_dtype]))
    if kind == "chain":
        return int(lib.norm_proj_chain_workspace_bytes(*shape))
    if kind == "preattn":
        return int(lib.preattn_qkv_bf16_workspace_bytes(*shape))
    if kind == "mla":
        return int(lib.mla_prolog_bf16_workspace_bytes(*shape))
    raise ValueError(kind)


def _residual(x, residual, x_add_out):
    """Checks the residual-add operands; returns x_add_out (allocated if None)."""
    _dev_tensor(residual, "residual", torch.bfloat16, 2)
    _shape(tuple(residual.shape) == tuple(x.shape), "residual must have the shape of x")
    if x_add_out is None:
        x_add_out = torch.empty_like(x)
    _dev_tensor(x_add_out, "x_add_out", torch.bfloat16, 2)
    _shape(tuple(x_add_out.shape) == tuple(x.shape), "x_add_out must have the shape of x")
    return x_add_out


def _bf16_call(x, residual, x_add_out, gamma, eps, W, out_dtype, rstd_out, y, workspace):
    lib = load_library()
    _dev_tensor(x, "x", torch.bfloat16, 2)
    _dev_tensor(gamma, "gamma", torch.bfloat16, 1)
    _dev_tensor(W, "W", (torch.bfloat16, torch.float32), 2)
    _dev_tensor(rstd_out, "rstd_out", torch.float32)
    T, K = x.shape
    N = W.shape[0]
    _shape(W.shape[1] == K, "W must be [N, K]")
    _shape(gamma is None or gamma.numel() == K, "gamma must be [K]")
    _shape(rstd_out is None or rstd_out.numel() >= T, "rstd_out must hold T values")
    wcode = _DTYPE_CODE[W.dtype]
    ocode = _DTYPE_CODE[out_dtype]
    if y is None:
        y = torch.empty((T, N), dtype=out_dtype, device=x.device)
    _dev_tensor(y, "y", out_dtype)
    _shape(tuple(y.shape) == (T, N), "y must be [T, N]")
    with torch.cuda.device(x.device):
        query = lib.rmsnorm_linear_bf16_workspace_bytes if residual is None else \
            lib.add_rmsnorm_linear_bf16_workspace_bytes
        need = int(query(T, K, N, wcode, ocode))
        ws, ws_bytes = _workspace(need, x.device, workspace)
        tail = (_ptr(gamma), float(eps), _ptr(W), wcode, _ptr(y), ocode, _ptr(rstd_out), T, K, N, _ptr(ws),
                ws_bytes, _stream(x.device))
        if residual is None:
            rc = lib.rmsnorm_linear_bf16(_ptr(x), *tail)
        else:
            rc = lib.add_rmsnorm_linear_bf16(_ptr(x), _ptr(residual), _ptr(x_add_out), *tail)
    _check(rc)
    return y


def rmsnorm_linear_bf16(x, gamma, eps, W, out_dtype=torch.bfloat16, rstd_out=None, y=None, workspace=None):
    """y[T,N] = bf16(RMSNorm(x) * gamma) . W[N,K]^T -- AT-10.

    ``W`` bf16 [N, K], or fp32 [N, K] for the fp32-compute variant.  ``gamma``
    may be None.  ``rstd_out`` (fp32 [T]) receives the per-token rstd.
    """
    return _bf16_call(x, None, None, gamma, eps, W, out_dtype, rstd_out, y, workspace)


def rmsnorm_linear_bf16_noalloc(x, gamma, eps, W, y, rstd_out=None):
    """rmsnorm_linear_bf16 without a workspace: the library's own per-GPU scratch
    array serves instead, so the call allocates nothing (``y`` [T, N], bf16 or
    fp32, is required; its dtype selects the output type).  Sizes that need more
    scratch than ``noalloc_scratch_bytes()`` raise.  Calls that overlap on one GPU
    share that scratch and race."""
    lib = load_library()
    _dev_tensor(x, "x", torch.bfloat16, 2)
    _dev_tensor(gamma, "gamma", torch.bfloat16, 1)
    _dev_tensor(W, "W", (torch.bfloat16, torch.float32), 2)
    _dev_tensor(y, "y", (torch.bfloat16, torch.float32), 2)
    _dev_tensor(rstd_out, "rstd_out", torch.float32)
    T, K = x.shape
    N = W.shape[0]
    _shape(W.shape[1] == K, "W must be [N, K]")
    _shape(gamma is None or gamma.numel() == K, "gamma must be [K]")
    _shape(tuple(y.shape) == (T, N), "y must be [T, N]")
    _shape(rstd_out is None or rstd_out.numel() >= T, "rstd_out must hold T values")
    with torch.cuda.device(x.device):
        rc = lib.rmsnorm_linear_bf16_noalloc(_ptr(x), _ptr(gamma), float(eps), _ptr(W), _DTYPE_CODE[W.dtype], _ptr(y),
                                             _DTYPE_CODE[y.dtype], _ptr(rstd_out), T, K, N, _stream(x.device))
    _check(rc)
    return y


def stream_read(src, workgroups=1024, unroll=8, sink=None):
    """HBM streaming probe (not a step of the method): one read of every byte of
    the device tensor ``src`` (size a multiple of 16 bytes) by ``workgroups``
    workgroups with ``unroll`` loads in flight per lane; returns the int32 sink
    (one word per workgroup) it folds the data into."""
    lib = load_library()
    _dev_tensor(src, "src")
    nbytes = src.numel() * src.element_size()
    if sink is None:
        sink = torch.empty(workgroups, dtype=torch.int32, device=src.device)
    _dev_tensor(sink, "sink", torch.int32)
    _shape(sink.numel() >= workgroups, "sink must hold one word per workgroup")
    with torch.cuda.device(src.device):
        rc = lib.rnl_stream_read(_ptr(src), nbytes, _ptr(sink), int(workgroups), int(unroll), _stream(src.device))
    _check(rc)
    return sink


MFMA_PROBE_KINDS = {"bf16": (0, 16384), "int8": (1, 32768), "fp8": (2, 65536)}  # kind code, flop (op) per instruction


def mfma_probe(kind, workgroups=256, waves=4, iterations=4096, sink=None, stream=None):
    """MFMA rate probe (not a step of the method): ``workgroups`` x ``waves`` wavefronts
    each issue ``iterations`` x 8 matrix instructions of ``kind`` ("bf16", "int8" or
    "fp8", see MFMA_PROBE_KINDS) on register operands, on ``stream`` (torch's current
    stream by default); returns the int32 sink, one word per wavefront."""
    lib = load_library()
    code = MFMA_PROBE_KINDS[kind][0]
    dev = torch.device("cuda", torch.cuda.current_device())
    if sink is None:
        sink = torch.empty(workgroups * waves, dtype=torch.int32, device=dev)
    _dev_tensor(sink, "sink", torch.int32)
    _shape(sink.numel() >= workgroups * waves, "sink must hold one word per wavefront")
    st = ctypes.c_void_p((stream or torch.cuda.current_stream(dev)).cuda_stream)
    _check(lib.rnl_mfma_probe(code, int(workgroups), int(waves), int(iterations), _ptr(sink), st))
    return sink


def clock_probe(microseconds, delay_us=0, workgroups=8, out=None, stream=None):
    """Clock probe (not a step of the method): enqueue ``workgroups`` wavefronts that
    wait ``delay_us``, then spin for ``microseconds`` of real time, on ``stream``
    (torch's current stream by default); wavefront b writes [shader clocks, real-time
    ticks at 100 MHz] to out[b] (int64 [workgroups, 2], on the current device).  The
    shader clock in MHz is 100 * out[b, 0] / out[b, 1]."""
    lib = load_library()
    dev = torch.device("cuda", torch.cuda.current_device())
    if out is None:
        out = torch.zeros((workgroups, 2), dtype=torch.int64, device=dev)
    _dev_tensor(out, "out", torch.int64)
    _shape(out.numel() >= 2 * workgroups, "out must hold two words per workgroup")
    st = ctypes.c_void_p((stream or torch.cuda.current_stream(dev)).cuda_stream)
    _check(lib.rnl_clock_probe(_ptr(out), int(delay_us), int(microseconds), int(workgroups), st))
    return out


def noalloc_scratch_bytes() -> int:
    """Size of the per-GPU scratch array behind rmsnorm_linear_bf16_noalloc."""
    return int(load_library().rnl_noalloc_scratch_bytes())


def add_rmsnorm_linear_bf16(x, residual, gamma, eps, W, out_dtype=torch.bfloat16, rstd_out=None, y=None,
                            x_add_out=None, workspace=None):
    """x_add = bf16(x + residual), then rmsnorm_linear_bf16 on x_add (the
    pre-attention input norm).  Returns (y, x_add_out)."""
    x_add_out = _residual(x, residual, x_add_out)
    y = _bf16_call(x, residual, x_add_out, gamma, eps, W, out_dtype, rstd_out, y, workspace)
    return y, x_add_out


def _int8_call(x, residual, x_add_out, gamma, eps, Wq, w_scale, out_dtype, xq_out, x_scale_out, rstd_out, y,
               workspace):
    lib = load_library()
    _dev_tensor(x, "x", torch.bfloat16, 2)
    _dev_tensor(gamma, "gamma", torch.bfloat16, 1)
    _dev_tensor(Wq, "Wq", torch.int8, 2)
    _dev_tensor(w_scale, "w_scale", torch.float32, 1)
    _dev_tensor(xq_out, "xq_out", torch.int8)
    _dev_tensor(x_scale_out, "x_scale_out", torch.float32)
    _dev_tensor(rstd_out, "rstd_out", torch.float32)
    T, K = x.shape
    N = Wq.shape[0]
    _shape(Wq.shape[1] == K, "Wq must be [N, K]")
    _shape(w_scale.numel() == N, "w_scale must be [N]")
    _shape(gamma is None or gamma.numel() == K, "gamma must be [K]")
    _shape(xq_out is None or xq_out.numel() == T * K, "xq_out must be [T, K]")
    _shape(x_scale_out is None or x_scale_out.numel() >= T, "x_scale_out must hold T values")
    _shape(rstd_out is None or rstd_out.numel() >= T, "rstd_out must hold T values")
    ocode = _DTYPE_CODE[out_dtype]
    if y is None:
        y = torch.empty((T, N), dtype=out_dtype, device=x.device)
    _dev_tensor(y, "y", out_dtype)
    _shape(tuple(y.shape) == (T, N), "y must be [T, N]")
    with torch.cuda.device(x.device):
        query = lib.rmsnorm_linear_int8_workspace_bytes if residual is None else \
            lib.add_rmsnorm_linear_int8_workspace_bytes
        need = int(query(T, K, N, ocode))
        if xq_out is not None and x_scale_out is not None:
            need = 0
        ws, ws_bytes = _workspace(need, x.device, workspace)
        tail = (_ptr(gamma), float(eps), _ptr(Wq), _ptr(w_scale), _ptr(y), ocode, _ptr(xq_out), _ptr(x_scale_out),
                _ptr(rstd_out), T, K, N, _ptr(ws), ws_bytes, _stream(x.device))
        if residual is None:
            rc = lib.rmsnorm_linear_int8(_ptr(x), *tail)
        else:
            rc = lib.add_rmsnorm_linear_int8(_ptr(x), _ptr(residual), _ptr(x_add_out), *tail)
    _check(rc)
    return y


def rmsnorm_linear_int8(x, gamma, eps, Wq, w_scale, out_dtype=torch.bfloat16, xq_out=None, x_scale_out=None,
                        rstd_out=None, y=None, workspace=None):
    """AT-11: RMSNorm -> per-token symmetric int8 quant -> int8 x int8 -> int32 ->
    dequant with x_scale and w_scale.  ``out_dtype`` torch.int32 returns the raw
    accumulators."""
    return _int8_call(x, None, None, gamma, eps, Wq, w_scale, out_dtype, xq_out, x_scale_out, rstd_out, y,
                      workspace)


def add_rmsnorm_linear_int8(x, residual, gamma, eps, Wq, w_scale, out_dtype=torch.bfloat16, xq_out=None,
                            x_scale_out=None, rstd_out=None, y=None, x_add_out=None, workspace=None):
    """x_add = bf16(x + residual), then rmsnorm_linear_int8 on x_add.  Returns
    (y, x_add_out)."""
    x_add_out = _residual(x, residual, x_add_out)
    y = _int8_call(x, residual, x_add_out, gamma, eps, Wq, w_scale, out_dtype, xq_out, x_scale_out, rstd_out, y,
                   workspace)
    return y, x_add_out


def norm_proj_chain(x, W_a, gamma, eps, W_b, qr_out=None, y=None, rstd_out=None, qa_out=None, workspace=None):
    """q_a_proj -> RMSNorm -> q_b_proj (MLA low-rank query).  Returns (y, qr_out).
    ``qa_out`` (bf16 [T, R]) receives q_a, the rows the norm reads."""
    lib = load_library()
    _dev_tensor(x, "x", torch.bfloat16, 2)
    _dev_tensor(W_a, "W_a", torch.bfloat16, 2)
    _dev_tensor(gamma, "gamma", torch.bfloat16, 1)
    _dev_tensor(W_b, "W_b", torch.bfloat16, 2)
    _dev_tensor(rstd_out, "rstd_out", torch.float32)
    T, K = x.shape
    R = W_a.shape[0]
    N = W_b.shape[0]
    _shape(W_a.shape[1] == K, "W_a must be [R, K]")
    _shape(W_b.shape[1] == R, "W_b must be [N, R]")
    _shape(gamma is None or gamma.numel() == R, "gamma must be [R]")
    _shape(rstd_out is None or rstd_out.numel() >= T, "rstd_out must hold T values")
    if qr_out is None:
        qr_out = torch.empty((T, R), dtype=torch.bfloat16, device=x.device)
    if y is None:
        y = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    _dev_tensor(qr_out, "qr_out", torch.bfloat16)
    _dev_tensor(y, "y", torch.bfloat16)
    _dev_tensor(qa_out, "qa_out", torch.bfloat16)
    _shape(tuple(qr_out.shape) == (T, R), "qr_out must be [T, R]")
    _shape(tuple(y.shape) == (T, N), "y must be [T, N]")
    _shape(qa_out is None or tuple(qa_out.shape) == (T, R), "qa_out must be [T, R]")
    with torch.cuda.device(x.device):
        need = int(lib.norm_proj_chain_workspace_bytes(T, K, R, N))
        ws, ws_bytes = _workspace(need, x.device, workspace)
        rc = lib.norm_proj_chain(_ptr(x), _ptr(W_a), _ptr(gamma), float(eps), _ptr(W_b), _ptr(qr_out), _ptr(y),
                                 _ptr(rstd_out), _ptr(qa_out), T, K, R, N, _ptr(ws), ws_bytes, _stream(x.device))
    _check(rc)
    return y, qr_out


def rmsnorm_linear_mxfp8(x, gamma, eps, Wq, w_scale, out_dtype=torch.bfloat16, xq_out=None, x_scale_out=None,
                         rstd_out=None, y=None, workspace=None):
    """AT-10 with AT-09's MXFP8 mode: RMSNorm -> MX quantisation of the normed rows
    (E4M3 codes, one E8M0 scale per 64 values) -> scaled product with Wq [N, K]
    (uint8 E4M3) and w_scale [N, K/64] (uint8 E8M0), fp32 accumulation."""
    lib = load_library()
    _dev_tensor(x, "x", torch.bfloat16, 2)
    _dev_tensor(gamma, "gamma", torch.bfloat16, 1)
    _dev_tensor(Wq, "Wq", torch.uint8, 2)
    _dev_tensor(w_scale, "w_scale", torch.uint8, 2)
    _dev_tensor(xq_out, "xq_out", torch.uint8)
    _dev_tensor(x_scale_out, "x_scale_out", torch.uint8)
    _dev_tensor(rstd_out, "rstd_out", torch.float32)
    T, K = x.shape
    N = Wq.shape[0]
    _shape(Wq.shape[1] == K, "Wq must be [N, K]")
    _shape(K % 64 == 0 and tuple(w_scale.shape) == (N, K // 64), "w_scale must be [N, K/64]")
    _shape(gamma is None or gamma.numel() == K, "gamma must be [K]")
    _shape(xq_out is None or xq_out.numel() == T * K, "xq_out must be [T, K]")
    _shape(x_scale_out is None or x_scale_out.numel() == T * (K // 64), "x_scale_out must be [T, K/64]")
    _shape(rstd_out is None or rstd_out.numel() >= T, "rstd_out must hold T values")
    ocode = _DTYPE_CODE[out_dtype]
    if y is None:
        y = torch.empty((T, N), dtype=out_dtype, device=x.device)
    _dev_tensor(y, "y", out_dtype)
    _shape(tuple(y.shape) == (T, N), "y must be [T, N]")
    with torch.cuda.device(x.device):
        need = int(lib.rmsnorm_linear_mxfp8_workspace_bytes(T, K, N, ocode))
        if xq_out is not None and x_scale_out is not None:
            need = 0
        ws, ws_bytes = _workspace(need, x.device, workspace)
        rc = lib.rmsnorm_linear_mxfp8(_ptr(x), _ptr(gamma), float(eps), _ptr(Wq), _ptr(w_scale), _ptr(y), ocode,
                                      _ptr(xq_out), _ptr(x_scale_out), _ptr(rstd_out), T, K, N, _ptr(ws), ws_bytes,
                                      _stream(x.device))
    _check(rc)
    return y


def rms_norm_quant_mxfp8(x, gamma, eps, xq=None, x_scale=None, rstd_out=None):
    """RMSNorm + MX quantisation: returns (xq [T, K] E4M3 bytes, x_scale [T, K/64] E8M0 bytes)."""
    lib = load_library()
    _dev_tensor(x, "x", torch.bfloat16, 2)
    _dev_tensor(gamma, "gamma", torch.bfloat16, 1)
    _dev_tensor(rstd_out, "rstd_out", torch.float32)
    T, K = x.shape
    _shape(K % 64 == 0, "K must be a multiple of 64")
    xq = torch.empty((T, K), dtype=torch.uint8, device=x.device) if xq is None else xq
    x_scale = torch.empty((T, K // 64), dtype=torch.uint8, device=x.device) if x_scale is None else x_scale
    _dev_tensor(xq, "xq", torch.uint8)
    _dev_tensor(x_scale, "x_scale", torch.uint8)
    _shape(xq.numel() == T * K and x_scale.numel() == T * (K // 64), "xq / x_scale sizes")
    with torch.cuda.device(x.device):
        rc = lib.rms_norm_quant_mxfp8(_ptr(x), _ptr(gamma), float(eps), _ptr(xq), _ptr(x_scale), _ptr(rstd_out), T,
                                      K, _stream(x.device))
    _check(rc)
    return xq, x_scale


def linear_mxfp8(xq, x_scale, Wq, w_scale, out_dtype=torch.bfloat16, y=None):
    """AT-09 MXFP8 mode on given MX operands: y [M, N] bf16 or fp32."""
    lib = load_library()
    for t, n in ((xq, "xq"), (x_scale, "x_scale"), (Wq, "Wq"), (w_scale, "w_scale")):
        _dev_tensor(t, n, torch.uint8, 2)
    M, K = xq.shape
    N = Wq.shape[0]
    _shape(Wq.shape[1] == K and K % 64 == 0, "Wq must be [N, K], K a multiple of 64")
    _shape(tuple(x_scale.shape) == (M, K // 64) and tuple(w_scale.shape) == (N, K // 64), "scales must be [*, K/64]")
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=xq.device)
    _dev_tensor(y, "y", out_dtype)
    _shape(tuple(y.shape) == (M, N), "y must be [M, N]")
    with torch.cuda.device(xq.device):
        rc = lib.linear_mxfp8(_ptr(xq), _ptr(x_scale), _ptr(Wq), _ptr(w_scale), _ptr(y), _DTYPE_CODE[out_dtype], M, K,
                              N, _stream(xq.device))
    _check(rc)
    return y


def mla_prolog_bf16(x, W_akv, R, gamma_cq, gamma_ckv, eps, W_b, qr_out=None, kv_out=None, y=None, rstd_q_out=None,
                    rstd_kv_out=None, qakv_out=None, workspace=None):
    """MLA prolog query chain + KV branch (AT-10 page section 5).  W_akv stacks the
    query down-projection (rows [0, R)) and the KV projection (rows [R, R + Rkv)).
    ``qakv_out`` (bf16 [T, R + Rkv]) receives [q_a | kv], the rows the norms read.
    Returns (y [T, N], qr [T, R], kv [T, Rkv])."""
    lib = load_library()
    for t, n in ((x, "x"), (W_akv, "W_akv"), (W_b, "W_b")):
        _dev_tensor(t, n, torch.bfloat16, 2)
    _dev_tensor(gamma_cq, "gamma_cq", torch.bfloat16, 1)
    _dev_tensor(gamma_ckv, "gamma_ckv", torch.bfloat16, 1)
    _dev_tensor(rstd_q_out, "rstd_q_out", torch.float32)
    _dev_tensor(rstd_kv_out, "rstd_kv_out", torch.float32)
    T, K = x.shape
    Rkv = W_akv.shape[0] - R
    N = W_b.shape[0]
    _shape(W_akv.shape[1] == K and Rkv > 0, "W_akv must be [R + Rkv, K] with Rkv > 0")
    _shape(W_b.shape[1] == R, "W_b must be [N, R]")
    _shape(gamma_cq is None or gamma_cq.numel() == R, "gamma_cq must be [R]")
    _shape(gamma_ckv is None or gamma_ckv.numel() == Rkv, "gamma_ckv must be [Rkv]")
    _shape(rstd_q_out is None or rstd_q_out.numel() >= T, "rstd_q_out must hold T values")
    _shape(rstd_kv_out is None or rstd_kv_out.numel() >= T, "rstd_kv_out must hold T values")
    outs = []
    for t, shp, n in ((qr_out, (T, R), "qr_out"), (kv_out, (T, Rkv), "kv_out"), (y, (T, N), "y")):
        if t is None:
            t = torch.empty(shp, dtype=torch.bfloat16, device=x.device)
        _dev_tensor(t, n, torch.bfloat16)
        _shape(tuple(t.shape) == shp, f"{n} must be {list(shp)}")
        outs.append(t)
    qr_out, kv_out, y = outs
    _dev_tensor(qakv_out, "qakv_out", torch.bfloat16)
    _shape(qakv_out is None or tuple(qakv_out.shape) == (T, R + Rkv), "qakv_out must be [T, R + Rkv]")
    with torch.cuda.device(x.device):
        need = int(lib.mla_prolog_bf16_workspace_bytes(T, K, R, Rkv, N))
        ws, ws_bytes = _workspace(need, x.device, workspace)
        rc = lib.mla_prolog_bf16(_ptr(x), _ptr(W_akv), _ptr(gamma_cq), _ptr(gamma_ckv), float(eps), _ptr(W_b),
                                 _ptr(qr_out), _ptr(kv_out), _ptr(y), _ptr(rstd_q_out), _ptr(rstd_kv_out),
                                 _ptr(qakv_out), T, K, R, Rkv, N, _ptr(ws), ws_bytes, _stream(x.device))
    _check(rc)
    return y, qr_out, kv_out


def _rope_tables(cos, sin, T, D):
    _dev_tensor(cos, "cos", torch.float32, 2)
    _dev_tensor(sin, "sin", torch.float32, 2)
    _shape((cos is None) == (sin is None), "cos and sin go together")
    _shape(cos is None or (tuple(cos.shape) == (T, D // 2) and tuple(sin.shape) == (T, D // 2)),
           "cos and sin must be [T, D/2]")


def preattn_qkv_bf16(x, gamma, eps, W, Hq, Hkv, D, gamma_q=None, gamma_k=None, head_eps=1e-6, cos=None, sin=None,
                     residual=None, x_add_out=None, y=None, rstd_out=None, head_rstd_out=None, workspace=None):
    """Pre-attention block (AT-10 page section 6): optional residual add, RMSNorm,
    fused QKV projection with W [(Hq + 2 Hkv) D, K], per-head RMSNorm of the query
    (gamma_q) and key (gamma_k) heads, RoPE with cos/sin [T, D/2] when given.
    Returns (y [T, (Hq + 2 Hkv) D] with columns Q | K | V, x_add_out or None)."""
    lib = load_library()
    _dev_tensor(x, "x", torch.bfloat16, 2)
    _dev_tensor(gamma, "gamma", torch.bfloat16, 1)
    _dev_tensor(W, "W", torch.bfloat16, 2)
    _dev_tensor(gamma_q, "gamma_q", torch.bfloat16, 1)
    _dev_tensor(gamma_k, "gamma_k", torch.bfloat16, 1)
    _dev_tensor(rstd_out, "rstd_out", torch.float32)
    _dev_tensor(head_rstd_out, "head_rstd_out", torch.float32)
    T, K = x.shape
    N = (Hq + 2 * Hkv) * D
    _shape(tuple(W.shape) == (N, K), "W must be [(Hq + 2 Hkv) D, K]")
    _shape(gamma is None or gamma.numel() == K, "gamma must be [K]")
    _shape(gamma_q is None or gamma_q.numel() == D, "gamma_q must be [D]")
    _shape(gamma_k is None or gamma_k.numel() == D, "gamma_k must be [D]")
    _shape(rstd_out is None or rstd_out.numel() >= T, "rstd_out must hold T values")
    _shape(head_rstd_out is None or head_rstd_out.numel() >= T * (Hq + Hkv), "head_rstd_out must be [T, Hq + Hkv]")
    _rope_tables(cos, sin, T, D)
    if residual is not None:
        x_add_out = _residual(x, residual, x_add_out)
    if y is None:
        y = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    _dev_tensor(y, "y", torch.bfloat16)
    _shape(tuple(y.shape) == (T, N), "y must be [T, (Hq + 2 Hkv) D]")
    with torch.cuda.device(x.device):
        need = int(lib.preattn_qkv_bf16_workspace_bytes(T, K, Hq, Hkv, D))
        ws, ws_bytes = _workspace(need, x.device, workspace)
        rc = lib.preattn_qkv_bf16(_ptr(x), _ptr(residual), _ptr(x_add_out if residual is not None else None),
                                  _ptr(gamma), float(eps), _ptr(W), _ptr(y), _ptr(rstd_out), _ptr(gamma_q),
                                  _ptr(gamma_k), float(head_eps), _ptr(cos), _ptr(sin), _ptr(head_rstd_out), T, K,
                                  Hq, Hkv, D, _ptr(ws), ws_bytes, _stream(x.device))
    _check(rc)
    return y, (x_add_out if residual is not None else None)


def head_rms_norm_bf16(y, col0, H, D, gamma=None, eps=1e-6, cos=None, sin=None, out=None, rstd_out=None):
    """Per-head RMSNorm (+ RoPE with cos/sin [T, D/2]) of the H heads of D columns
    from column col0 of y [T, ld].  Writes into ``out`` (same shape as y), or into
    y itself when ``out`` is None; returns the tensor written."""
    lib = load_library()
    _dev_tensor(y, "y", torch.bfloat16, 2)
    _dev_tensor(gamma, "gamma", torch.bfloat16, 1)
    _dev_tensor(rstd_out, "rstd_out", torch.float32)
    T, ld = y.shape
    _shape(gamma is None or gamma.numel() == D, "gamma must be [D]")
    _shape(rstd_out is None or rstd_out.numel() >= T * H, "rstd_out must be [T, H]")
    _rope_tables(cos, sin, T, D)
    if out is None:
        out = y
    _dev_tensor(out, "out", torch.bfloat16, 2)
    _shape(tuple(out.shape) == (T, ld), "out must have the shape of y")
    with torch.cuda.device(y.device):
        rc = lib.head_rms_norm_bf16(_ptr(y), _ptr(out), _ptr(gamma), float(eps), _ptr(cos), _ptr(sin),
                                    _ptr(rstd_out), T, ld, col0, H, D, _stream(y.device))
    _check(rc)
    return out


def rms_norm_bf16(x, gamma, eps, y=None, rstd_out=None):
    """AT-03 RMSNorm: y = bf16(fl(fl(x * rstd) * gamma)); returns y [T, K] bf16."""
    lib = load_library()
    _dev_tensor(x, "x", torch.bfloat16, 2)
    _dev_tensor(gamma, "gamma", torch.bfloat16, 1)
    _dev_tensor(rstd_out, "rstd_out", torch.float32)
    T, K = x.shape
    _shape(gamma is None or gamma.numel() == K, "gamma must be [K]")
    _shape(rstd_out is None or rstd_out.numel() >= T, "rstd_out must hold T values")
    if y is None:
        y = torch.empty_like(x)
    _dev_tensor(y, "y", torch.bfloat16)
    _shape(tuple(y.shape) == (T, K), "y must be [T, K]")
    with torch.cuda.device(x.device):
        rc = lib.rms_norm_bf16(_ptr(x), _ptr(gamma), float(eps), _ptr(y), _ptr(rstd_out), T, K, _stream(x.device))
    _check(rc)
    return y


def rms_norm_quant_int8(x, gamma, eps, xq=None, x_scale=None, rstd_out=None):
    """AT-03 + AT-05: per-token symmetric int8 quant of the normed rows.
    Returns (xq [T, K] int8, x_scale [T] fp32)."""
    lib = load_library()
    _dev_tensor(x, "x", torch.bfloat16, 2)
    _dev_tensor(gamma, "gamma", torch.bfloat16, 1)
    _dev_tensor(rstd_out, "rstd_out", torch.float32)
    T, K = x.shape
    _shape(gamma is None or gamma.numel() == K, "gamma must be [K]")
    _shape(rstd_out is None or rstd_out.numel() >= T, "rstd_out must hold T values")
    if xq is None:
        xq = torch.empty((T, K), dtype=torch.int8, device=x.device)
    if x_scale is None:
        x_scale = torch.empty(T, dtype=torch.float32, device=x.device)
    _dev_tensor(xq, "xq", torch.int8)
    _dev_tensor(x_scale, "x_scale", torch.float32)
    _shape(xq.numel() == T * K and x_scale.numel() >= T, "xq must be [T, K] and x_scale [T]")
    with torch.cuda.device(x.device):
        rc = lib.rms_norm_quant_int8(_ptr(x), _ptr(gamma), float(eps), _ptr(xq), _ptr(x_scale), _ptr(rstd_out),
                                     T, K, _stream(x.device))
    _check(rc)
    return xq, x_scale


def linear_bf16(a, W, out_dtype=torch.bfloat16, y=None):
    """AT-09 BF16 mode: y[M, N] = a[M, K] . W[N, K]^T, fp32 accumulation."""
    lib = load_library()
    _dev_tensor(a, "a", torch.bfloat16, 2)
    _dev_tensor(W, "W", torch.bfloat16, 2)
    M, K = a.shape
    N = W.shape[0]
    _shape(W.shape[1] == K, "W must be [N, K]")
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=a.device)
    _dev_tensor(y, "y", out_dtype)
    _shape(tuple(y.shape) == (M, N), "y must be [M, N]")
    with torch.cuda.device(a.device):
        rc = lib.linear_bf16(_ptr(a), _ptr(W), _ptr(y), _DTYPE_CODE[out_dtype], M, K, N, _stream(a.device))
    _check(rc)
    return y


def linear_heads_bf16(a, W, Hq, Hkv, D, gamma_q=None, gamma_k=None, head_eps=1e-6, cos=None, sin=None, y=None,
                      head_rstd_out=None):
    """y = bf16(a . W^T) with W [(Hq + 2 Hkv) D, K], then the per-head stage of
    :func:`preattn_qkv_bf16` on the query and key heads; returns y."""
    lib = load_library()
    _dev_tensor(a, "a", torch.bfloat16, 2)
    _dev_tensor(W, "W", torch.bfloat16, 2)
    _dev_tensor(gamma_q, "gamma_q", torch.bfloat16, 1)
    _dev_tensor(gamma_k, "gamma_k", torch.bfloat16, 1)
    _dev_tensor(head_rstd_out, "head_rstd_out", torch.float32)
    M, K = a.shape
    N = (Hq + 2 * Hkv) * D
    _shape(tuple(W.shape) == (N, K), "W must be [(Hq + 2 Hkv) D, K]")
    _shape(gamma_q is None or gamma_q.numel() == D, "gamma_q must be [D]")
    _shape(gamma_k is None or gamma_k.numel() == D, "gamma_k must be [D]")
    _shape(head_rstd_out is None or head_rstd_out.numel() >= M * (Hq + Hkv), "head_rstd_out must be [M, Hq + Hkv]")
    _rope_tables(cos, sin, M, D)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _dev_tensor(y, "y", torch.bfloat16)
    _shape(tuple(y.shape) == (M, N), "y must be [M, (Hq + 2 Hkv) D]")
    with torch.cuda.device(a.device):
        rc = lib.linear_heads_bf16(_ptr(a), _ptr(W), _ptr(y), _ptr(gamma_q), _ptr(gamma_k), float(head_eps), _ptr(cos),
                                   _ptr(sin), _ptr(head_rstd_out), M, K, Hq, Hkv, D, _stream(a.device))
    _check(rc)
    return y


def linear_int8(xq, x_scale, Wq, w_scale, out_dtype=torch.bfloat16, y=None):
    """AT-09 INT8 W8A8 mode + AT-06 dequant (out_dtype torch.int32: raw accumulators)."""
    lib = load_library()
    _dev_tensor(xq, "xq", torch.int8, 2)
    _dev_tensor(Wq, "Wq", torch.int8, 2)
    _dev_tensor(x_scale, "x_scale", torch.float32)
    _dev_tensor(w_scale, "w_scale", torch.float32)
    M, K = xq.shape
    N = Wq.shape[0]
    _shape(Wq.shape[1] == K, "Wq must be [N, K]")
    _shape(x_scale is None or x_scale.numel() >= M, "x_scale must be [M]")
    _shape(w_scale is None or w_scale.numel() >= N, "w_scale must be [N]")
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype, device=xq.device)
    _dev_tensor(y, "y", out_dtype)
    _shape(tuple(y.shape) == (M, N), "y must be [M, N]")
    with torch.cuda.device(xq.device):
        rc = lib.linear_int8(_ptr(xq), _ptr(x_scale), _ptr(Wq), _ptr(w_scale), _ptr(y), _DTYPE_CODE[out_dtype],
                             M, K, N, _stream(xq.device))
    _check(rc)
    return y
