"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/rnl.h declares, and rejects invalid arguments before any HIP call
(validation is host code that returns before touching the device)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import rmsnorm_linear_projection_amd as rnl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rnl.h")

NULL = None
FAKE = ctypes.c_void_p(0x10000)  # 16- and 256-byte aligned, never dereferenced
ODD = ctypes.c_void_p(0x10002)  # misaligned


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"RNL_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def header_define(name):
    m = re.search(rf"#define\s+{name}\s+\(?(-?\d+)\)?", open(HEADER).read())
    return int(m.group(1))


@pytest.fixture(scope="module")
def lib():
    return rnl.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) >= {"rmsnorm_linear_bf16", "rmsnorm_linear_int8", "norm_proj_chain",
                          "rnl_status_str", "rnl_last_error"}
    for n in names:
        assert hasattr(lib, n), n


def test_python_codes_match_header():
    for name, val in (("RNL_BF16", rnl.RNL_BF16), ("RNL_FP32", rnl.RNL_FP32),
                      ("RNL_INT8", rnl.RNL_INT8), ("RNL_INT32", rnl.RNL_INT32)):
        assert header_define(name) == val


def test_status_strings(lib):
    for code in range(0, -8, -1):
        s = lib.rnl_status_str(code).decode()
        assert s and s != "unknown status"
    assert lib.rnl_status_str(-99).decode() == "unknown status"


E = {n: header_define(n) for n in ("RNL_ERR_NULL", "RNL_ERR_SHAPE", "RNL_ERR_DTYPE", "RNL_ERR_ARG",
                                   "RNL_ERR_ALIGN", "RNL_ERR_WORKSPACE")}


def bf16_call(lib, x=FAKE, g=NULL, eps=1e-6, W=FAKE, wd=1, y=FAKE, od=1, rstd=NULL, T=4, K=64, N=8,
              ws=FAKE, wsb=1 << 30):
    return lib.rmsnorm_linear_bf16(x, g, eps, W, wd, y, od, rstd, T, K, N, ws, wsb, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(x=NULL), "RNL_ERR_NULL"),
    (dict(W=NULL), "RNL_ERR_NULL"),
    (dict(y=NULL), "RNL_ERR_NULL"),
    (dict(T=0), "RNL_ERR_SHAPE"),
    (dict(N=-1), "RNL_ERR_SHAPE"),
    (dict(K=12), "RNL_ERR_SHAPE"),
    (dict(K=(1 << 20) + 8), "RNL_ERR_SHAPE"),
    (dict(T=(1 << 24) + 1), "RNL_ERR_SHAPE"),
    (dict(T=1 << 24), "RNL_ERR_SHAPE"),  # T < 2^24: one 256-thread workgroup per row must fit a 32-bit grid axis
    (dict(wd=2, N=(1 << 20) + 1), "RNL_ERR_SHAPE"),  # fp32 weights: N <= 2^20
    (dict(wd=3), "RNL_ERR_DTYPE"),
    (dict(od=4), "RNL_ERR_DTYPE"),
    (dict(eps=-1.0), "RNL_ERR_ARG"),
    (dict(eps=float("nan")), "RNL_ERR_ARG"),
    (dict(eps=float("inf")), "RNL_ERR_ARG"),
    (dict(x=ODD), "RNL_ERR_ALIGN"),
    (dict(g=ODD), "RNL_ERR_ALIGN"),
    (dict(rstd=ctypes.c_void_p(0x10001)), "RNL_ERR_ALIGN"),
    (dict(T=64, ws=NULL), "RNL_ERR_WORKSPACE"),
    (dict(T=64, wsb=100), "RNL_ERR_WORKSPACE"),
    (dict(wd=2, wsb=10), "RNL_ERR_WORKSPACE"),
])
def test_bf16_validation(lib, kw, code):
    assert bf16_call(lib, **kw) == E[code]
    assert lib.rnl_last_error().decode() != ""


def test_workspace_queries(lib):
    # the bf16 path keeps the normed activations in the workspace
    assert lib.rmsnorm_linear_bf16_workspace_bytes(16, 4096, 6144, 1, 1) >= 16 * 4096 * 2
    assert lib.rmsnorm_linear_bf16_workspace_bytes(17, 4096, 6144, 1, 1) >= 17 * 4096 * 2
    assert lib.rmsnorm_linear_bf16_workspace_bytes(4096, 4096, 6144, 1, 1) >= 4096 * 4096 * 2
    assert lib.rmsnorm_linear_bf16_workspace_bytes(512, 28672, 24, 2, 2) > 512 * 24 * 4
    assert lib.rmsnorm_linear_int8_workspace_bytes(2048, 4096, 4096, 1) >= 2048 * 4096 + 2048 * 4
    assert lib.norm_proj_chain_workspace_bytes(1024, 7168, 1536, 24576) >= 1024 * 1536 * 2
    assert lib.rmsnorm_linear_bf16_workspace_bytes(0, 4096, 6144, 1, 1) == 0


def test_forced_variant_changes_workspace(lib, monkeypatch):
    # few tokens: the chain's first projection is not split; the tiled GEMM splits its K
    small = lib.norm_proj_chain_workspace_bytes(4, 7168, 1536, 24576)
    assert small == 4 * 1536 * 2 + (-(4 * 1536 * 2) % 256)
    monkeypatch.setenv("RNL_VARIANT", "gemm")
    assert lib.norm_proj_chain_workspace_bytes(4, 7168, 1536, 24576) > small


def add_bf16_call(lib, x=FAKE, r=ctypes.c_void_p(0x20000), xa=ctypes.c_void_p(0x30000), g=NULL, eps=1e-6, W=FAKE,
                  wd=1, y=FAKE, od=1, rstd=NULL, T=4, K=64, N=8, ws=FAKE, wsb=1 << 30):
    return lib.add_rmsnorm_linear_bf16(x, r, xa, g, eps, W, wd, y, od, rstd, T, K, N, ws, wsb, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(r=NULL), "RNL_ERR_NULL"),
    (dict(xa=NULL), "RNL_ERR_NULL"),
    (dict(x=NULL), "RNL_ERR_NULL"),
    (dict(r=ctypes.c_void_p(0x20008)), "RNL_ERR_ALIGN"),
    (dict(xa=ctypes.c_void_p(0x30004)), "RNL_ERR_ALIGN"),
    (dict(xa=FAKE), "RNL_ERR_ARG"),                      # x_add_out is x
    (dict(xa=ctypes.c_void_p(0x20000 + 496)), "RNL_ERR_ARG"),  # overlaps the residual's last row
    (dict(wd=2, xa=ctypes.c_void_p(0x20000)), "RNL_ERR_ARG"),
    (dict(K=12), "RNL_ERR_SHAPE"),
    (dict(T=64, ws=NULL), "RNL_ERR_WORKSPACE"),
])
def test_add_bf16_validation(lib, kw, code):
    assert add_bf16_call(lib, **kw) == E[code]


def test_add_bf16_accepts_adjacent_buffers(lib):
    # x_add_out right after the residual's last byte passes the overlap check; the call then
    # fails only on the missing workspace, which is checked after it
    assert add_bf16_call(lib, xa=ctypes.c_void_p(0x20000 + 64 * 64 * 2 - 16), T=64, ws=NULL) == E["RNL_ERR_ARG"]
    assert add_bf16_call(lib, xa=ctypes.c_void_p(0x20000 + 64 * 64 * 2), T=64, ws=NULL) == E["RNL_ERR_WORKSPACE"]


def test_add_workspace_queries_match(lib):
    for T, K, N, wd in ((16, 4096, 6144, 1), (4096, 4096, 6144, 1), (512, 28672, 24, 2)):
        assert lib.add_rmsnorm_linear_bf16_workspace_bytes(T, K, N, wd, 1) == \
            lib.rmsnorm_linear_bf16_workspace_bytes(T, K, N, wd, 1)
    assert lib.add_rmsnorm_linear_int8_workspace_bytes(2048, 4096, 4096, 1) == \
        lib.rmsnorm_linear_int8_workspace_bytes(2048, 4096, 4096, 1)


def int8_call(lib, x=FAKE, g=NULL, eps=1e-6, Wq=FAKE, ws=FAKE, y=FAKE, od=1, xq=NULL, xs=NULL, rstd=NULL,
              T=4, K=64, N=8, wsp=FAKE, wsb=1 << 30):
    return lib.rmsnorm_linear_int8(x, g, eps, Wq, ws, y, od, xq, xs, rstd, T, K, N, wsp, wsb, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(Wq=NULL), "RNL_ERR_NULL"),
    (dict(ws=NULL), "RNL_ERR_NULL"),
    (dict(K=24), "RNL_ERR_SHAPE"),  # int8 needs K % 16 == 0
    (dict(K=133152), "RNL_ERR_SHAPE"),
    (dict(od=3), "RNL_ERR_DTYPE"),
    (dict(xq=ODD), "RNL_ERR_ALIGN"),
    (dict(wsp=NULL), "RNL_ERR_WORKSPACE"),
    (dict(wsb=16), "RNL_ERR_WORKSPACE"),
])
def test_int8_validation(lib, kw, code):
    assert int8_call(lib, **kw) == E[code]


def add_int8_call(lib, x=FAKE, r=ctypes.c_void_p(0x20000), xa=ctypes.c_void_p(0x30000), g=NULL, eps=1e-6,
                  Wq=FAKE, ws=FAKE, y=FAKE, od=1, xq=NULL, xs=NULL, rstd=NULL, T=4, K=64, N=8, wsp=FAKE,
                  wsb=1 << 30):
    return lib.add_rmsnorm_linear_int8(x, r, xa, g, eps, Wq, ws, y, od, xq, xs, rstd, T, K, N, wsp, wsb, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(r=NULL), "RNL_ERR_NULL"),
    (dict(xa=NULL), "RNL_ERR_NULL"),
    (dict(Wq=NULL), "RNL_ERR_NULL"),
    (dict(xa=ctypes.c_void_p(0x20000)), "RNL_ERR_ARG"),
    (dict(K=24), "RNL_ERR_SHAPE"),
    (dict(wsp=NULL), "RNL_ERR_WORKSPACE"),
])
def test_add_int8_validation(lib, kw, code):
    assert add_int8_call(lib, **kw) == E[code]


def preattn_call(lib, x=FAKE, r=NULL, xa=NULL, g=NULL, eps=1e-6, W=FAKE, y=FAKE, rstd=NULL, gq=NULL, gk=NULL,
                 heps=1e-6, cos=NULL, sin=NULL, hrstd=NULL, T=4, K=64, Hq=4, Hkv=2, D=128, ws=FAKE, wsb=1 << 30):
    return lib.preattn_qkv_bf16(x, r, xa, g, eps, W, y, rstd, gq, gk, heps, cos, sin, hrstd, T, K, Hq, Hkv, D, ws,
                                wsb, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(r=ctypes.c_void_p(0x20000)), "RNL_ERR_NULL"),   # residual without x_add_out
    (dict(xa=ctypes.c_void_p(0x30000)), "RNL_ERR_NULL"),  # x_add_out without residual
    (dict(cos=ctypes.c_void_p(0x40000)), "RNL_ERR_NULL"),  # cos without sin
    (dict(W=NULL), "RNL_ERR_NULL"),
    (dict(D=24), "RNL_ERR_SHAPE"),
    (dict(D=528), "RNL_ERR_SHAPE"),
    (dict(D=8), "RNL_ERR_SHAPE"),
    (dict(Hq=0), "RNL_ERR_SHAPE"),
    (dict(Hkv=-1), "RNL_ERR_SHAPE"),
    (dict(Hq=1 << 20), "RNL_ERR_SHAPE"),
    (dict(T=(1 << 24) - 1, Hq=129, Hkv=0, D=16), "RNL_ERR_SHAPE"),  # T * (Hq + Hkv) > 2^31 heads
    (dict(heps=-1.0), "RNL_ERR_ARG"),
    (dict(gq=ODD), "RNL_ERR_ALIGN"),
    (dict(cos=ctypes.c_void_p(0x40004), sin=ctypes.c_void_p(0x50000)), "RNL_ERR_ALIGN"),
    (dict(T=64, ws=NULL), "RNL_ERR_WORKSPACE"),
])
def test_preattn_validation(lib, kw, code):
    assert preattn_call(lib, **kw) == E[code]


def heads_call(lib, a=FAKE, W=FAKE, y=FAKE, gq=NULL, gk=NULL, heps=1e-6, cos=NULL, sin=NULL, hrstd=NULL, M=64, K=64,
               Hq=4, Hkv=2, D=128):
    return lib.linear_heads_bf16(a, W, y, gq, gk, heps, cos, sin, hrstd, M, K, Hq, Hkv, D, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(a=NULL), "RNL_ERR_NULL"),
    (dict(y=NULL), "RNL_ERR_NULL"),
    (dict(sin=ctypes.c_void_p(0x40000)), "RNL_ERR_NULL"),  # sin without cos
    (dict(D=24), "RNL_ERR_SHAPE"),
    (dict(D=528), "RNL_ERR_SHAPE"),
    (dict(K=60), "RNL_ERR_SHAPE"),
    (dict(M=0), "RNL_ERR_SHAPE"),
    (dict(Hq=0), "RNL_ERR_SHAPE"),
    (dict(Hkv=-1), "RNL_ERR_SHAPE"),
    (dict(Hq=1 << 20), "RNL_ERR_SHAPE"),
    (dict(M=(1 << 24) - 1, Hq=129, Hkv=0, D=16), "RNL_ERR_SHAPE"),  # M * (Hq + Hkv) > 2^31 heads
    (dict(heps=float("inf")), "RNL_ERR_ARG"),
    (dict(W=ODD), "RNL_ERR_ALIGN"),
    (dict(gk=ODD), "RNL_ERR_ALIGN"),
    (dict(hrstd=ctypes.c_void_p(0x10002)), "RNL_ERR_ALIGN"),
])
def test_linear_heads_validation(lib, kw, code):
    assert heads_call(lib, **kw) == E[code]


def test_preattn_workspace_is_the_projection_workspace(lib):
    assert lib.preattn_qkv_bf16_workspace_bytes(4096, 4096, 32, 8, 128) == \
        lib.rmsnorm_linear_bf16_workspace_bytes(4096, 4096, 6144, 1, 1)
    assert lib.preattn_qkv_bf16_workspace_bytes(0, 4096, 32, 8, 128) == 0


def head_call(lib, yi=FAKE, yo=FAKE, g=NULL, eps=1e-6, cos=NULL, sin=NULL, rstd=NULL, T=4, ld=512, col0=0, H=4,
              D=128):
    return lib.head_rms_norm_bf16(yi, yo, g, eps, cos, sin, rstd, T, ld, col0, H, D, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(yi=NULL), "RNL_ERR_NULL"),
    (dict(yo=NULL), "RNL_ERR_NULL"),
    (dict(sin=ctypes.c_void_p(0x40000)), "RNL_ERR_NULL"),
    (dict(H=5), "RNL_ERR_SHAPE"),            # col0 + H * D > ld
    (dict(col0=8), "RNL_ERR_SHAPE"),
    (dict(col0=4, H=1), "RNL_ERR_SHAPE"),    # col0 not a multiple of 8
    (dict(ld=516, H=1), "RNL_ERR_SHAPE"),    # ld not a multiple of 8
    (dict(D=40, H=1), "RNL_ERR_SHAPE"),      # D not a multiple of 16
    (dict(T=0), "RNL_ERR_SHAPE"),
    (dict(T=(1 << 24) - 1, ld=4096, H=256, D=16), "RNL_ERR_SHAPE"),  # T * H > 2^31 heads
    (dict(T=1 << 24, H=1), "RNL_ERR_SHAPE"),  # T < 2^24
    (dict(eps=float("nan")), "RNL_ERR_ARG"),
    (dict(yo=ctypes.c_void_p(0x10000 + 1024)), "RNL_ERR_ARG"),  # overlaps y_in without being it
    (dict(g=ODD), "RNL_ERR_ALIGN"),
    (dict(rstd=ctypes.c_void_p(0x10002)), "RNL_ERR_ALIGN"),
])
def test_head_norm_validation(lib, kw, code):
    assert head_call(lib, **kw) == E[code]


def mla_call(lib, x=FAKE, W=FAKE, gq=NULL, gkv=NULL, eps=1e-6, Wb=FAKE, qr=FAKE, kv=FAKE, y=FAKE, rq=NULL, rkv=NULL,
             qakv=NULL, T=4, K=64, R=32, Rkv=16, N=8, ws=FAKE, wsb=1 << 30):
    return lib.mla_prolog_bf16(x, W, gq, gkv, eps, Wb, qr, kv, y, rq, rkv, qakv, T, K, R, Rkv, N, ws, wsb, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(kv=NULL), "RNL_ERR_NULL"),
    (dict(W=NULL), "RNL_ERR_NULL"),
    (dict(Rkv=12), "RNL_ERR_SHAPE"),
    (dict(Rkv=0), "RNL_ERR_SHAPE"),
    (dict(R=20), "RNL_ERR_SHAPE"),
    (dict(gkv=ODD), "RNL_ERR_ALIGN"),
    (dict(rkv=ctypes.c_void_p(0x10001)), "RNL_ERR_ALIGN"),
    (dict(qakv=ODD), "RNL_ERR_ALIGN"),
    (dict(ws=NULL), "RNL_ERR_WORKSPACE"),
    (dict(eps=-1.0), "RNL_ERR_ARG"),
])
def test_mla_validation(lib, kw, code):
    assert mla_call(lib, **kw) == E[code]


def test_mla_workspace(lib):
    # few tokens: no split, bf16 [q_a | kv]; many: fp32 split partials of both
    assert lib.mla_prolog_bf16_workspace_bytes(4, 7168, 1536, 512, 24576) == 4 * 2048 * 2 + (-(4 * 2048 * 2) % 256)
    assert lib.mla_prolog_bf16_workspace_bytes(1024, 7168, 1536, 512, 24576) >= 2 * 1024 * 2048 * 4


def mx_call(lib, x=FAKE, g=NULL, eps=1e-6, Wq=FAKE, ws=FAKE, y=FAKE, od=1, xq=NULL, xs=NULL, rstd=NULL, T=4, K=128,
            N=8, wsp=FAKE, wsb=1 << 30):
    return lib.rmsnorm_linear_mxfp8(x, g, eps, Wq, ws, y, od, xq, xs, rstd, T, K, N, wsp, wsb, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(ws=NULL), "RNL_ERR_NULL"),
    (dict(Wq=NULL), "RNL_ERR_NULL"),
    (dict(K=96), "RNL_ERR_SHAPE"),         # not a multiple of 64
    (dict(K=(1 << 20) + 64), "RNL_ERR_SHAPE"),
    (dict(od=4), "RNL_ERR_DTYPE"),         # no raw accumulator output
    (dict(od=3), "RNL_ERR_DTYPE"),
    (dict(xq=ODD), "RNL_ERR_ALIGN"),
    (dict(Wq=ODD), "RNL_ERR_ALIGN"),
    (dict(wsp=NULL), "RNL_ERR_WORKSPACE"),
    (dict(wsb=64), "RNL_ERR_WORKSPACE"),
    (dict(eps=float("inf")), "RNL_ERR_ARG"),
])
def test_mxfp8_validation(lib, kw, code):
    assert mx_call(lib, **kw) == E[code]


def test_mxfp8_workspace_and_atoms(lib):
    assert lib.rmsnorm_linear_mxfp8_workspace_bytes(4096, 4096, 6144, 1) >= 4096 * 4096 + 4096 * 64
    assert lib.rms_norm_quant_mxfp8(FAKE, NULL, 1e-6, FAKE, NULL, NULL, 4, 128, NULL) == E["RNL_ERR_NULL"]
    assert lib.rms_norm_quant_mxfp8(FAKE, NULL, 1e-6, FAKE, FAKE, NULL, 4, 100, NULL) == E["RNL_ERR_SHAPE"]
    assert lib.linear_mxfp8(FAKE, FAKE, FAKE, NULL, FAKE, 1, 4, 128, 8, NULL) == E["RNL_ERR_NULL"]
    assert lib.linear_mxfp8(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 160, 8, NULL) == E["RNL_ERR_SHAPE"]
    assert lib.linear_mxfp8(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 4, 128, 8, NULL) == E["RNL_ERR_DTYPE"]


def chain_call(lib, x=FAKE, Wa=FAKE, g=NULL, eps=1e-6, Wb=FAKE, qr=FAKE, y=FAKE, rstd=NULL, qa=NULL, T=4, K=64,
               R=32, N=8, ws=FAKE, wsb=1 << 30):
    return lib.norm_proj_chain(x, Wa, g, eps, Wb, qr, y, rstd, qa, T, K, R, N, ws, wsb, NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(qr=NULL), "RNL_ERR_NULL"),
    (dict(Wb=NULL), "RNL_ERR_NULL"),
    (dict(R=12), "RNL_ERR_SHAPE"),
    (dict(K=0), "RNL_ERR_SHAPE"),
    (dict(eps=-0.5), "RNL_ERR_ARG"),
    (dict(Wa=ODD), "RNL_ERR_ALIGN"),
    (dict(qa=ODD), "RNL_ERR_ALIGN"),
    (dict(ws=NULL), "RNL_ERR_WORKSPACE"),
])
def test_chain_validation(lib, kw, code):
    assert chain_call(lib, **kw) == E[code]


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        rnl.rmsnorm_linear_bf16(x, None, 1e-6, torch.zeros(8, 64, dtype=torch.bfloat16))


def test_noalloc_validation(lib):
    """The allocation-free entry point validates before any HIP call: sizes whose workspace exceeds the fixed
    scratch are rejected, like the other argument errors."""
    assert lib.rnl_noalloc_scratch_bytes() == 32 << 20
    f = lib.rmsnorm_linear_bf16_noalloc
    assert f(FAKE, NULL, 1e-6, FAKE, 1, FAKE, 1, NULL, 4097, 4096, 8, NULL) == E["RNL_ERR_WORKSPACE"]
    assert f(FAKE, NULL, 1e-6, FAKE, 2, FAKE, 2, NULL, 300000, 28672, 24, NULL) == E["RNL_ERR_WORKSPACE"]
    assert f(NULL, NULL, 1e-6, FAKE, 1, FAKE, 1, NULL, 4, 64, 8, NULL) == E["RNL_ERR_NULL"]
    assert f(FAKE, NULL, 1e-6, FAKE, 3, FAKE, 1, NULL, 4, 64, 8, NULL) == E["RNL_ERR_DTYPE"]
    assert f(FAKE, NULL, 1e-6, FAKE, 1, FAKE, 1, NULL, 4, 60, 8, NULL) == E["RNL_ERR_SHAPE"]


def test_stream_probe_validation(lib):
    assert lib.rnl_stream_read(NULL, 64, FAKE, 8, 4, NULL) == E["RNL_ERR_NULL"]
    assert lib.rnl_stream_read(FAKE, 0, FAKE, 8, 4, NULL) == E["RNL_ERR_SHAPE"]
    assert lib.rnl_stream_read(FAKE, 24, FAKE, 8, 4, NULL) == E["RNL_ERR_SHAPE"]
    assert lib.rnl_stream_read(FAKE, 64, FAKE, 0, 4, NULL) == E["RNL_ERR_SHAPE"]
    assert lib.rnl_stream_read(FAKE, 64, FAKE, 8, 3, NULL) == E["RNL_ERR_ARG"]
    assert lib.rnl_stream_read(ODD, 64, FAKE, 8, 4, NULL) == E["RNL_ERR_ALIGN"]


def test_mfma_probe_validation(lib):
    assert lib.rnl_mfma_probe(0, 8, 4, 16, NULL, NULL) == E["RNL_ERR_NULL"]
    assert lib.rnl_mfma_probe(3, 8, 4, 16, FAKE, NULL) == E["RNL_ERR_ARG"]
    assert lib.rnl_mfma_probe(-1, 8, 4, 16, FAKE, NULL) == E["RNL_ERR_ARG"]
    assert lib.rnl_mfma_probe(0, 0, 4, 16, FAKE, NULL) == E["RNL_ERR_SHAPE"]
    assert lib.rnl_mfma_probe(0, 8, 17, 16, FAKE, NULL) == E["RNL_ERR_SHAPE"]
    assert lib.rnl_mfma_probe(0, 8, 4, 0, FAKE, NULL) == E["RNL_ERR_SHAPE"]
    assert lib.rnl_mfma_probe(0, 8, 4, (1 << 24) + 1, FAKE, NULL) == E["RNL_ERR_SHAPE"]
    assert lib.rnl_mfma_probe(1, 8, 4, 16, ODD, NULL) == E["RNL_ERR_ALIGN"]


def test_clock_probe_validation(lib):
    assert lib.rnl_clock_probe(NULL, 0, 10, 1, NULL) == E["RNL_ERR_NULL"]
    assert lib.rnl_clock_probe(FAKE, 0, 0, 1, NULL) == E["RNL_ERR_SHAPE"]
    assert lib.rnl_clock_probe(FAKE, -1, 10, 1, NULL) == E["RNL_ERR_SHAPE"]
    assert lib.rnl_clock_probe(FAKE, 0, 10, 0, NULL) == E["RNL_ERR_SHAPE"]
    assert lib.rnl_clock_probe(ctypes.c_void_p(0x10004), 0, 10, 1, NULL) == E["RNL_ERR_ALIGN"]
