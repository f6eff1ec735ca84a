"""Calls in flight on several streams at once give the bits of a lone call.

The library keeps no mutable state between calls (every intermediate lives in
the caller's workspace or outputs), so calls enqueued on different streams with
their own outputs and workspaces may overlap on the GPU in any way and must
still produce exactly what one call alone produces.  Each case runs one call on
the default stream for reference, then four streams (default priority) each run
the same call three times into their own buffers, interleaved so that the
streams' kernels overlap, and every stream's outputs are compared bit for bit.
"""
from __future__ import annotations

import pytest
import torch

import rmsnorm_linear_projection_amd as rnl
import synthetic

pytestmark = pytest.mark.gpu

EPS = 1e-6
STREAMS = 4


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    rnl.load_library()
    yield
    torch.cuda.synchronize()


def dev(case):
    return {k: (v.cuda() if v is not None else None) for k, v in case.tensors.items()}


def check_concurrent(make):
    """make() allocates one set of outputs (and workspace) on the current stream and returns (call, outputs);
    call() enqueues the library call on the current stream, writing those outputs."""
    call, outs = make()
    call()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    streams = [torch.cuda.Stream() for _ in range(STREAMS)]
    jobs = []
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            jobs.append(make())
    for _ in range(3):
        for s, (c, o) in zip(streams, jobs):
            with torch.cuda.stream(s):
                for t in o:
                    t.view(torch.uint8).fill_(0x5A)
                c()
    torch.cuda.synchronize()
    for i, (_, o) in enumerate(jobs):
        for j, (a, b) in enumerate(zip(o, ref)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"stream {i}, output {j} differs"


def ws_for(kind, *shape, **kw):
    n = rnl.workspace_bytes(kind, *shape, **kw)
    return torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("T,K,N", [(1000, 2056, 1000), (16, 4096, 1024), (1, 4096, 2048), (4, 2048, 512)])
def test_concurrent_bf16(T, K, N):
    """Tiled GEMM, weight streaming after the pre-pass, the single-row kernel, the fused-norm streaming kernel."""
    t = dev(synthetic.norm_linear_case(T, K, N, seed=T + N))

    def make():
        y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        r = torch.empty(T, dtype=torch.float32, device="cuda")
        ws = ws_for("bf16", T, K, N)
        return (lambda: rnl.rmsnorm_linear_bf16(t["x"], t["gamma"], EPS, t["W"], y=y, rstd_out=r, workspace=ws)), [y, r]
    check_concurrent(make)


def test_concurrent_fp32_weights():
    """Split-K partials in each caller's workspace, then the fixed-order finalize."""
    T, K, N = 512, 28672, 24
    t = dev(synthetic.norm_linear_case(T, K, N, seed=7, gamma=False, w_dtype="fp32"))

    def make():
        y = torch.empty((T, N), dtype=torch.float32, device="cuda")
        r = torch.empty(T, dtype=torch.float32, device="cuda")
        ws = ws_for("bf16", T, K, N, w_dtype=torch.float32, out_dtype=torch.float32)
        return (lambda: rnl.rmsnorm_linear_bf16(t["x"], None, EPS, t["W"], out_dtype=torch.float32, y=y, rstd_out=r,
                                                workspace=ws)), [y, r]
    check_concurrent(make)


def test_concurrent_int8_with_residual():
    T, K, N = 600, 4096, 1024
    t = dev(synthetic.with_residual(synthetic.int8_case(T, K, N, seed=8)))

    def make():
        y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        xa = torch.empty_like(t["x"])
        xq = torch.empty((T, K), dtype=torch.int8, device="cuda")
        xs = torch.empty(T, dtype=torch.float32, device="cuda")
        return (lambda: rnl.add_rmsnorm_linear_int8(t["x"], t["residual"], t["gamma"], EPS, t["Wq"], t["w_scale"],
                                                    y=y, x_add_out=xa, xq_out=xq, x_scale_out=xs)), [y, xa, xq, xs]
    check_concurrent(make)


def test_concurrent_chain_and_mla():
    """Both use a split-K first stage whose partials live in the caller's workspace."""
    T, K, R, Rkv, N = 256, 7168, 512, 256, 1024
    t = dev(synthetic.mla_case(T, K, R, Rkv, N, seed=9))
    W_akv = torch.cat([t["W_a"], t["W_kv"]], 0).contiguous()

    def make_mla():
        y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        qr = torch.empty((T, R), dtype=torch.bfloat16, device="cuda")
        kv = torch.empty((T, Rkv), dtype=torch.bfloat16, device="cuda")
        ws = ws_for("mla", T, K, R, Rkv, N)
        return (lambda: rnl.mla_prolog_bf16(t["x"], W_akv, R, t["gamma"], t["gamma_ckv"], EPS, t["W_b"], qr_out=qr,
                                            kv_out=kv, y=y, workspace=ws)), [y, qr, kv]
    check_concurrent(make_mla)

    def make_chain():
        y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        qr = torch.empty((T, R), dtype=torch.bfloat16, device="cuda")
        r = torch.empty(T, dtype=torch.float32, device="cuda")
        ws = ws_for("chain", T, K, R, N)
        return (lambda: rnl.norm_proj_chain(t["x"], t["W_a"], t["gamma"], EPS, t["W_b"], qr_out=qr, y=y, rstd_out=r,
                                            workspace=ws)), [y, qr, r]
    check_concurrent(make_chain)


@pytest.mark.parametrize("T", [512, 12])
def test_concurrent_preattn_block(T):
    """The per-head stage in the GEMM's epilogue (T = 512) and as its own pass after weight streaming (T = 12)."""
    K, Hq, Hkv, D = 2048, 8, 2, 128
    t = dev(synthetic.preattn_case(T, K, Hq, Hkv, D, seed=T, residual=True))
    N = (Hq + 2 * Hkv) * D

    def make():
        y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        xa = torch.empty_like(t["x"])
        hr = torch.empty((T, Hq + Hkv), dtype=torch.float32, device="cuda")
        ws = ws_for("preattn", T, K, Hq, Hkv, D)
        return (lambda: rnl.preattn_qkv_bf16(t["x"], t["gamma"], EPS, t["W"], Hq, Hkv, D, t["gamma_q"], t["gamma_k"],
                                             EPS, t["cos"], t["sin"], residual=t["residual"], x_add_out=xa, y=y,
                                             head_rstd_out=hr, workspace=ws)), [y, xa, hr]
    check_concurrent(make)


def test_concurrent_mxfp8():
    T, K, N = 700, 4096, 1000
    t = dev(synthetic.mxfp8_case(T, K, N, seed=10))

    def make():
        y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        xq = torch.empty((T, K), dtype=torch.uint8, device="cuda")
        xs = torch.empty((T, K // 64), dtype=torch.uint8, device="cuda")
        return (lambda: rnl.rmsnorm_linear_mxfp8(t["x"], t["gamma"], EPS, t["Wq"], t["w_scale"], y=y, xq_out=xq,
                                                 x_scale_out=xs)), [y, xq, xs]
    check_concurrent(make)
