"""Graph replay: every entry point captured in a HIP graph (as the benchmark
times it) gives, on each of several replays, the same bits as the eager call.
Between replays the outputs are overwritten by eager work and the device is
synchronised, so a replay that skipped or reordered work would show."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import rmsnorm_linear_projection_amd as rnl
import synthetic

pytestmark = pytest.mark.gpu

EPS = 1e-6


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    rnl.load_library()
    yield
    torch.cuda.synchronize()


def dev(case):
    return {k: (v.cuda() if v is not None else None) for k, v in case.tensors.items()}


def check_replays(fn, outs, replays=3):
    """fn() writes into the preallocated tensors ``outs``."""
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm the side stream once before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        fn()
    for r in range(replays):
        for o in outs:
            o.view(torch.uint8).fill_(0xA5)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, ref):
            assert torch.equal(o.view(torch.uint8), e.view(torch.uint8)), f"replay {r} differs"


def ws_for(kind, *shape, **kw):
    n = rnl.workspace_bytes(kind, *shape, **kw)
    return torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("T,K,N", [(300, 1032, 200), (16, 4096, 512), (1, 256, 64), (1, 4104, 333)])
def test_graph_bf16(T, K, N):
    t = dev(synthetic.norm_linear_case(T, K, N, seed=1))
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    ws = ws_for("bf16", T, K, N)
    check_replays(lambda: rnl.rmsnorm_linear_bf16(t["x"], t["gamma"], EPS, t["W"], y=y, rstd_out=rstd, workspace=ws),
                  [y, rstd])


def test_graph_fp32_weights():
    T, K, N = 64, 8192, 24
    t = dev(synthetic.norm_linear_case(T, K, N, seed=2, gamma=False, w_dtype="fp32"))
    y = torch.empty((T, N), dtype=torch.float32, device="cuda")
    ws = ws_for("bf16", T, K, N, w_dtype=torch.float32, out_dtype=torch.float32)
    check_replays(lambda: rnl.rmsnorm_linear_bf16(t["x"], None, EPS, t["W"], out_dtype=torch.float32, y=y,
                                                  workspace=ws), [y])


def test_graph_int8_and_add():
    T, K, N = 130, 4112, 100
    t = dev(synthetic.with_residual(synthetic.int8_case(T, K, N, seed=3)))
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    xa = torch.empty_like(t["x"])
    xq = torch.empty((T, K), dtype=torch.int8, device="cuda")
    xs = torch.empty(T, dtype=torch.float32, device="cuda")
    check_replays(lambda: rnl.add_rmsnorm_linear_int8(t["x"], t["residual"], t["gamma"], EPS, t["Wq"], t["w_scale"],
                                                      y=y, x_add_out=xa, xq_out=xq, x_scale_out=xs),
                  [y, xa, xq, xs])


def test_graph_chain_and_mla():
    T, K, R, Rkv, N = 64, 4096, 128, 64, 64  # stage 1 split over K
    t = dev(synthetic.mla_case(T, K, R, Rkv, N, seed=4))
    W_akv = torch.cat([t["W_a"], t["W_kv"]], 0).contiguous()
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    qr = torch.empty((T, R), dtype=torch.bfloat16, device="cuda")
    kv = torch.empty((T, Rkv), dtype=torch.bfloat16, device="cuda")
    ws = ws_for("mla", T, K, R, Rkv, N)
    qakv = torch.empty((T, R + Rkv), dtype=torch.bfloat16, device="cuda")
    check_replays(lambda: rnl.mla_prolog_bf16(t["x"], W_akv, R, t["gamma"], t["gamma_ckv"], EPS, t["W_b"], qr_out=qr,
                                              kv_out=kv, y=y, qakv_out=qakv, workspace=ws), [y, qr, kv, qakv])
    y2 = torch.empty_like(y)
    qr2 = torch.empty_like(qr)
    qa2 = torch.empty((T, R), dtype=torch.bfloat16, device="cuda")
    ws2 = ws_for("chain", T, K, R, N)
    check_replays(lambda: rnl.norm_proj_chain(t["x"], t["W_a"], t["gamma"], EPS, t["W_b"], qr_out=qr2, y=y2,
                                              qa_out=qa2, workspace=ws2), [y2, qr2, qa2])


def test_graph_preattn_block():
    T = 40
    t = dev(synthetic.preattn_case(T, 1032, 6, 1, 128, seed=5, residual=True))
    N = 8 * 128
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    xa = torch.empty_like(t["x"])
    hr = torch.empty((T, 7), dtype=torch.float32, device="cuda")
    ws = ws_for("preattn", T, 1032, 6, 1, 128)
    check_replays(lambda: rnl.preattn_qkv_bf16(t["x"], t["gamma"], EPS, t["W"], 6, 1, 128, t["gamma_q"], t["gamma_k"],
                                               EPS, t["cos"], t["sin"], residual=t["residual"], x_add_out=xa, y=y,
                                               head_rstd_out=hr, workspace=ws), [y, xa, hr])


def test_graph_mxfp8():
    T, K, N = 300, 4160, 520  # K not a multiple of 1024: byte-wise scale staging
    t = dev(synthetic.mxfp8_case(T, K, N, seed=6))
    y = torch.empty((T, N), dtype=torch.float32, device="cuda")
    xq = torch.empty((T, K), dtype=torch.uint8, device="cuda")
    xs = torch.empty((T, K // 64), dtype=torch.uint8, device="cuda")
    check_replays(lambda: rnl.rmsnorm_linear_mxfp8(t["x"], t["gamma"], EPS, t["Wq"], t["w_scale"],
                                                   out_dtype=torch.float32, y=y, xq_out=xq, x_scale_out=xs),
                  [y, xq, xs])


@pytest.mark.parametrize("T,K,N", [(300, 1032, 200), (16, 4096, 512)])
def test_graph_noalloc(T, K, N):
    """The allocation-free entry point, captured as a caller that cannot allocate would capture it.  Between
    replays an eager call on other inputs runs through the same static scratch, so a replay that read anything
    left over in the scratch would show; every replay equals the eager call bit for bit."""
    t = dev(synthetic.norm_linear_case(T, K, N, seed=T + 7))
    o = dev(synthetic.norm_linear_case(T + 5, K + 8, N, seed=T + 8))
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    r = torch.empty(T, dtype=torch.float32, device="cuda")
    yo = torch.empty((T + 5, N), dtype=torch.bfloat16, device="cuda")

    def fn():
        rnl.rmsnorm_linear_bf16_noalloc(t["x"], t["gamma"], EPS, t["W"], y, rstd_out=r)
    fn()
    torch.cuda.synchronize()
    ref = [y.clone(), r.clone()]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        fn()
    for rep in range(3):
        rnl.rmsnorm_linear_bf16_noalloc(o["x"], o["gamma"], EPS, o["W"], yo)  # other data through the scratch
        y.view(torch.uint8).fill_(0xA5)
        r.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.uint8), ref[0].view(torch.uint8)), f"replay {rep}: y differs"
        assert torch.equal(r.view(torch.uint8), ref[1].view(torch.uint8)), f"replay {rep}: rstd differs"


@pytest.mark.parametrize("nbytes,workgroups,unroll", [(16, 1, 1), (4096 + 16, 3, 4), (48 << 20, 1024, 8),
                                                      (29 << 20, 2048, 16)])
def test_stream_probe_reads_every_word_once(nbytes, workgroups, unroll):
    """The HBM streaming probe folds every 32-bit word of the buffer exactly once: the XOR of its sink words is
    the XOR of the buffer's words (a word read twice or skipped would change it)."""
    g = torch.Generator().manual_seed(nbytes)
    host = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), generator=g, dtype=torch.int32)
    sink = rnl.stream_read(host.cuda(), workgroups, unroll)
    torch.cuda.synchronize()
    want = int(np.bitwise_xor.reduce(host.numpy().view(np.uint32)))
    got = int(np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)))
    assert got == want


@pytest.mark.parametrize("kind", ["bf16", "int8", "fp8"])
def test_mfma_probe_runs_its_instructions(kind):
    """The MFMA rate probe really issues its matrix instructions: the same launch gives the same sink twice, and
    the rate it implies (workgroups x waves x iterations x 8 instructions of known size over the measured time)
    lies between 5% and 120% of the published dense peak -- above it the work would have been dropped."""
    code, flop = rnl.MFMA_PROBE_KINDS[kind]
    peak = {"bf16": 2500.0, "int8": 5000.0, "fp8": 5000.0}[kind]
    wg, waves, iters = 256, 4, 2048
    s1 = rnl.mfma_probe(kind, wg, waves, iters)
    s2 = rnl.mfma_probe(kind, wg, waves, iters)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        rnl.mfma_probe(kind, wg, waves, iters, sink=s1)
    e1.record()
    torch.cuda.synchronize()
    rate = 5 * wg * waves * iters * 8 * flop / (e0.elapsed_time(e1) * 1e-3) / 1e12
    assert 0.05 * peak <= rate <= 1.2 * peak, rate


def test_clock_probe_reads_a_plausible_clock():
    """The clock probe waits, then spins for the requested wall time counting shader clocks: every wavefront's
    ratio is a clock between 100 MHz and 3 GHz, and its real-time ticks cover the requested time."""
    out = rnl.clock_probe(200, delay_us=50, workgroups=8)
    torch.cuda.synchronize()
    for cycles, ticks in out.cpu().tolist():
        assert ticks >= 200 * 100
        assert 100 <= 100.0 * cycles / ticks <= 3000
