#!/usr/bin/env python3
"""Throughput of the fused RMSNorm -> Linear hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME | --all]

A step is one call of the entry point over one batch of seeded synthetic
input already resident in HBM.  The default workload is the pre-attention
norm + fused QKV projection (bf16, T=4096, K=4096, N=6144).  One JSON line is
printed per workload with:
  value / unit   whole-step throughput: TFLOP/s (TOP/s for int8) where the
                 path is bound by MFMA, HBM GB/s where it is bound by memory;
  roofline       the dominant kernel's algorithmic flops or bytes per launch
                 over its average duration, timed with HIP events on the
                 stream it runs on, against the MI355X peak;
  cpu_baseline   the CPU oracle timed on a bounded sample of the same
                 workload on this host's cores.
Weight-bound workloads rotate through enough input copies that the 256 MB
Infinity Cache cannot serve them between steps.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused RMSNorm+Linear TFLOP/s (TOP/s int8) and HBM GB/s, % of roofline"
PEAK = {"bf16": 2500.0, "int8": 5000.0, "fp8": 5000.0, "hbm": 8000.0}  # TFLOP/s, TOP/s, GB/s (MI355X dense)
CSRC = os.path.join(ROOT, "rmsnorm_linear_projection_amd", "csrc")

WORKLOADS = {
    "preattn_qkv_T4096": dict(kind="bf16", T=4096, K=4096, N=6144, bound="mfma", dtype="bf16",
                              desc="pre-attention norm + fused QKV projection (Q 4096 + K 1024 + V 1024)"),
    "preattn_qkv_T16": dict(kind="bf16", T=16, K=4096, N=6144, bound="hbm", dtype="bf16",
                            desc="pre-attention norm + QKV, 16 decode tokens"),
    "preattn_qkv_T1": dict(kind="bf16", T=1, K=4096, N=6144, bound="hbm", dtype="bf16",
                           desc="pre-attention norm + QKV, 1 decode token"),
    "preattn_qkv_add_T4096": dict(kind="bf16", add=True, T=4096, K=4096, N=6144, bound="mfma", dtype="bf16",
                                  desc="residual add -> pre-attention norm -> fused QKV projection"),
    "preattn_qkv_add_T16": dict(kind="bf16", add=True, T=16, K=4096, N=6144, bound="hbm", dtype="bf16",
                                desc="residual add -> pre-attention norm -> QKV, 16 decode tokens"),
    "preattn_block_T4096": dict(kind="preattn", T=4096, K=4096, N=6144, Hq=32, Hkv=8, D=128, bound="mfma",
                                dtype="bf16", desc="residual add -> norm -> fused QKV -> per-head norm of Q, K -> RoPE"),
    "preattn_block_T16": dict(kind="preattn", T=16, K=4096, N=6144, Hq=32, Hkv=8, D=128, bound="hbm",
                              dtype="bf16", desc="pre-attention block, 16 decode tokens"),
    "small_T8": dict(kind="bf16", T=8, K=256, N=128, bound="hbm", dtype="bf16",
                     desc="bf16 RMSNorm + Linear, T=8 K=256 N=128"),
    "int8_w8a8": dict(kind="int8", T=2048, K=4096, N=4096, bound="mfma", dtype="int8",
                      desc="RMSNorm -> per-token int8 quant -> int8 GEMM -> dequant"),
    "mxfp8_qkv_T4096": dict(kind="mxfp8", T=4096, K=4096, N=6144, bound="mfma", dtype="fp8",
                            desc="RMSNorm -> MX quant (E4M3, E8M0 per 64) -> MXFP8 scaled GEMM, QKV shape"),
    "mla_q_chain": dict(kind="chain", T=1024, K=7168, R=1536, N=24576, bound="mfma", dtype="bf16",
                        desc="x -> W_a[1536,7168] -> RMSNorm -> W_b[24576,1536]"),
    "mla_prolog": dict(kind="mla", T=1024, K=7168, R=1536, Rkv=512, N=24576, bound="mfma", dtype="bf16",
                       desc="x -> [W_a; W_kv] -> RMSNorm of q_a and of kv -> W_b[24576,1536]"),
    "skinny_fp32": dict(kind="fp32w", T=512, K=28672, N=24, bound="hbm", dtype="f32",
                        desc="large-reduction tiny-width norm + linear, fp32 weight, no gamma"),
}
DEFAULT = "preattn_qkv_T4096"
KERNEL_SOURCES = {
    "gemm": ["gemm_kernel.hpp", "gemm_bf16.hip", "gemm_int8.hip", "common.hpp", "rows.hpp"],
    "small_m": ["small_m.hip", "common.hpp", "rows.hpp"],
    "small_m_norm": ["small_m.hip", "common.hpp", "rows.hpp"],
    "row_gemv": ["row_gemv.hip", "common.hpp"],
    "gemm_mx": ["gemm_mx.hip", "common.hpp"],
    "skinny": ["skinny.hip", "common.hpp"],
}


def flops_of(w):
    if w["kind"] == "mla":
        return 2.0 * w["T"] * (w["K"] * (w["R"] + w["Rkv"]) + w["R"] * w["N"])
    if w["kind"] == "chain":
        return 2.0 * w["T"] * (w["K"] * w["R"] + w["R"] * w["N"])
    return 2.0 * w["T"] * w["K"] * w["N"]


def bytes_of(w):
    """Algorithmic bytes: every input read once, every output written once."""
    T, K, N = w["T"], w["K"], w["N"]
    if w["kind"] == "preattn":
        # x, residual read, x_add written; gamma, W, both head gammas and the angle tables read; y written once
        return T * K * 2 * 3 + K * 2 + N * K * 2 + 2 * w["D"] * 2 + 2 * T * (w["D"] // 2) * 4 + T * N * 2
    if w["kind"] == "bf16":
        # with the residual add: the residual is read and x_add written as well
        return T * K * 2 * (3 if w.get("add") else 1) + K * 2 + N * K * 2 + T * N * 2
    if w["kind"] == "int8":
        return T * K * 2 + K * 2 + N * K + N * 4 + T * N * 2
    if w["kind"] == "mxfp8":
        return T * K * 2 + K * 2 + N * K + N * (K // 64) + T * N * 2
    if w["kind"] == "fp32w":
        return T * K * 2 + N * K * 4 + T * N * 4
    R = w["R"] + w.get("Rkv", 0)  # the KV branch adds its weight rows, gamma and normed outputs
    return T * K * 2 + R * K * 2 + R * 2 + w["R"] * N * 2 + T * R * 2 + T * N * 2


def src_sha(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def fused_small_norm(w):
    """True when the library norms the rows inside the weight-streaming kernel (no
    residual): normed rows within 64 KiB, and at most 4 rows, or 5 to 16 rows of
    at most 4096 values."""
    T, K = w["T"], w["K"]
    if w["kind"] != "bf16" or w.get("add"):
        return False
    return T * ((K + 31) // 32) * 64 <= 64 * 1024 and (T <= 4 or (T <= 16 and K <= 4096))


def row_gemv(w):
    """True when the tokens go to the whole-row VALU kernel: T at most 2, no
    residual, K at most 8192."""
    return w["kind"] == "bf16" and not w.get("add") and w["T"] <= 2 and w["K"] <= 8192


def kernel_key_of(w):
    """Key of the dominant kernel of a workload (KERNEL_MATCH, KERNEL_SOURCES)."""
    if w["kind"] == "fp32w":
        return "skinny"
    if w["kind"] == "mxfp8":
        return "gemm_mx"
    if row_gemv(w):
        return "row_gemv"
    if fused_small_norm(w):
        return "small_m_norm"
    return "small_m" if w["kind"] in ("bf16", "preattn") and w["T"] <= 16 else "gemm"


def load_traffic(name, kernel_key, launches_per_step=1):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3
    counters (FETCH_SIZE, WRITE_SIZE in KiB per dispatch, each scaled by the
    factor a plain copy of known size gives), or None when the counters were
    taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    rec = data.get("workloads", {}).get(name)
    if not rec or rec.get("src_sha") != src_sha(KERNEL_SOURCES[kernel_key]):
        return None
    cal = data["copy_calibration"]
    return (rec["fetch_kib"] * cal["fetch_scale"] + rec["write_kib"] * cal["write_scale"]) * 1024.0


class Setup:
    """Device inputs, outputs and the step / dominant-kernel closures."""

    def __init__(self, name, w):
        import torch

        import rmsnorm_linear_projection_amd as rnl
        import synthetic

        self.name, self.w = name, w
        dev = torch.device("cuda:0")
        kind = w["kind"]
        self.case = {
            "bf16": lambda: synthetic.norm_linear_case(w["T"], w["K"], w["N"], name=name),
            "fp32w": lambda: synthetic.norm_linear_case(w["T"], w["K"], w["N"], gamma=False, w_dtype="fp32", name=name),
            "int8": lambda: synthetic.int8_case(w["T"], w["K"], w["N"], name=name),
            "mxfp8": lambda: synthetic.mxfp8_qkv(w["T"]),
            "chain": lambda: synthetic.chain_case(w["T"], w["K"], w["R"], w["N"], name=name),
            "preattn": lambda: synthetic.preattn_block(w["T"]),
            "mla": lambda: synthetic.mla_prolog(),
        }[kind]()
        if w.get("add"):
            self.case = synthetic.with_residual(self.case)
            self.case.name = name
        t = {k: (v.to(dev) if v is not None else None) for k, v in self.case.tensors.items()}
        T, K, N = w["T"], w["K"], w["N"]
        eps = self.case.eps
        # rotate copies of the streamed operand when the path is bound by HBM
        self.copies = 1
        if w["bound"] == "hbm":
            rot = "W" if kind in ("bf16", "preattn") else "x"
            nbytes = t[rot].numel() * t[rot].element_size()
            self.copies = max(1, math.ceil(640e6 / nbytes)) if nbytes > 1e6 else 1
            t[rot + "_copies"] = [t[rot]] + [t[rot].clone() for _ in range(self.copies - 1)]
        self.t = t
        self.kernel = None
        self.kernel_key = None
        self.vendor = None  # (description, fn(i)): the vendor library on the dominant kernel's operands
        if kind == "bf16":
            y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(max(1, rnl.workspace_bytes("add_bf16" if w.get("add") else "bf16", T, K, N)),
                             dtype=torch.uint8, device=dev)
            Wc = t.get("W_copies", [t["W"]])
            if w.get("add"):
                xa = torch.empty_like(t["x"])
                self.step = lambda i: rnl.add_rmsnorm_linear_bf16(t["x"], t["residual"], t["gamma"], eps,
                                                                  Wc[i % len(Wc)], y=y, x_add_out=xa, workspace=ws)
            else:
                self.step = lambda i: rnl.rmsnorm_linear_bf16(t["x"], t["gamma"], eps, Wc[i % len(Wc)], y=y,
                                                              workspace=ws)
            a = rnl.rms_norm_bf16(t["x"], t["gamma"], eps)
            if row_gemv(w) or fused_small_norm(w):
                # the norm runs inside the weight-streaming kernel: the step is that one launch
                self.kernel_key = kernel_key_of(w)
                self.kernel = KERNEL_MATCH[self.kernel_key]
                self.kern = self.step
                self.kern_units = ("hbm", bytes_of(w))
            elif T <= 16:
                # weight streaming: the normed activations are re-read from L2,
                # the weight (rotated) from HBM
                self.kernel, self.kernel_key = "small_m_kernel", "small_m"
                self.kern = lambda i: rnl.linear_bf16(a, Wc[i % len(Wc)], y=y)
                self.kern_units = ("hbm", N * K * 2 + T * K * 2 + T * N * 2)
            else:
                self.kernel, self.kernel_key = "gemm_nt_kernel<bf16>", "gemm"
                self.kern = lambda i: rnl.linear_bf16(a, t["W"], y=y)
                self.kern_units = ("bf16", flops_of(w))
            Wv = Wc if T <= 16 else [t["W"]]
            self.vendor = ("torch.matmul(a, W.t()), bf16", lambda i: torch.matmul(a, Wv[i % len(Wv)].t(), out=y))
        elif kind == "mxfp8":
            y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(rnl.workspace_bytes("mxfp8", T, K, N), dtype=torch.uint8, device=dev)
            self.step = lambda i: rnl.rmsnorm_linear_mxfp8(t["x"], t["gamma"], eps, t["Wq"], t["w_scale"], y=y,
                                                           workspace=ws)
            xq, xs = rnl.rms_norm_quant_mxfp8(t["x"], t["gamma"], eps)
            self.kernel, self.kernel_key = "gemm_mx_kernel", "gemm_mx"
            self.kern = lambda i: rnl.linear_mxfp8(xq, xs, t["Wq"], t["w_scale"], y=y)
            self.kern_units = ("fp8", flops_of(w))
        elif kind == "preattn":
            Hq, Hkv, D = w["Hq"], w["Hkv"], w["D"]
            y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
            xa = torch.empty_like(t["x"])
            ws = torch.empty(max(1, rnl.workspace_bytes("preattn", T, K, Hq, Hkv, D)), dtype=torch.uint8, device=dev)
            Wc = t.get("W_copies", [t["W"]])
            self.step = lambda i: rnl.preattn_qkv_bf16(t["x"], t["gamma"], eps, Wc[i % len(Wc)], Hq, Hkv, D,
                                                       t["gamma_q"], t["gamma_k"], eps, t["cos"], t["sin"],
                                                       residual=t["residual"], x_add_out=xa, y=y, workspace=ws)
            a = rnl.rms_norm_bf16(t["x"], t["gamma"], eps)
            if T <= 16:
                self.kernel, self.kernel_key = "small_m_kernel", "small_m"
                self.kern = lambda i: rnl.linear_bf16(a, Wc[i % len(Wc)], y=y)
                self.kern_units = ("hbm", N * K * 2 + T * K * 2 + T * N * 2)
            else:
                # the step's GEMM: heads of 128 run the per-head stage in its epilogue
                self.kernel, self.kernel_key = "gemm_nt_kernel<bf16> (with the per-head epilogue)", "gemm"
                self.kern = lambda i: rnl.linear_heads_bf16(a, t["W"], Hq, Hkv, D, t["gamma_q"], t["gamma_k"], eps,
                                                            t["cos"], t["sin"], y=y)
                self.kern_units = ("bf16", flops_of(w))
            Wv = Wc if T <= 16 else [t["W"]]
            self.vendor = ("torch.matmul(a, W.t()), bf16", lambda i: torch.matmul(a, Wv[i % len(Wv)].t(), out=y))
        elif kind == "fp32w":
            y = torch.empty((T, N), dtype=torch.float32, device=dev)
            ws = torch.empty(max(1, rnl.workspace_bytes("bf16", T, K, N, w_dtype=torch.float32,
                                                        out_dtype=torch.float32)), dtype=torch.uint8, device=dev)
            xc = t.get("x_copies", [t["x"]])
            self.step = lambda i: rnl.rmsnorm_linear_bf16(xc[i % len(xc)], None, eps, t["W"], out_dtype=torch.float32,
                                                          y=y, workspace=ws)
            self.kernel, self.kernel_key = "skinny_partial_kernel+skinny_finalize_kernel", "skinny"
            self.kern = self.step
            self.kern_units = ("hbm", bytes_of(w))
            xf = [v.float() for v in xc]  # the vendor contraction takes fp32 rows
            self.vendor = ("torch.matmul(x.float(), W.t()), fp32 (the contraction only: no norm)",
                           lambda i: torch.matmul(xf[i % len(xf)], t["W"].t(), out=y))
        elif kind == "int8":
            y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(rnl.workspace_bytes("int8", T, K, N), dtype=torch.uint8, device=dev)
            self.step = lambda i: rnl.rmsnorm_linear_int8(t["x"], t["gamma"], eps, t["Wq"], t["w_scale"], y=y,
                                                          workspace=ws)
            xq, xs = rnl.rms_norm_quant_int8(t["x"], t["gamma"], eps)
            self.kernel, self.kernel_key = "gemm_nt_kernel<int8>", "gemm"
            self.kern = lambda i: rnl.linear_int8(xq, xs, t["Wq"], t["w_scale"], y=y)
            self.kern_units = ("int8", flops_of(w))
            acc = torch.empty((T, N), dtype=torch.int32, device=dev)
            Wqt = t["Wq"].t()
            self.vendor = ("torch._int_mm(xq, Wq.t()), int32 accumulators (no dequant)",
                           lambda i: torch._int_mm(xq, Wqt, out=acc))
        elif kind == "mla":
            R, Rkv = w["R"], w["Rkv"]
            y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
            qr = torch.empty((T, R), dtype=torch.bfloat16, device=dev)
            kvo = torch.empty((T, Rkv), dtype=torch.bfloat16, device=dev)
            W_akv = torch.cat([t["W_a"], t["W_kv"]], dim=0).contiguous()
            ws = torch.empty(rnl.workspace_bytes("mla", T, K, R, Rkv, N), dtype=torch.uint8, device=dev)
            self.step = lambda i: rnl.mla_prolog_bf16(t["x"], W_akv, R, t["gamma"], t["gamma_ckv"], eps, t["W_b"],
                                                      qr_out=qr, kv_out=kvo, y=y, workspace=ws)
            self.step(0)
            self.kernel, self.kernel_key = "gemm_nt_kernel<bf16> (stage 2, qr . W_b^T)", "gemm"
            self.kern = lambda i: rnl.linear_bf16(qr, t["W_b"], y=y)
            self.kern_units = ("bf16", 2.0 * T * R * N)
            self.vendor = ("torch.matmul(qr, W_b.t()), bf16 (stage 2)", lambda i: torch.matmul(qr, t["W_b"].t(), out=y))
        else:
            R = w["R"]
            y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
            qr = torch.empty((T, R), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(rnl.workspace_bytes("chain", T, K, R, N), dtype=torch.uint8, device=dev)
            self.step = lambda i: rnl.norm_proj_chain(t["x"], t["W_a"], t["gamma"], eps, t["W_b"], qr_out=qr, y=y,
                                                      workspace=ws)
            self.step(0)
            self.kernel, self.kernel_key = "gemm_nt_kernel<bf16> (stage 2, qr . W_b^T)", "gemm"
            self.kern = lambda i: rnl.linear_bf16(qr, t["W_b"], y=y)
            self.kern_units = ("bf16", 2.0 * T * R * N)
            self.vendor = ("torch.matmul(qr, W_b.t()), bf16 (stage 2)", lambda i: torch.matmul(qr, t["W_b"].t(), out=y))
        torch.cuda.synchronize()


def smu_mclk():
    """The memory clock (MHz) as the SMU's metrics table reports it (amdsmi), or None."""
    try:
        import amdsmi

        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]
        u = amdsmi.amdsmi_get_gpu_metrics_info(h).get("current_uclk")
        if isinstance(u, (int, float)) and 0 < u < 65535:
            return float(u)
        return float(amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.MEM)["clk"])
    except Exception:  # no amdsmi, no permission or no such metric
        return None


def clock_during(fn, steps, ms_per_step, replays=4):
    """Shader clock while fn's steps run: the `steps` calls are captured into a
    graph and replayed `replays` times back to back (untimed) while the library's
    clock probe, one wavefront per XCD on a second stream, waits out the first
    replay and then counts shader clocks against the 100 MHz real-time counter over
    the next two.  Returns {mean, min, max} MHz over the XCDs, or None for replays
    too short to sample."""
    import torch

    import rmsnorm_linear_projection_amd as rnl

    replay_us = steps * ms_per_step * 1e3
    if replay_us < 20:
        return None
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                fn(i)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    out = torch.zeros((8, 2), dtype=torch.int64, device="cuda:0")
    rnl.clock_probe(int(2 * replay_us), delay_us=int(replay_us), workgroups=8, out=out, stream=side)
    for _ in range(replays):
        g.replay()
    torch.cuda.synchronize()
    mhz = [100.0 * c / t for c, t in out.cpu().tolist() if t]
    del g
    if not mhz:
        return None
    return {"mean": round(sum(mhz) / len(mhz), 1), "min": round(min(mhz), 1), "max": round(max(mhz), 1)}


def time_loop(fn, steps, warmup, graph=True, repeats=1):
    """Median ms per call of fn(i) over `repeats` timed runs of `steps` calls,
    after exactly `warmup` untimed calls; also returns every run's ms per call.

    With graph=True the `steps` calls are captured once into a HIP graph after
    the warm-up calls (capturing runs nothing), and each timed run is one
    replay, so host-side launch overhead (Python, ctypes) does not leak into
    the device time; the captured work is exactly the eager calls' kernels.
    Events bracket each replay on the stream it runs on, after a device
    synchronisation.
    """
    import statistics

    import torch

    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    runs = []
    if graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(steps):
                    fn(warmup + i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for _ in range(repeats):
            start.record()
            g.replay()
            end.record()
            torch.cuda.synchronize()
            runs.append(start.elapsed_time(end) / steps)
        del g
    else:
        for r in range(repeats):
            start.record()
            for i in range(steps):
                fn(warmup + r * steps + i)
            end.record()
            torch.cuda.synchronize()
            runs.append(start.elapsed_time(end) / steps)
    return statistics.median(runs), runs  # ms


def oracle_threads():
    """Threads the oracle's row loops get: every CPU this process may run on, at most
    16 (the host CPU share one GPU of the box gets)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def config1_single_thread_ms(reps=20):
    """The C oracle on the small configuration (bf16, T=8, K=256, N=128, seed 0),
    single-threaded: median ms of `reps` whole calls (norm + bf16 projection)."""
    import statistics

    import numpy as np
    import torch

    import oracle as O
    import synthetic

    case = synthetic.small_norm_linear(seed=0)

    def bits(x):
        return x.contiguous().view(torch.int16).numpy().view(np.uint16)

    x, g, W = bits(case["x"]), bits(case["gamma"]), bits(case["W"])
    prev = O.threads()
    O.set_threads(1)
    try:
        times = []
        for _ in range(reps):
            t0 = time.perf_counter()
            O.rmsnorm_linear_bf16(x, g, case.eps, W)
            times.append((time.perf_counter() - t0) * 1e3)
    finally:
        O.set_threads(prev)
    return round(statistics.median(times), 4)


def cpu_baseline(setup, target_s=10.0):
    """The C oracle as it stands (plain loops, double accumulation, rows split over
    threads), on a bounded row sample of the same inputs, plus the small
    configuration single-threaded in ms."""
    import numpy as np
    import torch

    import oracle as O

    w, c = setup.w, setup.case

    def bits(x):
        return x.contiguous().view(torch.int16).numpy().view(np.uint16)

    kind = w["kind"]
    T = w["T"]
    nthreads = oracle_threads()
    O.set_threads(nthreads)

    def run(rows):
        x = bits(c["x"][:rows])
        g = None if c["gamma"] is None else bits(c["gamma"])
        if kind == "preattn":
            O.preattn_qkv(x, bits(c["residual"][:rows]), g, c.eps, bits(c["W"]), w["Hq"], w["Hkv"], w["D"],
                          bits(c["gamma_q"]), bits(c["gamma_k"]), c.eps, c["cos"][:rows].numpy(),
                          c["sin"][:rows].numpy())
        elif kind == "bf16" and w.get("add"):
            O.add_rmsnorm_linear_bf16(x, bits(c["residual"][:rows]), g, c.eps, bits(c["W"]))
        elif kind == "bf16":
            O.rmsnorm_linear_bf16(x, g, c.eps, bits(c["W"]))
        elif kind == "fp32w":
            O.rmsnorm_linear_fp32w(x, g, c.eps, c["W"].numpy())
        elif kind == "mxfp8":
            O.rmsnorm_linear_mxfp8(x, g, c.eps, c["Wq"].numpy(), c["w_scale"].numpy())
        elif kind == "int8":
            O.rmsnorm_linear_int8(x, g, c.eps, c["Wq"].numpy(), c["w_scale"].numpy())
        elif kind == "mla":
            O.mla_prolog(x, bits(c["W_a"]), g, c.eps, bits(c["W_b"]), bits(c["W_kv"]), bits(c["gamma_ckv"]))
        else:
            O.norm_proj_chain(x, bits(c["W_a"]), g, c.eps, bits(c["W_b"]))

    rows = min(T, 16)
    t0 = time.perf_counter()
    run(rows)
    dt = time.perf_counter() - t0
    # grow the row sample toward ~1/4 of the budget per call, then repeat
    while rows < T and dt < target_s / 4:
        rows = min(T, rows * 2)
        t0 = time.perf_counter()
        run(rows)
        dt = time.perf_counter() - t0
    calls, t_total = 0, 0.0
    while calls == 0 or t_total < target_s:
        t0 = time.perf_counter()
        run(rows)
        t_total += time.perf_counter() - t0
        calls += 1
    per_call = t_total / calls
    sub = dict(w, T=rows)
    if w["bound"] == "hbm":
        value, unit = bytes_of(sub) / per_call / 1e9, "GB/s"
    else:
        value, unit = flops_of(sub) / per_call / 1e12, "TOP/s" if kind == "int8" else "TFLOP/s"
    return {"value": round(value, 6), "unit": unit, "cores": nthreads, "kind": "oracle",
            "sample": f"first {rows} of {T} token rows, {calls} call(s), {per_call:.3f} s per call",
            "impl": "C (oracle/c/rnl_oracle.c): plain loops, double accumulation, gcc -O2 -ffp-contract=off",
            "host_cpus": {"nproc": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
                          "online": O.cpu_count()},
            "config1_single_thread_ms": config1_single_thread_ms()}


def bench_one(name, steps, warmup, with_cpu=True, graph=True, vendor=False, repeats=1):
    import torch

    w = WORKLOADS[name]
    s = Setup(name, w)
    ms, runs = time_loop(s.step, steps, warmup, graph, repeats)
    kms = time_loop(s.kern, steps, warmup, graph, repeats)[0] if s.kern is not s.step else ms
    sclk = clock_during(s.step, steps, ms)
    mclk = smu_mclk()
    if w["bound"] == "hbm":
        value, unit = bytes_of(w) / (ms * 1e-3) / 1e9, "GB/s"
    else:
        value = flops_of(w) / (ms * 1e-3) / 1e12
        unit = "TOP/s" if w["kind"] == "int8" else "TFLOP/s"
    peak_key, per_launch = s.kern_units
    if peak_key == "hbm":
        achieved, ru, bound = per_launch / (kms * 1e-3) / 1e9, "GB/s", "hbm"
    else:
        achieved, ru, bound = per_launch / (kms * 1e-3) / 1e12, ("TOP/s" if peak_key == "int8" else "TFLOP/s"), "mfma"
    traffic = load_traffic(name, s.kernel_key)
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic",
        "config": {"workload": s.case.name, "description": w["desc"],
                   **{k: w[k] for k in ("T", "K", "R", "Rkv", "N", "Hq", "Hkv", "D") if k in w},
                   "parallelism": "none (1 GPU)", "input_copies": s.copies,
                   "timing": ("hip graph of the timed steps" if graph else "eager launches")
                   + (f", median of {repeats} timed runs" if repeats > 1 else "")},
        "roofline": {"bound": bound, "kernel": s.kernel, "achieved": round(achieved, 3), "peak": PEAK[peak_key],
                     "unit": ru, "frac": round(achieved / PEAK[peak_key], 4),
                     "kernel_ms": round(kms, 6),
                     "traffic": None if traffic is None else int(traffic)},
    }
    if repeats > 1:
        line["ms_per_step_runs"] = [round(r, 6) for r in runs]
    line["clocks"] = {"sclk_mhz": sclk,
                      "sclk_source": "clock probe (s_memtime against the 100 MHz s_memrealtime), one wavefront per "
                                     "XCD on a second stream, over the 2nd and 3rd of 4 extra untimed replays of "
                                     "the timed steps",
                      "mclk_mhz": mclk, "mclk_source": "amdsmi (as the SMU reports it)"}
    if w["kind"] in ("chain", "mla"):
        # stage 2 is timed alone (the GEMM on the step's own qr); stage 1 with its reduce
        # and norm is the rest of the step
        f2 = 2.0 * w["T"] * w["R"] * w["N"]
        f1 = flops_of(w) - f2
        ms1 = ms - kms
        line["stages"] = [
            {"stage": "x . W^T (split-K) + reduce + norm (step minus stage 2)", "ms": round(ms1, 6),
             "achieved": round(f1 / (ms1 * 1e-3) / 1e12, 3), "peak": PEAK["bf16"], "unit": "TFLOP/s",
             "frac": round(f1 / (ms1 * 1e-3) / 1e12 / PEAK["bf16"], 4)},
            {"stage": "qr . W_b^T (timed alone)", "ms": round(kms, 6),
             "achieved": round(f2 / (kms * 1e-3) / 1e12, 3), "peak": PEAK["bf16"], "unit": "TFLOP/s",
             "frac": round(f2 / (kms * 1e-3) / 1e12 / PEAK["bf16"], 4)},
        ]
    if vendor and s.vendor is not None:
        # context, not a target: the vendor library (hipBLASLt / rocBLAS through torch) timed the same
        # way on the same operands as the dominant kernel, in the same process
        desc, fn = s.vendor
        try:
            line["vendor"] = {"op": desc, "ms": round(time_loop(fn, steps, warmup, graph)[0], 6),
                              "kernel_ms": round(kms, 6)}
        except RuntimeError as e:  # an op the installed torch cannot run or capture
            line["vendor"] = {"op": desc, "error": str(e).splitlines()[0][:200]}
    if with_cpu:
        line["cpu_baseline"] = cpu_baseline(s)
    del s
    torch.cuda.empty_cache()
    return line


COPY_BYTES = 256 << 20  # size of the plain device copy that calibrates FETCH_SIZE / WRITE_SIZE
KERNEL_MATCH = {"gemm": "gemm_nt_kernel", "small_m": "small_m_kernel", "small_m_norm": "small_m_norm_kernel",
                "row_gemv": "row_gemv_norm_kernel",
                "skinny": "skinny_", "gemm_mx": "gemm_mx_kernel"}


def copy_calibration(steps=5):
    """A plain device-to-device copy of COPY_BYTES, launched `steps` times, for
    scaling the HBM counters (each dispatch reads and writes COPY_BYTES)."""
    import torch

    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": steps}), flush=True)


def _counter_kib(csv_path, name_part, counter, all_names=False):
    """Per-dispatch value of `counter` (KiB) from a rocprofv3 counter_collection.csv,
    averaged over the dispatches of the most frequent kernel whose name contains
    name_part (the timed kernel), or, with all_names, the sum of those averages
    over every matching kernel (a kernel pair timed as one unit)."""
    import csv

    per = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter:
                d = per.setdefault(r["Kernel_Name"], {})
                d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} records for kernels matching {name_part!r} in {csv_path}")
    avg = {k: sum(v.values()) / len(v) for k, v in per.items()}
    if all_names:
        return sum(avg.values()), min(len(v) for v in per.values())
    top = max(per, key=lambda k: len(per[k]))
    return avg[top], len(per[top])


def record_counters(name, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """Fold two rocprofv3 --pmc runs of a workload (FETCH_SIZE, then WRITE_SIZE)
    and the same two counters of the calibration copy into profiles/counters.json."""
    key = kernel_key_of(WORKLOADS[name])
    pair = key == "skinny"
    fk, nf = _counter_kib(fetch_csv, KERNEL_MATCH[key], "FETCH_SIZE", pair)
    wk, nw = _counter_kib(write_csv, KERNEL_MATCH[key], "WRITE_SIZE", pair)
    cf, _ = _counter_kib(copy_fetch_csv, "", "FETCH_SIZE")
    cw, _ = _counter_kib(copy_write_csv, "", "WRITE_SIZE")
    path = os.path.join(ROOT, "profiles", "counters.json")
    data = {"workloads": {}}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    data["copy_calibration"] = {"copy_bytes": COPY_BYTES, "fetch_kib": cf, "write_kib": cw,
                                "fetch_scale": COPY_BYTES / 1024.0 / cf, "write_scale": COPY_BYTES / 1024.0 / cw}
    data["workloads"][name] = {"kernel": KERNEL_MATCH[key], "src_sha": src_sha(KERNEL_SOURCES[key]),
                               "fetch_kib": fk, "write_kib": wk, "dispatches": [nf, nw]}
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print(json.dumps(data["workloads"][name]))


CEILING_SIZES = [(512 * 28672 * 2, "x of the skinny fp32 workload (29 MiB)"),
                 (6144 * 4096 * 2, "the decode QKV weight (48 MiB)"),
                 (256 << 20, "256 MiB"), (1 << 30, "1 GiB"), (4 << 30, "4 GiB")]


CEILING_SHAPES = [(256, 8), (256, 16), (512, 4), (512, 8), (512, 16), (768, 16), (1024, 4), (1024, 8), (1024, 16),
                  (2048, 4), (2048, 8)]


def hbm_ceiling(steps, warmup, repeats):
    """HBM read ceiling: the library's read-only streaming probe (rnl_stream_read) on
    buffers of the sizes above, rotated over enough copies (>= 640 MB in all) that
    the 256 MB Infinity Cache cannot serve a read from the previous one; one JSON
    line per size."""
    import torch

    import rmsnorm_linear_projection_amd as rnl

    for nbytes, what in CEILING_SIZES:
        copies = max(1, math.ceil(640e6 / nbytes))
        bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device="cuda:0") for _ in range(copies)]
        sink = torch.empty(max(w for w, _ in CEILING_SHAPES), dtype=torch.int32, device="cuda:0")
        shapes = {}
        for wgs, unroll in CEILING_SHAPES:
            ms, _ = time_loop(lambda i: rnl.stream_read(bufs[i % copies], wgs, unroll, sink), steps, warmup, True,
                              repeats)
            shapes[f"{wgs}x{unroll}"] = round(ms * 1e3, 3)
        best = min(shapes, key=shapes.get)
        us = shapes[best]
        print(json.dumps({"probe": "rnl_stream_read (read-only HBM stream)", "buffer": what, "bytes": nbytes,
                          "copies": copies, "best_shape": best, "us_per_read": us,
                          "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                          "frac_of_8000_GB/s": round(nbytes / (us * 1e-6) / 1e9 / PEAK["hbm"], 4),
                          "us_by_shape (workgroups x loads in flight per lane)": shapes,
                          "timing": f"hip graph of {steps} reads, median of {repeats} runs, {warmup} untimed"}),
              flush=True)
        del bufs
        torch.cuda.empty_cache()


def mfma_ceiling(steps, warmup, repeats):
    """Matrix-core ceiling: the library's MFMA rate probe (rnl_mfma_probe), one
    workgroup per CU, with one and with two wavefronts per SIMD, for the bf16,
    int8 and scaled-E4M3 instructions the contractions use; the shader clock is
    read beside the timed replays.  One JSON line per instruction."""
    import torch

    import rmsnorm_linear_projection_amd as rnl

    peaks = {"bf16": PEAK["bf16"], "int8": PEAK["int8"], "fp8": PEAK["fp8"]}
    for kind, (_, flop) in rnl.MFMA_PROBE_KINDS.items():
        res = {}
        for waves in (4, 8):
            iters = 2048
            sink = torch.empty(256 * waves, dtype=torch.int32, device="cuda:0")
            fn = lambda i: rnl.mfma_probe(kind, 256, waves, iters, sink)  # noqa: E731
            ms, _ = time_loop(fn, steps, warmup, True, repeats)
            sclk = clock_during(fn, steps, ms)
            rate = 256 * waves * iters * 8 * flop / (ms * 1e-3) / 1e12
            res[f"{waves // 4} per SIMD"] = {"us_per_launch": round(ms * 1e3, 2), "rate": round(rate, 1),
                                             "frac_of_peak": round(rate / peaks[kind], 4),
                                             "sclk_mhz": sclk and sclk["mean"]}
        print(json.dumps({"probe": "rnl_mfma_probe (register-only matrix instructions, 8 accumulators per wavefront)",
                          "kind": kind, "unit": "TOP/s" if kind == "int8" else "TFLOP/s", "peak": peaks[kind],
                          "wavefronts": res,
                          "timing": f"hip graph of {steps} launches, median of {repeats} runs, {warmup} untimed"}),
              flush=True)


def _short_kernel(name):
    """Kernel name without namespaces and argument list."""
    n = name[5:] if name.startswith("void ") else name
    n = n.replace("rnl::(anonymous namespace)::", "").replace("rnl::", "")
    depth = 0
    for i in range(len(n) - 1, -1, -1):
        if n[i] == ")":
            depth += 1
        elif n[i] == "(":
            depth -= 1
            if depth == 0:
                n = n[:i]
                break
    return n.strip()


def record_mfma(name, run_dir):
    """Fold one rocprofv3 run with --pmc MfmaUtil GRBM_GUI_ACTIVE --kernel-trace of a
    workload into profiles/counters.json: per library kernel, the average over its
    dispatches of the MFMA busy percentage, of GRBM_GUI_ACTIVE (GPU clock cycles
    while the kernel ran, summed over the 8 XCDs) and of the kernel's duration,
    and the clock they imply (cycles per XCD / duration)."""
    import csv
    import glob

    cc = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    kt = glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not cc or not kt:
        raise SystemExit(f"no counter_collection / kernel_trace CSV under {run_dir}")
    dur = {}
    for r in csv.DictReader(open(kt[0])):
        dur[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3  # us
    per = {}
    for r in csv.DictReader(open(cc[0])):
        if "rnl::" not in r["Kernel_Name"]:
            continue
        k = _short_kernel(r["Kernel_Name"])
        d = per.setdefault(k, {}).setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    out = {}
    for k, disp in per.items():
        rows = [(v, dur.get(i)) for i, v in disp.items() if dur.get(i)]
        if not rows:
            continue
        n = len(rows)
        util = sum(v.get("MfmaUtil", 0.0) for v, _ in rows) / n
        grbm = sum(v.get("GRBM_GUI_ACTIVE", 0.0) for v, _ in rows) / n
        us = sum(t for _, t in rows) / n
        out[k] = {"dispatches": n, "mfma_busy_pct": round(util, 2), "grbm_gui_active": round(grbm),
                  "duration_us": round(us, 3), "sclk_mhz": round(grbm / 8 / us, 1)}
    path = os.path.join(ROOT, "profiles", "counters.json")
    data = json.load(open(path)) if os.path.exists(path) else {"workloads": {}}
    key = kernel_key_of(WORKLOADS[name])
    rec = data["workloads"].setdefault(name, {})
    rec["mfma"] = {"src_sha": src_sha(KERNEL_SOURCES[key]), "kernels": out}
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print(json.dumps(rec["mfma"]))


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=1000, help="untimed calls before the timed ones")
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed runs of --steps calls each (each bracketed by synchronisations); the line reports "
                         "their median")
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(WORKLOADS))
    ap.add_argument("--all", action="store_true", help="one line per workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a captured graph")
    ap.add_argument("--vendor", action="store_true",
                    help="also time the vendor library (torch.matmul / torch._int_mm) on the dominant kernel's operands")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="measure only the matrix-core rate of the bf16, int8 and scaled-E4M3 instructions")
    ap.add_argument("--hbm-ceiling", action="store_true",
                    help="measure only the read-only HBM streaming ceiling at several buffer sizes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only the plain copy that calibrates the HBM byte counters")
    ap.add_argument("--record-counters", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="fold rocprofv3 counter_collection.csv files of --workload into profiles/counters.json")
    ap.add_argument("--record-mfma", metavar="RUN_DIR",
                    help="fold a rocprofv3 --pmc MfmaUtil GRBM_GUI_ACTIVE --kernel-trace run of --workload "
                         "into profiles/counters.json")
    args = ap.parse_args()
    if args.record_counters:
        record_counters(args.workload, *args.record_counters)
        return
    if args.record_mfma:
        record_mfma(args.workload, args.record_mfma)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); multi-GPU runs are not supported",
              file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.mfma_ceiling:
        mfma_ceiling(args.steps, args.warmup, args.repeats)
        return
    if args.hbm_ceiling:
        hbm_ceiling(args.steps, args.warmup, args.repeats)
        return
    import rmsnorm_linear_projection_amd as rnl

    if not os.path.exists(rnl.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    names = sorted(WORKLOADS, key=lambda n: n != DEFAULT) if args.all else [args.workload]
    for n in names:
        print(json.dumps(bench_one(n, args.steps, args.warmup, with_cpu=not args.no_cpu, graph=not args.eager,
                                   vendor=args.vendor, repeats=args.repeats)),
              flush=True)


if __name__ == "__main__":
    main()
