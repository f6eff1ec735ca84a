"""Operands past 4 GiB, the largest T and N the library accepts, and grids past 2^16
workgroups per axis, through the C ABI.

One MI355X holds 288 GB, so a single activation, weight or output can exceed the
4 GiB that a 32-bit byte offset reaches.  The kernels address every row, weight
row and tile from a 64-bit base and keep only offsets inside one row or tile in
32 bits; these cases put rows on both sides of the 4 GiB mark of each operand and
check them against the oracle with the rules of the parity suite:

  * rstd within 8 fp32 ulps of the oracle's own;
  * bf16 outputs within 1e-2 (|y_ref| + 1e-2) of the oracle evaluated with the
    device's rstd (identical bf16 normed rows on both sides);
  * int8 codes and scales bit-exact given the device's rstd, int32 accumulators
    bit-exact against the int64 product of the device's codes;
  * fp32 outputs of the fp32-weight path within 1e-5 max(|y_ref|, rms(y_ref));
  * MXFP8 codes and scales bit-exact, the product within the scaled-MFMA bound.

Inputs of several GB are drawn on the device (``synthetic.normal_on_device``);
only the checked rows come back to the host.  Every output is filled beforehand
with a value the path cannot produce (NaN, INT32_MIN, int8 -128), and the whole
output is checked on the device to hold none of it afterwards, so no tile or
row past the sampled ones was skipped.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import rmsnorm_linear_projection_amd as rnl
import synthetic
from tests._util import bits, f32
from tests.test_gpu_parity import (EPS, assert_bf16_close, assert_mx_close, assert_rstd, check_normed_stage,
                                   mx_abs_sum, mx_step_max)

pytestmark = pytest.mark.gpu

GIB4 = 1 << 32


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    rnl.load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def sample(n, row_bytes, seed, extra=40):
    """Indices to check out of n rows: both ends, 8 on each side of the 4 GiB mark of every operand whose row is
    row_bytes long (for each entry of row_bytes), and `extra` drawn at random."""
    rng = np.random.default_rng(seed)
    pick = {0, 1, 2, 3, n - 4, n - 3, n - 2, n - 1}
    for rb in row_bytes:
        mark = GIB4 // rb  # the row holding (or starting at) byte 2^32
        pick |= set(range(max(0, mark - 8), min(n, mark + 9)))
    pick |= set(rng.integers(0, n, extra).tolist())
    return np.array(sorted(i for i in pick if 0 <= i < n), dtype=np.int64)


def rows_of(t, idx):
    return t.index_select(0, torch.as_tensor(idx, device=t.device)).cpu()


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# x [557093, 4096] bf16 is 4.56 GB: rows from 524288 on start past 4 GiB
T_BIG, K_BIG = 557_093, 4096


@pytest.fixture(scope="module")
def x_big():
    x = synthetic.normal_on_device((T_BIG, K_BIG), 1.0, seed=41, stream=1)
    yield x
    del x
    free()


def test_bf16_activations_and_output_past_4gib(x_big):
    """x, the normed activations and y [557093, 4000] (4.46 GB) all cross 4 GiB; the tiled GEMM path."""
    T, K, N = T_BIG, K_BIG, 4000
    case = synthetic.norm_linear_case(1, K, N, seed=41)
    g, W = case["gamma"].cuda(), case["W"].cuda()
    y = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    rstd = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    rnl.rmsnorm_linear_bf16(x_big, g, EPS, W, y=y, rstd_out=rstd)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()) and bool((rstd > 0).all()), "outputs left unwritten"
    rows = sample(T, [K * 2, N * 2], seed=1)
    xb, gb = bits(rows_of(x_big, rows)), bits(case["gamma"])
    r = rows_of(rstd, rows).numpy()
    assert_rstd(r, O.rms_norm_rows(xb, gb, EPS)[1], "bf16 past 4 GiB")
    y32, _, _ = O.rmsnorm_linear_bf16(xb, gb, EPS, bits(case["W"]), rstd=r)
    assert_bf16_close(f32(rows_of(y, rows)), y32, "bf16 past 4 GiB")
    del y, rstd
    free()


def test_fp32_weights_past_4gib(x_big):
    """The split-K fp32-weight path over the same 4.56 GB of x (no gamma, fp32 out)."""
    T, K, N = T_BIG, K_BIG, 24
    case = synthetic.norm_linear_case(1, K, N, seed=42, gamma=False, w_dtype="fp32")
    W = case["W"].cuda()
    y = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
    rstd = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    rnl.rmsnorm_linear_bf16(x_big, None, EPS, W, out_dtype=torch.float32, y=y, rstd_out=rstd)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()) and bool((rstd > 0).all()), "outputs left unwritten"
    rows = sample(T, [K * 2], seed=2)
    xb = bits(rows_of(x_big, rows))
    r = rows_of(rstd, rows).numpy()
    assert_rstd(r, O.rms_norm_rows(xb, None, EPS)[1], "fp32 weights past 4 GiB")
    y_ref, _ = O.rmsnorm_linear_fp32w(xb, None, EPS, case["W"].numpy(), rstd=r)
    scale = max(float(np.sqrt(np.mean(y_ref.astype(np.float64) ** 2))), 1e-30)
    err = np.abs(rows_of(y, rows).numpy().astype(np.float64) - y_ref)
    assert (err <= 1e-5 * np.maximum(np.abs(y_ref), scale)).all(), f"max err {err.max():.3g} (rms {scale:.3g})"
    del y, rstd
    free()


def test_mxfp8_past_4gib(x_big):
    """MXFP8 over the same x: codes [T, K] and scales written past row 524288 of x's 4 GiB mark."""
    T, K, N = T_BIG, K_BIG, 64
    case = synthetic.mxfp8_case(1, K, N, seed=43)
    wq, ws = case["Wq"], case["w_scale"]
    xq = torch.empty((T, K), dtype=torch.uint8, device="cuda")
    xs = torch.empty((T, K // 64), dtype=torch.uint8, device="cuda")
    rstd = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    y = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
    rnl.rmsnorm_linear_mxfp8(x_big, case["gamma"].cuda(), EPS, wq.cuda(), ws.cuda(), out_dtype=torch.float32,
                             xq_out=xq, x_scale_out=xs, rstd_out=rstd, y=y)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()) and bool((rstd > 0).all()), "outputs left unwritten"
    rows = sample(T, [K * 2], seed=3)
    xb, gb = bits(rows_of(x_big, rows)), bits(case["gamma"])
    r = rows_of(rstd, rows).numpy()
    assert_rstd(r, O.rms_norm_rows(xb, gb, EPS)[1], "MXFP8 past 4 GiB")
    ref = O.rmsnorm_linear_mxfp8(xb, gb, EPS, wq.numpy(), ws.numpy(), rstd=r)
    assert np.array_equal(rows_of(xq, rows).numpy(), ref["q"]), "codes differ"
    assert np.array_equal(rows_of(xs, rows).numpy(), ref["x_scale"]), "scales differ"
    s_abs = mx_abs_sum(ref["q"], ref["x_scale"], wq.numpy(), ws.numpy())
    sm = mx_step_max(ref["q"], ref["x_scale"]) @ mx_step_max(wq.numpy(), ws.numpy()).T
    assert_mx_close(rows_of(y, rows).numpy(), ref["y32"].astype(np.float64), s_abs, sm, "MXFP8 past 4 GiB", K)
    del xq, xs, rstd, y
    free()


def test_int8_codes_past_4gib():
    """int8 W8A8 with xq [1049613, 4096] (4.30 GB) crossing 4 GiB, and x (8.6 GB) crossing it twice over;
    int32 accumulators out."""
    T, K, N = 1_049_613, 4096, 48
    x = synthetic.normal_on_device((T, K), 1.0, seed=44, stream=1)
    case = synthetic.int8_case(1, K, N, seed=44)
    xq = torch.full((T, K), -128, dtype=torch.int8, device="cuda")  # -128 is never a code
    xs = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    rstd = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    acc = torch.full((T, N), -(2 ** 31), dtype=torch.int32, device="cuda")  # |acc| <= K * 127^2 < 2^31
    rnl.rmsnorm_linear_int8(x, case["gamma"].cuda(), EPS, case["Wq"].cuda(), case["w_scale"].cuda(),
                            out_dtype=torch.int32, xq_out=xq, x_scale_out=xs, rstd_out=rstd, y=acc)
    torch.cuda.synchronize()
    assert bool((xq != -128).all()) and bool(torch.isfinite(xs).all()) and bool((rstd > 0).all())
    assert bool((acc != -(2 ** 31)).all()), "accumulators left unwritten"
    rows = sample(T, [K * 2, K], seed=4)
    xb, gb = bits(rows_of(x, rows)), bits(case["gamma"])
    r = rows_of(rstd, rows).numpy()
    assert_rstd(r, O.rms_norm_rows(xb, gb, EPS)[1], "int8 past 4 GiB")
    n, _ = O.rms_norm_rows(xb, gb, EPS, rstd=r)
    q_ref, xs_ref, _ = O.quant_rows(n)
    q = rows_of(xq, rows).numpy()
    assert np.array_equal(q, q_ref), f"xq not bit-exact ({int((q != q_ref).sum())} differ)"
    assert np.array_equal(rows_of(xs, rows).numpy(), xs_ref), "x_scale not bit-exact"
    acc_ref = O.int8_gemm(q, case["Wq"].numpy())
    assert np.array_equal(rows_of(acc, rows).numpy().astype(np.int64), acc_ref), "int32 accumulators not bit-exact"
    del x, xq, xs, rstd, acc
    free()


# W [270000, 8192] bf16 is 4.42 GB: weight rows from 262144 on start past 4 GiB
N_WBIG, K_WBIG = 270_000, 8192


@pytest.fixture(scope="module")
def w_big():
    W = synthetic.normal_on_device((N_WBIG, K_WBIG), K_WBIG ** -0.5, seed=45, stream=3)
    yield W
    del W
    free()


@pytest.mark.parametrize("T", [1, 4, 16])
def test_decode_weight_past_4gib(w_big, T):
    """A 4.42 GB weight (a vocabulary-sized projection) through the decode kernels: one token (whole weight rows
    per wavefront), four (norm fused into the weight stream) and sixteen (norm pre-pass, weight streaming)."""
    N, K = N_WBIG, K_WBIG
    case = synthetic.norm_linear_case(T, K, 1, seed=45 + T)
    y = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    rstd = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    rnl.rmsnorm_linear_bf16(case["x"].cuda(), case["gamma"].cuda(), EPS, w_big, y=y, rstd_out=rstd)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()), "outputs left unwritten"
    cols = sample(N, [K * 2], seed=5 + T, extra=64)
    xb, gb = bits(case["x"]), bits(case["gamma"])
    r = rstd.cpu().numpy()
    assert_rstd(r, O.rms_norm_rows(xb, gb, EPS)[1], f"decode T={T}")
    y32, _, _ = O.rmsnorm_linear_bf16(xb, gb, EPS, bits(rows_of(w_big, cols)), rstd=r)
    assert_bf16_close(f32(y)[:, cols], y32, f"decode T={T}")
    del y, rstd
    free()


def test_mla_prolog_past_2_23_tokens():
    """The MLA prolog's paired norm (query and key-value rows in one launch) at 2^23 + 5 tokens: its grid holds
    one workgroup per token on each of two axes, where a single axis of 2T workgroups of 256 threads would pass
    the 32-bit work-item count of a dispatch."""
    T, K, R, Rkv, N = (1 << 23) + 5, 64, 64, 32, 40
    case = synthetic.mla_case(1, K, R, Rkv, N, seed=46)
    x = synthetic.normal_on_device((T, K), 1.0, seed=46, stream=1)
    W_akv = torch.cat([case["W_a"], case["W_kv"]], dim=0).contiguous().cuda()
    rq = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    rkv = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    qakv = torch.empty((T, R + Rkv), dtype=torch.bfloat16, device="cuda")
    y = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    _, qr, kv = rnl.mla_prolog_bf16(x, W_akv, R, case["gamma"].cuda(), case["gamma_ckv"].cuda(), EPS,
                                    case["W_b"].cuda(), rstd_q_out=rq, rstd_kv_out=rkv, qakv_out=qakv, y=y)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()) and bool((rq > 0).all()) and bool((rkv > 0).all()), "rows left unwritten"
    rows = sample(T, [], seed=6, extra=64)
    sb = bits(rows_of(qakv, rows))
    W_akv_b = np.concatenate([bits(case["W_a"]), bits(case["W_kv"])], axis=0)
    xr = O.bf16_bits_to_f32(bits(rows_of(x, rows)))
    assert_bf16_close(O.bf16_bits_to_f32(sb), O.project_bf16(xr, W_akv_b), "[q_a | kv]")
    qr_b = bits(rows_of(qr, rows))
    check_normed_stage(np.ascontiguousarray(sb[:, :R]), bits(case["gamma"]), rows_of(rq, rows).numpy(), qr_b, "qr")
    check_normed_stage(np.ascontiguousarray(sb[:, R:]), bits(case["gamma_ckv"]), rows_of(rkv, rows).numpy(),
                       bits(rows_of(kv, rows)), "kv")
    assert_bf16_close(f32(rows_of(y, rows)), O.project_bf16(O.bf16_bits_to_f32(qr_b), bits(case["W_b"])), "y")
    del x, qr, kv, rq, rkv, qakv, y
    free()


def test_head_norm_two_grid_rows():
    """The per-head stage with more workgroups than one grid axis row holds (70000 tokens x 32 heads of 128: 70000
    workgroups of 32 heads, the x axis capped at 65536): heads on the second row of the grid are normed too."""
    T, H, D = 70_000, 32, 128
    ld = H * D
    y = synthetic.normal_on_device((T, ld), 2.0, seed=47, stream=1)
    g = synthetic.uniform((D,), 0.5, 1.5, 47, 2)
    c, s = synthetic.rope_tables(T, D // 2, 47)
    rstd = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full_like(y, float("nan"))
    rnl.head_rms_norm_bf16(y, 0, H, D, g.cuda(), EPS, c.cuda(), s.cuda(), out=out, rstd_out=rstd)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()) and bool((rstd > 0).all()), "heads left unwritten"
    rows = sample(T, [], seed=7, extra=40)
    rows = np.union1d(rows, np.arange(65536 - 4, 65536 + 4))  # the first tokens on the grid's second row
    yb, gb = bits(rows_of(y, rows)), bits(g)
    r = rows_of(rstd, rows).numpy()
    cr, sr = c.numpy()[rows], s.numpy()[rows]
    _, r_own = O.head_rms_norm(yb, 0, H, D, gb, EPS, cr, sr)
    assert_rstd(r, r_own, "heads on two grid rows")
    ref, _ = O.head_rms_norm(yb, 0, H, D, gb, EPS, cr, sr, rstd=r)
    ob = bits(rows_of(out, rows))
    assert np.array_equal(ob, ref), f"{int((ob != ref).sum())} head values differ"
    del y, rstd, out
    free()


# The largest token count the library accepts: 2^24 - 1 rows.  Launches with one 256-thread workgroup per row on
# one grid axis (the fp32-weight finalize, the MLA prolog's paired norm) then hold 2^32 - 256 work-items on it.
T_MAX = (1 << 24) - 1


def test_max_tokens_fp32_weights():
    T, K, N = T_MAX, 8, 8
    x = synthetic.normal_on_device((T, K), 1.0, seed=48, stream=1)
    case = synthetic.norm_linear_case(1, K, N, seed=48, gamma=False, w_dtype="fp32")
    y = torch.full((T, N), float("nan"), dtype=torch.float32, device="cuda")
    rstd = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    rnl.rmsnorm_linear_bf16(x, None, EPS, case["W"].cuda(), out_dtype=torch.float32, y=y, rstd_out=rstd)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()) and bool((rstd > 0).all()), "outputs left unwritten"
    rows = sample(T, [], seed=8, extra=64)
    xb = bits(rows_of(x, rows))
    r = rows_of(rstd, rows).numpy()
    assert_rstd(r, O.rms_norm_rows(xb, None, EPS)[1], "fp32 weights, 2^24 - 1 tokens")
    y_ref, _ = O.rmsnorm_linear_fp32w(xb, None, EPS, case["W"].numpy(), rstd=r)
    scale = max(float(np.sqrt(np.mean(y_ref.astype(np.float64) ** 2))), 1e-30)
    err = np.abs(rows_of(y, rows).numpy().astype(np.float64) - y_ref)
    assert (err <= 1e-5 * np.maximum(np.abs(y_ref), scale)).all(), f"max err {err.max():.3g}"
    del x, y, rstd
    free()


def test_max_tokens_mla_prolog():
    T, K, R, Rkv, N = T_MAX, 8, 8, 8, 8
    case = synthetic.mla_case(1, K, R, Rkv, N, seed=49)
    x = synthetic.normal_on_device((T, K), 1.0, seed=49, stream=1)
    W_akv = torch.cat([case["W_a"], case["W_kv"]], dim=0).contiguous().cuda()
    rq = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    rkv = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    qakv = torch.empty((T, R + Rkv), dtype=torch.bfloat16, device="cuda")
    y = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    _, qr, kv = rnl.mla_prolog_bf16(x, W_akv, R, case["gamma"].cuda(), case["gamma_ckv"].cuda(), EPS,
                                    case["W_b"].cuda(), rstd_q_out=rq, rstd_kv_out=rkv, qakv_out=qakv, y=y)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()) and bool((rq > 0).all()) and bool((rkv > 0).all()), "rows left unwritten"
    rows = sample(T, [], seed=9, extra=64)
    sb = bits(rows_of(qakv, rows))
    qr_b = bits(rows_of(qr, rows))
    check_normed_stage(np.ascontiguousarray(sb[:, :R]), bits(case["gamma"]), rows_of(rq, rows).numpy(), qr_b, "qr")
    check_normed_stage(np.ascontiguousarray(sb[:, R:]), bits(case["gamma_ckv"]), rows_of(rkv, rows).numpy(),
                       bits(rows_of(kv, rows)), "kv")
    assert_bf16_close(f32(rows_of(y, rows)), O.project_bf16(O.bf16_bits_to_f32(qr_b), bits(case["W_b"])), "y")
    del x, qr, kv, rq, rkv, qakv, y
    free()


@pytest.mark.parametrize("kind", ["bf16", "int8"])
def test_max_tokens_gemm(kind):
    """2^24 - 1 rows through the norm pre-pass and the tiled GEMM (65536 row tiles)."""
    T, N = T_MAX, 8
    K = 8 if kind == "bf16" else 16
    x = synthetic.normal_on_device((T, K), 1.0, seed=50, stream=1)
    rstd = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    rows = sample(T, [], seed=10, extra=64)
    if kind == "bf16":
        case = synthetic.norm_linear_case(1, K, N, seed=50)
        y = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        rnl.rmsnorm_linear_bf16(x, case["gamma"].cuda(), EPS, case["W"].cuda(), y=y, rstd_out=rstd)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(y).all()) and bool((rstd > 0).all()), "outputs left unwritten"
        xb, gb, r = bits(rows_of(x, rows)), bits(case["gamma"]), rows_of(rstd, rows).numpy()
        assert_rstd(r, O.rms_norm_rows(xb, gb, EPS)[1], "bf16, 2^24 - 1 tokens")
        y32, _, _ = O.rmsnorm_linear_bf16(xb, gb, EPS, bits(case["W"]), rstd=r)
        assert_bf16_close(f32(rows_of(y, rows)), y32, "bf16, 2^24 - 1 tokens")
    else:
        case = synthetic.int8_case(1, K, N, seed=50)
        xq = torch.full((T, K), -128, dtype=torch.int8, device="cuda")
        acc = torch.full((T, N), -(2 ** 31), dtype=torch.int32, device="cuda")
        rnl.rmsnorm_linear_int8(x, case["gamma"].cuda(), EPS, case["Wq"].cuda(), case["w_scale"].cuda(),
                                out_dtype=torch.int32, xq_out=xq, rstd_out=rstd, y=acc)
        torch.cuda.synchronize()
        assert bool((xq != -128).all()) and bool((acc != -(2 ** 31)).all()) and bool((rstd > 0).all())
        xb, gb, r = bits(rows_of(x, rows)), bits(case["gamma"]), rows_of(rstd, rows).numpy()
        assert_rstd(r, O.rms_norm_rows(xb, gb, EPS)[1], "int8, 2^24 - 1 tokens")
        q_ref, _, _ = O.quant_rows(O.rms_norm_rows(xb, gb, EPS, rstd=r)[0])
        q = rows_of(xq, rows).numpy()
        assert np.array_equal(q, q_ref), f"xq not bit-exact ({int((q != q_ref).sum())} differ)"
        assert np.array_equal(rows_of(acc, rows).numpy().astype(np.int64), O.int8_gemm(q, case["Wq"].numpy()))
    free()


@pytest.mark.parametrize("T", [1, 16, 40])
def test_max_width(T):
    """N = 2^24 output columns (the largest the library accepts), K = 8: the single-row kernel, the weight
    streaming kernel (524288 workgroups) and the tiled GEMM."""
    N, K = 1 << 24, 8
    W = synthetic.normal_on_device((N, K), K ** -0.5, seed=51, stream=3)
    case = synthetic.norm_linear_case(T, K, 1, seed=51 + T)
    y = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    rstd = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    rnl.rmsnorm_linear_bf16(case["x"].cuda(), case["gamma"].cuda(), EPS, W, y=y, rstd_out=rstd)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()), "outputs left unwritten"
    cols = sample(N, [], seed=11 + T, extra=80)
    xb, gb, r = bits(case["x"]), bits(case["gamma"]), rstd.cpu().numpy()
    assert_rstd(r, O.rms_norm_rows(xb, gb, EPS)[1], f"N = 2^24, T={T}")
    y32, _, _ = O.rmsnorm_linear_bf16(xb, gb, EPS, bits(rows_of(W, cols)), rstd=r)
    assert_bf16_close(f32(y)[:, cols], y32, f"N = 2^24, T={T}")
    del W, y, rstd
    free()
