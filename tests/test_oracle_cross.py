"""The C oracle against the numpy reference (two independent implementations of
the same definitions) on the same seeded inputs, no GPU needed.

Bit-exact where both evaluate the same fp32 operations (normed values given
rstd, codes, adds, heads, dequant, integer sums).  Where a sum is accumulated in
fp64 and rounded once (the sum of squares and the projections), the two
summation orders (k order in C, pairwise or BLAS-blocked in numpy) differ by a
few fp64 ulps, which can move the fp32 rounding by one ulp only for sums that
sit within that distance of a rounding boundary: at most one fp32 ulp apart,
and only on a small fraction of the values.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synthetic
from tests._util import bits, ulp_diff

C, NP = oracle.c, oracle.numpy_ref
EPS = 1e-6


def _few_one_ulp(a, b, what, frac=1e-3):
    d = ulp_diff(a, b)
    assert d.max() <= 1, f"{what}: {int(d.max())} ulps apart"
    assert (d != 0).mean() <= frac, f"{what}: {(d != 0).mean():.2e} of the values differ"


@pytest.mark.parametrize("T,K", [(64, 4096), (33, 1032), (5, 28672)])
def test_norm(T, K):
    x = bits(synthetic.normal((T, K), 1.0, T, 1))
    g = bits(synthetic.uniform((K,), 0.5, 1.5, T, 2))
    nc, rc = C.rms_norm_rows(x, g, EPS)
    nn, rn = NP.rms_norm_rows(x, g, EPS)
    _few_one_ulp(rc, rn, "rstd", frac=0.05)
    nc2, _ = C.rms_norm_rows(x, g, EPS, rstd=rn)
    assert np.array_equal(nc2, nn)
    for variant in ("A",):
        assert np.array_equal(C.rms_norm_rows(x, g, EPS, rstd=rn, variant=variant)[0], nn)


def test_projections():
    T, K, N = 48, 4096, 640
    a = synthetic.normal((T, K), 1.0, 7, 1).float().numpy()
    W = bits(synthetic.normal((N, K), K ** -0.5, 7, 2))
    _few_one_ulp(C.project_bf16(a, W), NP.project_bf16(a, W), "bf16 projection")
    Wf = synthetic.normal((N, K), K ** -0.5, 7, 3, dtype=synthetic.torch.float32).numpy()
    _few_one_ulp(C.project_fp32(a, Wf), NP.project_fp32(a, Wf), "fp32 projection")


def test_int8_chain():
    case = synthetic.int8_case(40, 4096, 300, seed=9)
    x, g = bits(case["x"]), bits(case["gamma"])
    Wq, ws = case["Wq"].numpy(), case["w_scale"].numpy()
    rstd = NP.rms_norm_rows(x, g, EPS)[1]
    rc = C.rmsnorm_linear_int8(x, g, EPS, Wq, ws, rstd=rstd)
    rn = NP.rmsnorm_linear_int8(x, g, EPS, Wq, ws, rstd=rstd)
    for key in ("q", "x_scale", "acc", "y32", "y_bf16"):
        assert np.array_equal(rc[key], rn[key]), key


def test_add_and_heads():
    T, N, D = 9, 6 * 128, 128
    x = bits(synthetic.normal((T, N), 1.0, 3, 1))
    r = bits(synthetic.normal((T, N), 2.0, 3, 2))
    assert np.array_equal(C.add_residual(x, r), NP.add_residual(x, r))
    g = bits(synthetic.uniform((D,), 0.5, 1.5, 3, 3))
    c, s = synthetic.rope_tables(T, D // 2, 3)
    c, s = c.numpy(), s.numpy()
    _, hr = NP.head_rms_norm(x, 128, 4, D, g, EPS, c, s)
    oc, _ = C.head_rms_norm(x, 128, 4, D, g, EPS, c, s, rstd=hr)
    on, _ = NP.head_rms_norm(x, 128, 4, D, g, EPS, c, s, rstd=hr)
    assert np.array_equal(oc, on)
    n = synthetic.normal((T, D), 1.0, 3, 4).float().numpy()
    assert np.array_equal(C.rope_rotate_half(n, c, s), NP.rope_rotate_half(n, c, s))


def test_mx():
    v = np.random.default_rng(5).standard_normal(20000) * 10.0 ** np.random.default_rng(6).integers(-4, 4, 20000)
    assert np.array_equal(C.e4m3_encode(v), NP.e4m3_encode(v))
    codes = np.arange(256, dtype=np.uint8)
    assert np.array_equal(C.e4m3_decode(codes), NP.e4m3_decode(codes), equal_nan=True)
    assert np.array_equal(C.e8m0_decode(codes), NP.e8m0_decode(codes), equal_nan=True)
    n = synthetic.normal((20, 1024), 1.0, 8, 1).float().numpy()
    qc, sc = C.mx_quant_rows(n)
    qn, sn = NP.mx_quant_rows(n)
    assert np.array_equal(qc, qn) and np.array_equal(sc, sn)
    wq = synthetic.e4m3_codes((70, 1024), 8.0, 8, 2).numpy()
    ws = synthetic.e8m0_codes((70, 16), 117, 119, 8, 3).numpy()
    _few_one_ulp(C.mx_scaled_mm(qc, sc, wq, ws), NP.mx_scaled_mm(qc, sc, wq, ws), "MX scaled product")


def test_chain_and_mla_compose_the_same_steps():
    T, K, R, Rkv, N = 16, 1024, 128, 64, 96
    x = bits(synthetic.normal((T, K), 1.0, 4, 1))
    Wa = bits(synthetic.normal((R, K), K ** -0.5, 4, 2))
    Wkv = bits(synthetic.normal((Rkv, K), K ** -0.5, 4, 3))
    Wb = bits(synthetic.normal((N, R), R ** -0.5, 4, 4))
    g = bits(synthetic.uniform((R,), 0.5, 1.5, 4, 5))
    gkv = bits(synthetic.uniform((Rkv,), 0.5, 1.5, 4, 6))
    qa = NP.norm_proj_chain(x, Wa, g, EPS, Wb)["qa"]
    r = NP.rms_norm_rows(qa, g, EPS)[1]
    oc = C.norm_proj_chain(x, Wa, g, EPS, Wb, rstd=r, qa_bits=qa)
    on = NP.norm_proj_chain(x, Wa, g, EPS, Wb, rstd=r, qa_bits=qa)
    assert np.array_equal(oc["qr"], on["qr"])
    _few_one_ulp(oc["y32"], on["y32"], "chain stage 2")
    mc = C.mla_prolog(x, Wa, g, EPS, Wb, Wkv, gkv)
    mn = NP.mla_prolog(x, Wa, g, EPS, Wb, Wkv, gkv)
    # bf16 values at most one bf16 ulp (2^16 fp32 ulps) apart
    assert ulp_diff(C.bf16_bits_to_f32(mc["kv"]), NP.bf16_bits_to_f32(mn["kv"])).max() <= 1 << 16
