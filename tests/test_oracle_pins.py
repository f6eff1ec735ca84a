"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Each test checks the oracle against something it does not compute itself:
exact rational arithmetic, closed forms, invariants of the definition, special
cases that reduce to a known answer, independent library conversions, and a
hand-derived fixture (tests/golden/int8_quant_ties.txt).  The pages print no
worked numeric example, so no test compares against page values.
"""
from __future__ import annotations

import decimal
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests._util import bits, fraction_to_f32, golden_cases, ulp_diff

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
IMPLS = {"c": oracle.c, "numpy": oracle.numpy_ref}


@pytest.fixture(params=sorted(IMPLS))
def O(request):
    """The oracle under test: the C oracle and the numpy reference each face every pin."""
    return IMPLS[request.param]
RNG = np.random.default_rng(12345)


def _rand_bf16_rows(T, K, seed=0, std=1.0):
    return bits(synthetic.normal((T, K), std, seed, 99))


# ---------------------------------------------------------------------------
# bf16 conversions
# ---------------------------------------------------------------------------
def test_bf16_rne_against_nearest_neighbour(O):
    """Round-to-nearest-even chosen by exact distance to the two bf16 neighbours."""
    raw = RNG.integers(0, 2**32, size=4000, dtype=np.uint64).astype(np.uint32)
    # add exact ties (low half = 0x8000) with both parities of the kept lsb
    ties = (raw[:1000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    vals = np.concatenate([raw, ties]).view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) < 3e38)]
    got = O.f32_to_bf16_bits(vals)
    for v, g in zip(vals[:3000], got[:3000]):
        u = int(np.float32(v).view(np.uint32))
        lo = u & 0xFFFF0000
        hi = lo + 0x10000
        flo = Fraction(float(np.uint32(lo).view(np.float32)))
        fhi = Fraction(float(np.uint32(hi).view(np.float32)))
        fv = Fraction(float(v))
        dlo, dhi = abs(fv - flo), abs(fhi - fv)
        if dlo < dhi or (dlo == dhi and ((lo >> 16) & 1) == 0):
            want = lo >> 16
        else:
            want = hi >> 16
        assert int(g) == want, hex(u)


def test_bf16_conversions_match_torch(O):
    vals = (RNG.standard_normal(20000) * 10.0 ** RNG.integers(-20, 20, 20000)).astype(np.float32)
    ref = bits(torch.from_numpy(vals).to(torch.bfloat16))
    assert np.array_equal(O.f32_to_bf16_bits(vals), ref)
    b = RNG.integers(0, 2**16, 5000, dtype=np.uint64).astype(np.uint16)
    b = b[((b >> 7) & 0xFF) != 0xFF]  # finite only
    want = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(O.bf16_bits_to_f32(b), want)


def test_bf16_nan_stays_nan(O):
    v = np.array([np.nan, -np.nan], dtype=np.float32)
    back = O.bf16_bits_to_f32(O.f32_to_bf16_bits(v))
    assert np.isnan(back).all()


# ---------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------
def _exact_rstd(x_row_f32, eps):
    """rstd from exact rationals (sum of squares exact) and 60-digit decimals,
    following the stated roundings: fl(S), fl(S*fl(1/K)), fl(ms+eps)."""
    K = len(x_row_f32)
    S = sum(Fraction(float(v)) ** 2 for v in x_row_f32)
    S32 = fraction_to_f32(S)
    c = fraction_to_f32(Fraction(1, K))
    ms = fraction_to_f32(Fraction(float(S32)) * Fraction(float(c)))
    var = fraction_to_f32(Fraction(float(ms)) + Fraction(float(np.float32(eps))))
    with decimal.localcontext() as ctx:
        ctx.prec = 60
        r = decimal.Decimal(1) / decimal.Decimal(float(var)).sqrt()
    return Fraction(r)


@pytest.mark.parametrize("K", [256, 1536, 4104])
def test_rstd_within_one_ulp_of_exact(O, K):
    x = _rand_bf16_rows(24, K, seed=K)
    _, rstd = O.rms_norm_rows(x, None, 1e-6)
    xf = O.bf16_bits_to_f32(x)
    for t in range(x.shape[0]):
        exact = _exact_rstd(xf[t], 1e-6)
        assert ulp_diff(rstd[t], fraction_to_f32(exact)) <= 1


def test_rsqrt_and_sqrt_div_variants_agree(O):
    """AT-10 page section 3: variant A (rsqrt) and B (sqrt + div) agree."""
    for K in (8, 256, 1000, 4096):
        x = _rand_bf16_rows(2500 if K <= 1000 else 300, K, seed=K + 1)
        _, ra = O.rms_norm_rows(x, None, 1e-6, variant="A")
        _, rb = O.rms_norm_rows(x, None, 1e-6, variant="B")
        assert ulp_diff(ra, rb).max() <= 1


def test_division_form_matches_product_form(O):
    """Golden ``rms_norm_new`` divides by sqrt; the kernel multiplies by rstd."""
    x = _rand_bf16_rows(64, 4096, seed=7)
    n, _ = O.rms_norm_rows(x, None, 1e-6)
    nd = O.rms_norm_rows_golden_div(x, 1e-6)
    assert ulp_diff(n, nd).max() <= 2


def test_mla_ordering_equivalent(O):
    """1/D applied per element before the sum (MLA code) vs after (variant A)."""
    for K in (256, 4096):  # power of two: scaling by 1/K is exact
        x = _rand_bf16_rows(200, K, seed=K + 3)
        _, r1 = O.rms_norm_rows(x, None, 1e-6)
        _, r2 = O.rms_norm_rows_mla_order(x, 1e-6)
        assert np.array_equal(r1, r2)
    x = _rand_bf16_rows(200, 1536, seed=11)
    _, r1 = O.rms_norm_rows(x, None, 1e-6)
    _, r2 = O.rms_norm_rows_mla_order(x, 1e-6)
    assert ulp_diff(r1, r2).max() <= 4


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.5, 3.0])
def test_unit_rms_invariant(O, eps):
    """With gamma = 1: rms(n) = sqrt(ms / (ms + eps)); exactly 1 when eps = 0."""
    x = _rand_bf16_rows(128, 2048, seed=5)
    n, _ = O.rms_norm_rows(x, None, eps)
    xf = O.bf16_bits_to_f32(x).astype(np.float64)
    ms = np.mean(xf * xf, axis=1)
    want = np.sqrt(ms / (ms + eps))
    got = np.sqrt(np.mean(n.astype(np.float64) ** 2, axis=1))
    assert np.max(np.abs(got / want - 1.0)) < 5e-7


def test_scale_invariance_eps0(O):
    """eps = 0: scaling x by 2^p leaves n unchanged bit for bit."""
    x = _rand_bf16_rows(64, 512, seed=9)
    n0, _ = O.rms_norm_rows(x, None, 0.0)
    xf = O.bf16_bits_to_f32(x)
    for p in (-6, -1, 3, 9):
        xs = O.f32_to_bf16_bits((xf * np.float32(2.0**p)).astype(np.float32))
        n1, _ = O.rms_norm_rows(xs, None, 0.0)
        assert np.array_equal(n0, n1)


@pytest.mark.parametrize("c", [1.0, -0.375, 3.25, 1e-3])
@pytest.mark.parametrize("eps", [1e-6, 0.25])
def test_constant_row_closed_form(O, c, eps):
    """x_k = c for all k: n = c / sqrt(c^2 + eps)."""
    cb = O.f32_to_bf16_bits(np.array([c], dtype=np.float32))[0]
    cf = float(O.bf16_bits_to_f32(np.array([cb]))[0])
    x = np.full((1, 64), cb, dtype=np.uint16)
    n, _ = O.rms_norm_rows(x, None, eps)
    want = np.float32(cf / np.sqrt(cf * cf + float(np.float32(eps))))
    assert ulp_diff(n[0], np.full(64, want, dtype=np.float32)).max() <= 2


def test_gamma_scales_columns(O):
    """gamma = 2^j_k per column multiplies column k exactly and leaves rstd alone."""
    K = 64
    x = _rand_bf16_rows(16, K, seed=21)
    j = (np.arange(K) % 7) - 3
    g = O.f32_to_bf16_bits((2.0 ** j).astype(np.float32))
    n0, r0 = O.rms_norm_rows(x, None, 1e-6)
    n1, r1 = O.rms_norm_rows(x, g, 1e-6)
    assert np.array_equal(r0, r1)
    assert np.array_equal(n1, (n0 * (2.0 ** j)[None, :]).astype(np.float32))


def test_gamma_after_rstd_each_product_rounded(O):
    """Reading R5 (AT-10 page section 5: rms_norm gives the normed rows, gamma multiplies them after): each
    normed value is fl(fl(x * rstd) * gamma), two correctly rounded products in that order.  Checked with exact
    rationals on rows where the other order, fl(fl(x * gamma) * rstd), differs somewhere."""
    T, K = 6, 64
    x = _rand_bf16_rows(T, K, seed=23)
    g = bits(synthetic.uniform((K,), 0.5, 1.5, 23, 2))
    r = np.random.default_rng(23).uniform(0.3, 3.0, T).astype(np.float32)
    n, _ = O.rms_norm_rows(x, g, 1e-6, rstd=r)
    xf, gf = O.bf16_bits_to_f32(x), O.bf16_bits_to_f32(g)
    other = 0
    for t in range(T):
        for k in range(K):
            xr = fraction_to_f32(Fraction(float(xf[t, k])) * Fraction(float(r[t])))
            want = fraction_to_f32(Fraction(float(xr)) * Fraction(float(gf[k])))
            assert n[t, k] == want, (t, k)
            xg = fraction_to_f32(Fraction(float(xf[t, k])) * Fraction(float(gf[k])))
            other += int(fraction_to_f32(Fraction(float(xg)) * Fraction(float(r[t]))) != want)
    assert other > 0, "the rows do not separate the two orders"


def test_given_rstd_is_used(O):
    x = _rand_bf16_rows(4, 32, seed=2)
    r = np.array([0.5, 1.0, 2.0, 0.25], dtype=np.float32)
    n, r2 = O.rms_norm_rows(x, None, 1e-6, rstd=r)
    assert np.array_equal(r2, r)
    assert np.array_equal(n, (O.bf16_bits_to_f32(x) * r[:, None]).astype(np.float32))


# ---------------------------------------------------------------------------
# projections
# ---------------------------------------------------------------------------
def _exact_proj(a_f32, w_f32):
    T, K = a_f32.shape
    N = w_f32.shape[0]
    out = np.zeros((T, N), dtype=np.float32)
    af = [[Fraction(float(v)) for v in row] for row in a_f32]
    wf = [[Fraction(float(v)) for v in row] for row in w_f32]
    for t in range(T):
        for j in range(N):
            out[t, j] = fraction_to_f32(sum(af[t][k] * wf[j][k] for k in range(K)))
    return out


@pytest.mark.parametrize("T,K,N", [(3, 16, 5), (5, 40, 7), (2, 64, 3)])
def test_bf16_projection_is_correctly_rounded(O, T, K, N):
    case = synthetic.norm_linear_case(T, K, N, seed=T * K + N)
    x, g, W = bits(case["x"]), bits(case["gamma"]), bits(case["W"])
    y32, ybf, _ = O.rmsnorm_linear_bf16(x, g, 1e-6, W)
    n, _ = O.rms_norm_rows(x, g, 1e-6)
    a = O.bf16_bits_to_f32(O.f32_to_bf16_bits(n))
    want = _exact_proj(a, O.bf16_bits_to_f32(W))
    assert np.array_equal(y32, want)
    assert np.array_equal(ybf, O.f32_to_bf16_bits(want))


def test_bf16_projection_identity_weight(O):
    """W = I: y = bf16(n) exactly."""
    K = 48
    x = _rand_bf16_rows(6, K, seed=4)
    g = bits(synthetic.uniform((K,), 0.5, 1.5, 0, 7))
    I = O.f32_to_bf16_bits(np.eye(K, dtype=np.float32))
    y32, ybf, _ = O.rmsnorm_linear_bf16(x, g, 1e-6, I)
    n, _ = O.rms_norm_rows(x, g, 1e-6)
    assert np.array_equal(ybf, O.f32_to_bf16_bits(n))


def test_bf16_projection_selects_weight_rows(O):
    """W[j, k_j] = 1 (N != K): y[:, j] = a[:, k_j] -- catches a transposed W."""
    T, K, N = 5, 32, 9
    x = _rand_bf16_rows(T, K, seed=6)
    kj = RNG.permutation(K)[:N]
    Wf = np.zeros((N, K), dtype=np.float32)
    Wf[np.arange(N), kj] = 1.0
    y32, _, _ = O.rmsnorm_linear_bf16(x, None, 1e-6, O.f32_to_bf16_bits(Wf))
    n, _ = O.rms_norm_rows(x, None, 1e-6)
    a = O.bf16_bits_to_f32(O.f32_to_bf16_bits(n))
    assert np.array_equal(y32, a[:, kj])


def test_bf16_projection_square_permutation(O):
    """Square W = permutation matrix P (not symmetric): y = a @ P.T, so
    y[:, j] = a[:, perm[j]]; a transposed W would give the inverse permutation."""
    K = 16
    x = _rand_bf16_rows(4, K, seed=8)
    perm = np.roll(np.arange(K), 3)
    Wf = np.zeros((K, K), dtype=np.float32)
    Wf[np.arange(K), perm] = 1.0
    y32, _, _ = O.rmsnorm_linear_bf16(x, None, 1e-6, O.f32_to_bf16_bits(Wf))
    n, _ = O.rms_norm_rows(x, None, 1e-6)
    a = O.bf16_bits_to_f32(O.f32_to_bf16_bits(n))
    assert np.array_equal(y32, a[:, perm])


def test_fp32_projection_exact_and_keeps_fp32(O):
    """mhc_pre FP32 compute: normed rows are not cast to bf16."""
    T, K, N = 3, 24, 4
    case = synthetic.norm_linear_case(T, K, N, seed=3, gamma=False, w_dtype="fp32")
    x, W = bits(case["x"]), case["W"].numpy()
    y32, _ = O.rmsnorm_linear_fp32w(x, None, 1e-6, W)
    n, _ = O.rms_norm_rows(x, None, 1e-6)
    assert np.array_equal(y32, _exact_proj(n, W))
    yI, _ = O.rmsnorm_linear_fp32w(x, None, 1e-6, np.eye(K, dtype=np.float32))
    assert np.array_equal(yI, n)
    assert not np.array_equal(n, O.bf16_bits_to_f32(O.f32_to_bf16_bits(n)))


# ---------------------------------------------------------------------------
# int8 W8A8
# ---------------------------------------------------------------------------
def test_int8_quant_golden_ties(O):
    for c in golden_cases(os.path.join(GOLDEN, "int8_quant_ties.txt")):
        x = O.f32_to_bf16_bits(np.array(c["x"], dtype=np.float32))
        g = O.f32_to_bf16_bits(np.array(c["gamma"], dtype=np.float32))
        # the fixture's values must be bf16-exact
        assert np.array_equal(O.bf16_bits_to_f32(x), np.array(c["x"], dtype=np.float32))
        assert np.array_equal(O.bf16_bits_to_f32(g), np.array(c["gamma"], dtype=np.float32))
        n, _ = O.rms_norm_rows(x, g, c["eps"])
        q, xs, _ = O.quant_rows(n)
        assert np.array_equal(q, np.array(c["q"], dtype=np.int8)), c["name"]
        assert np.array_equal(xs, np.array(c["x_scale"], dtype=np.float32)), c["name"]


def test_int8_saturation_rule(O):
    n = np.array([[1.0, -1.0, 0.5, 0.63, -0.0]], dtype=np.float32)
    q = O.quant_values(n, np.array([[200.0]], dtype=np.float32))
    assert q.tolist() == [[127, -127, 100, 126, 0]]


def test_int8_quant_invariants(O):
    case = synthetic.int8_case(64, 512, 8, seed=1)
    n, _ = O.rms_norm_rows(bits(case["x"]), bits(case["gamma"]), 1e-6)
    q, xs, s = O.quant_rows(n)
    assert q.dtype == np.int8 and np.abs(q.astype(int)).max() <= 127
    amax_idx = np.argmax(np.abs(n), axis=1)
    assert np.array_equal(np.abs(q[np.arange(64), amax_idx]).astype(int), np.full(64, 127))
    # reconstruction error is at most half a step (plus fp32 slack)
    err = np.abs(q.astype(np.float64) * xs[:, None] - n)
    assert np.all(err <= xs[:, None] * (0.5 + 1e-5))
    # scale multiplier and dequant scale are the pages' 127/amax and amax/127
    amax = np.abs(n).max(axis=1).astype(np.float64)
    assert np.max(np.abs(s / (127.0 / amax) - 1)) <= 2**-24
    assert np.max(np.abs(xs / (amax / 127.0) - 1)) <= 2**-24


def test_int8_gemm_brute_force_and_unit_rows(O):
    T, K, N = 4, 32, 6
    q = RNG.integers(-127, 128, (T, K)).astype(np.int8)
    Wq = RNG.integers(-127, 128, (N, K)).astype(np.int8)
    acc = O.int8_gemm(q, Wq)
    for t in range(T):
        for j in range(N):
            assert acc[t, j] == sum(int(q[t, k]) * int(Wq[j, k]) for k in range(K))
    sel = RNG.permutation(K)[:N]
    E = np.zeros((N, K), dtype=np.int8)
    E[np.arange(N), sel] = 1
    assert np.array_equal(O.int8_gemm(q, E), q[:, sel].astype(np.int64))


def test_int8_gemm_fp64_form_is_exact(O):
    """The fp64 evaluation equals the int64 sum, also at the extremes: every product +-127^2 or -128 * 127 over
    K = 132096, the longest row for which 128 * 127 * K still fits int32 (all partial sums stay far below 2^53),
    and random codes at K = 4096."""
    K = 132096
    for a, b in ((127, 127), (-127, 127), (-128, 127), (127, -128)):
        q = np.full((2, K), a, dtype=np.int8)
        Wq = np.full((3, K), b, dtype=np.int8)
        assert np.array_equal(O.int8_gemm(q, Wq), O.int8_gemm_int64(q, Wq))
        assert O.int8_gemm(q, Wq)[0, 0] == a * b * K
    q = RNG.integers(-127, 128, (40, 4096)).astype(np.int8)
    Wq = RNG.integers(-128, 128, (70, 4096)).astype(np.int8)
    assert np.array_equal(O.int8_gemm(q, Wq), O.int8_gemm_int64(q, Wq))


def test_int8_gemm_overflow_detected(O):
    K = 133160  # K * 127 * 127 > 2^31 - 1
    q = np.full((1, K), 127, dtype=np.int8)
    with pytest.raises(OverflowError):
        O.int8_gemm(q, q)


def test_dequant_closed_form(O):
    """w_scale = 2^-k, x_scale exact: y = float(acc) * x_scale * w_scale exactly,
    with the int -> fp32 cast rounding acc above 2^24."""
    acc = np.array([[3, -5, 2**24 + 1, 2**25 + 3]], dtype=np.int64)
    xs = np.array([0.015625], dtype=np.float32)
    ws = np.array([2.0**-3, 2.0**-7, 2.0**-1, 1.0], dtype=np.float32)
    y = O.dequant(acc, xs, ws)
    want = np.array([[3 / 512, -5 / 8192, 2**24 / 128, (2**25 + 4) / 64]], dtype=np.float32)
    assert np.array_equal(y, want)


def test_dequant_rounding_order(O):
    """SK-14 page, QuantMatMulReduceSum: scale_mul = x1_scale * x2_scale is
    formed first (one rounding), then acc_fp32 * scale_mul (one rounding).
    Expected values from exact rationals with those two roundings."""
    acc = RNG.integers(-2**20, 2**20, (6, 40)).astype(np.int64)
    xs = RNG.uniform(1e-3, 1e-1, 6).astype(np.float32)
    ws = RNG.uniform(1e-3, 1e-2, 40).astype(np.float32)
    y = O.dequant(acc, xs, ws)
    diff = 0
    for t in range(6):
        for j in range(40):
            sm = fraction_to_f32(Fraction(float(xs[t])) * Fraction(float(ws[j])))
            want = fraction_to_f32(Fraction(int(acc[t, j])) * Fraction(float(sm)))
            assert y[t, j] == want
            step = fraction_to_f32(Fraction(int(acc[t, j])) * Fraction(float(xs[t])))
            other = fraction_to_f32(Fraction(float(step)) * Fraction(float(ws[j])))
            diff += int(other != want)
    assert diff > 0  # the two orders are distinguishable on this data


def test_int8_zero_row(O):
    x = np.zeros((2, 16), dtype=np.uint16)
    Wq = RNG.integers(-127, 128, (3, 16)).astype(np.int8)
    r = O.rmsnorm_linear_int8(x, None, 1e-6, Wq, np.ones(3, dtype=np.float32))
    assert (r["q"] == 0).all() and (r["x_scale"] == 0).all() and (r["y32"] == 0).all()


# ---------------------------------------------------------------------------
# chain
# ---------------------------------------------------------------------------
def test_chain_identity_stages(O):
    """W_a = I: q_a = x, qr = bf16(norm(x)); W_b = I: y = qr."""
    K = 32
    x = _rand_bf16_rows(5, K, seed=13)
    g = bits(synthetic.uniform((K,), 0.5, 1.5, 0, 8))
    I = O.f32_to_bf16_bits(np.eye(K, dtype=np.float32))
    r = O.norm_proj_chain(x, I, g, 1e-6, I)
    assert np.array_equal(r["qa"], x)
    n, _ = O.rms_norm_rows(x, g, 1e-6)
    assert np.array_equal(r["qr"], O.f32_to_bf16_bits(n))
    assert np.array_equal(r["y_bf16"], r["qr"])


def test_chain_stage_one_exact(O):
    case = synthetic.chain_case(3, 24, 16, 5, seed=2)
    x, Wa, g, Wb = (bits(case[k]) for k in ("x", "W_a", "gamma", "W_b"))
    r = O.norm_proj_chain(x, Wa, g, 1e-6, Wb)
    qa32 = _exact_proj(O.bf16_bits_to_f32(x), O.bf16_bits_to_f32(Wa))
    assert np.array_equal(r["qa"], O.f32_to_bf16_bits(qa32))
    y = _exact_proj(O.bf16_bits_to_f32(r["qr"]), O.bf16_bits_to_f32(Wb))
    assert np.array_equal(r["y32"], y)


# ---------------------------------------------------------------------------
# residual add before the norm
# ---------------------------------------------------------------------------
def _fraction_to_bf16_bits(fr: Fraction) -> int:
    """Nearest-even bf16 (8 significant bits) of an exact rational, from the
    definition of the format (normal range only), as a bit pattern."""
    if fr == 0:
        return 0
    sign = 0x8000 if fr < 0 else 0
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    m = a / Fraction(2) ** (e - 7)  # in [2^7, 2^8)
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    if fl == 256:  # rounded up to the next binade
        fl, e = 128, e + 1
    return sign | ((e + 127) << 7) | (fl - 128)


def test_add_residual_is_correctly_rounded_sum(O):
    """Two bf16 values whose exponents differ by at most 15 add exactly in fp32, so
    x_add must be the nearest-even bf16 of the exact sum."""
    x = _rand_bf16_rows(6, 64, seed=21)
    r = _rand_bf16_rows(6, 64, seed=22, std=0.3)
    got = O.add_residual(x, r)
    xf, rf = O.bf16_bits_to_f32(x), O.bf16_bits_to_f32(r)
    checked = 0
    for a, b, g in zip(xf.ravel(), rf.ravel(), got.ravel()):
        if a == 0 or b == 0 or abs(np.frexp(a)[1] - np.frexp(b)[1]) > 15:
            continue
        s = Fraction(float(a)) + Fraction(float(b))
        assert int(g) == _fraction_to_bf16_bits(s), (a, b)
        checked += 1
    assert checked > 300


def test_add_residual_ties_round_to_even(O):
    """1 + 2^-8 and 1 + 3 * 2^-8 are halfway between bf16 neighbours: the first rounds
    down to 1 (even), the second up to 1 + 2^-6."""
    one, half_ulp, three_half = (int(O.f32_to_bf16_bits(np.float32(v))[0]) for v in (1.0, 2.0 ** -8, 3 * 2.0 ** -8))
    got = O.add_residual(np.array([[one, one]], dtype=np.uint16), np.array([[half_ulp, three_half]], dtype=np.uint16))
    assert O.bf16_bits_to_f32(got).tolist() == [[1.0, 1.0 + 2.0 ** -6]]


def test_add_residual_zero_and_negation(O):
    case = synthetic.norm_linear_case(5, 96, 7, seed=3)
    x, g, W = bits(case["x"]), bits(case["gamma"]), bits(case["W"])
    zero = np.zeros_like(x)
    xa, y32, ybf, rstd = O.add_rmsnorm_linear_bf16(x, zero, g, 1e-6, W)
    ref32, refbf, refr = O.rmsnorm_linear_bf16(x, g, 1e-6, W)
    assert np.array_equal(xa, x) and np.array_equal(y32, ref32) and np.array_equal(rstd, refr)
    neg = x ^ np.uint16(0x8000)
    xa, y32, _, _ = O.add_rmsnorm_linear_bf16(x, neg, g, 1e-6, W)
    assert not np.any(O.bf16_bits_to_f32(xa)) and not np.any(y32)
    q = O.add_rmsnorm_linear_int8(x, neg, g, 1e-6, synthetic.int8_uniform((7, 96), 0, 3).numpy(),
                                  np.ones(7, dtype=np.float32))
    assert not q["q"].any() and not q["x_scale"].any()


def test_add_residual_commutes(O):
    x = _rand_bf16_rows(4, 32, seed=30)
    r = _rand_bf16_rows(4, 32, seed=31)
    assert np.array_equal(O.add_residual(x, r), O.add_residual(r, x))


# ---------------------------------------------------------------------------
# post-projection stage: per-head RMSNorm and rotary embedding
# ---------------------------------------------------------------------------
def _angles(T, half, seed):
    phi = np.random.default_rng(seed).uniform(0.0, 2.0 * np.pi, size=(T, half))
    return np.cos(phi).astype(np.float32), np.sin(phi).astype(np.float32)


def test_head_norm_matches_per_head_loop(O):
    """Head (t, h) is the norm of its own D columns, rotated by token t's angles, and
    nothing else: a loop over tokens and heads gives the same bits."""
    T, D, H, col0, N = 5, 16, 3, 8, 64
    y = _rand_bf16_rows(T, N, seed=40, std=3.0)
    g = bits(synthetic.uniform((D,), 0.5, 1.5, 4, 2))
    c, s = _angles(T, D // 2, 41)
    out, r = O.head_rms_norm(y, col0, H, D, g, 1e-6, c, s)
    assert r.shape == (T, H)
    for t in range(T):
        for h in range(H):
            a = col0 + h * D
            n, rr = O.rms_norm_rows(y[t:t + 1, a:a + D], g, 1e-6)
            want = O.f32_to_bf16_bits(O.rope_rotate_half(n, c[t:t + 1], s[t:t + 1]))[0]
            assert np.array_equal(out[t, a:a + D], want), (t, h)
            assert r[t, h] == rr[0]


def test_head_norm_leaves_other_columns(O):
    T, D, H, col0, N = 4, 32, 2, 32, 128
    y = _rand_bf16_rows(T, N, seed=42)
    out, _ = O.head_rms_norm(y, col0, H, D, None, 1e-6)
    assert np.array_equal(out[:, :col0], y[:, :col0])
    assert np.array_equal(out[:, col0 + H * D:], y[:, col0 + H * D:])
    assert not np.array_equal(out[:, col0:col0 + H * D], y[:, col0:col0 + H * D])


def test_head_norm_heads_are_independent(O):
    """eps = 0: scaling one head by 2^p changes no output bit; zeroing a head zeroes
    that head only."""
    T, D, H = 6, 64, 4
    y = _rand_bf16_rows(T, H * D, seed=43)
    out0, _ = O.head_rms_norm(y, 0, H, D, None, 0.0)
    yf = O.bf16_bits_to_f32(y).copy()
    yf[:, 2 * D:3 * D] *= np.float32(2.0 ** 5)
    out1, _ = O.head_rms_norm(O.f32_to_bf16_bits(yf), 0, H, D, None, 0.0)
    assert np.array_equal(out0, out1)
    yz = y.copy()
    yz[3, D:2 * D] = 0
    out2, _ = O.head_rms_norm(yz, 0, H, D, None, 1e-6)
    assert not O.bf16_bits_to_f32(out2[3, D:2 * D]).any()
    mask = np.ones_like(y, dtype=bool)
    mask[3, D:2 * D] = False
    out3, _ = O.head_rms_norm(y, 0, H, D, None, 1e-6)
    assert np.array_equal(out2[mask], out3[mask])


def test_head_norm_constant_head_closed_form(O):
    """A head of constant c normed with eps: every value is c / sqrt(c^2 + eps), times gamma."""
    D = 32
    c = 0.75
    y = np.full((1, 2 * D), O.f32_to_bf16_bits(np.float32(c))[0], dtype=np.uint16)
    g = O.f32_to_bf16_bits(np.full(D, 2.0, dtype=np.float32))
    out, _ = O.head_rms_norm(y, 0, 2, D, g, 0.25)
    want = 2.0 * c / np.sqrt(c * c + 0.25)  # 1.5 / sqrt(0.8125) = 1.664..., bf16 1.6640625
    assert O.bf16_bits_to_f32(out).tolist() == [[float(O.bf16_bits_to_f32(O.f32_to_bf16_bits(np.float32(want)))[0])] * (2 * D)]


def test_rope_identity_and_half_turn(O):
    n = O.bf16_bits_to_f32(_rand_bf16_rows(3, 16, seed=44)).astype(np.float32)
    one, zero = np.ones((3, 8), np.float32), np.zeros((3, 8), np.float32)
    assert np.array_equal(O.rope_rotate_half(n, one, zero), n)
    assert np.array_equal(O.rope_rotate_half(n, -one, zero), -n)


def test_rope_quarter_turn_pairs_i_with_i_plus_half(O):
    """cos = 0, sin = 1 maps (a_i, b_i) = (n[i], n[i + D/2]) to (-b_i, a_i): this fixes
    both the pairing and the sign."""
    n = np.arange(1, 17, dtype=np.float32).reshape(1, 16)
    out = O.rope_rotate_half(n, np.zeros((1, 8), np.float32), np.ones((1, 8), np.float32))
    assert out.tolist() == [[-9, -10, -11, -12, -13, -14, -15, -16, 1, 2, 3, 4, 5, 6, 7, 8]]


def test_rope_is_a_rotation(O):
    """Each pair keeps its length, and rotating by phi then by -phi returns the input,
    within a few fp32 roundings."""
    n = O.bf16_bits_to_f32(_rand_bf16_rows(8, 64, seed=45)).astype(np.float32)
    c, s = _angles(8, 32, 46)
    out = O.rope_rotate_half(n, c, s)
    len_in = n[:, :32].astype(np.float64) ** 2 + n[:, 32:].astype(np.float64) ** 2
    len_out = out[:, :32].astype(np.float64) ** 2 + out[:, 32:].astype(np.float64) ** 2
    assert np.max(np.abs(len_out / len_in - 1.0)) < 4e-7
    back = O.rope_rotate_half(out, c, -s)
    assert np.max(np.abs(back - n)) <= 4e-7 * np.max(np.abs(n))
    # two rotations add their angles
    phi = np.random.default_rng(47).uniform(0, 2 * np.pi, size=(8, 32))
    c1, s1 = np.cos(phi).astype(np.float32), np.sin(phi).astype(np.float32)
    c2, s2 = np.cos(2 * phi).astype(np.float32), np.sin(2 * phi).astype(np.float32)
    twice = O.rope_rotate_half(O.rope_rotate_half(n, c1, s1), c1, s1)
    assert np.max(np.abs(twice - O.rope_rotate_half(n, c2, s2))) <= 2e-6 * np.max(np.abs(n))


def test_preattn_split_and_gammas(O):
    """V columns are the projection output; gamma_q acts on the query heads only and
    gamma_k on the key heads only (gamma_k = 2 doubles the key heads exactly)."""
    T, K, Hq, Hkv, D = 4, 64, 4, 2, 16
    N = (Hq + 2 * Hkv) * D
    case = synthetic.norm_linear_case(T, K, N, seed=48)
    x, g, W = bits(case["x"]), bits(case["gamma"]), bits(case["W"])
    ones = O.f32_to_bf16_bits(np.ones(D, np.float32))
    twos = O.f32_to_bf16_bits(np.full(D, 2.0, np.float32))
    a = O.preattn_qkv(x, None, g, 1e-6, W, Hq, Hkv, D, ones, ones, 1e-6)
    b = O.preattn_qkv(x, None, g, 1e-6, W, Hq, Hkv, D, ones, twos, 1e-6)
    q, k = slice(0, Hq * D), slice(Hq * D, (Hq + Hkv) * D)
    v = slice((Hq + Hkv) * D, N)
    assert np.array_equal(a["y"][:, v], a["y_proj"][:, v])
    assert np.array_equal(a["y"][:, q], b["y"][:, q])
    assert np.array_equal(O.bf16_bits_to_f32(b["y"][:, k]), 2 * O.bf16_bits_to_f32(a["y"][:, k]))
    _, ybf, _ = O.rmsnorm_linear_bf16(x, g, 1e-6, W)
    assert np.array_equal(a["y_proj"], ybf)
    # a zero residual changes nothing
    z = O.preattn_qkv(x, np.zeros_like(x), g, 1e-6, W, Hq, Hkv, D, ones, twos, 1e-6)
    assert np.array_equal(z["y"], b["y"]) and np.array_equal(z["x_add"], x)


# ---------------------------------------------------------------------------
# MLA prolog: the KV branch beside the query chain
# ---------------------------------------------------------------------------
def _mla_inputs(T, K, R, Rkv, N, seed):
    x = _rand_bf16_rows(T, K, seed=seed)
    Wa = bits(synthetic.normal((R, K), K ** -0.5, seed, 5))
    Wb = bits(synthetic.normal((N, R), R ** -0.5, seed, 6))
    gq = bits(synthetic.uniform((R,), 0.5, 1.5, seed, 2))
    gkv = bits(synthetic.uniform((Rkv,), 0.5, 1.5, seed, 8))
    return x, Wa, Wb, gq, gkv


def test_mla_kv_branch_selection_weight(O):
    """W_kv = [I | 0] selects the first Rkv columns of x exactly (products with 1 and
    0 are exact), so kv is x[:, :Rkv] and kv_out is the norm of those columns."""
    T, K, R, Rkv, N = 6, 96, 32, 48, 40
    x, Wa, Wb, gq, gkv = _mla_inputs(T, K, R, Rkv, N, 50)
    sel = np.zeros((Rkv, K), dtype=np.float32)
    sel[np.arange(Rkv), np.arange(Rkv)] = 1.0
    out = O.mla_prolog(x, Wa, gq, 1e-6, Wb, O.f32_to_bf16_bits(sel), gkv)
    assert np.array_equal(out["kv"], x[:, :Rkv])
    n, r = O.rms_norm_rows(x[:, :Rkv], gkv, 1e-6)
    assert np.array_equal(out["kv_out"], O.f32_to_bf16_bits(n)) and np.array_equal(out["rstd_kv"], r)


def test_mla_kv_branch_permuted_weight(O):
    """A permutation weight permutes the kv columns; with gamma_ckv permuted the same
    way the normed row is the permutation of the unpermuted one."""
    T, K, R, N = 4, 64, 16, 8
    x, Wa, Wb, gq, _ = _mla_inputs(T, K, R, K, N, 51)
    perm = np.random.default_rng(52).permutation(K)
    P = np.zeros((K, K), dtype=np.float32)
    P[np.arange(K), perm] = 1.0
    g = bits(synthetic.uniform((K,), 0.5, 1.5, 51, 9))
    a = O.mla_prolog(x, Wa, gq, 1e-6, Wb, O.f32_to_bf16_bits(P), g[perm])
    n, _ = O.rms_norm_rows(x, g, 1e-6)
    assert np.array_equal(a["kv"], x[:, perm])
    assert np.array_equal(a["kv_out"], O.f32_to_bf16_bits(n)[:, perm])


def test_mla_query_outputs_unchanged_by_kv_branch(O):
    T, K, R, Rkv, N = 5, 128, 32, 24, 20
    x, Wa, Wb, gq, gkv = _mla_inputs(T, K, R, Rkv, N, 53)
    Wkv = bits(synthetic.normal((Rkv, K), K ** -0.5, 53, 7))
    out = O.mla_prolog(x, Wa, gq, 1e-6, Wb, Wkv, gkv)
    ref = O.norm_proj_chain(x, Wa, gq, 1e-6, Wb)
    for k in ("qa", "qr", "y_bf16", "rstd"):
        assert np.array_equal(out[k], ref[k]), k


# ---------------------------------------------------------------------------
# MXFP8: E4M3 elements, E8M0 scales, 64-element blocks
# ---------------------------------------------------------------------------
def test_e4m3_decode_table(O):
    """Values fixed by the E4M3 (FN) format: bias 7, 3 mantissa bits, subnormals
    below 2^-6, largest normal 448, NaN at S.1111.111, no infinities."""
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6,
             0x30: 0.5, 0x38: 1.0, 0x39: 1.125, 0x40: 2.0, 0x77: 240.0, 0x78: 256.0, 0x7E: 448.0,
             0xB8: -1.0, 0xFE: -448.0}
    for code, val in known.items():
        assert float(O.e4m3_decode(np.array([code], dtype=np.uint8))[0]) == val, hex(code)
    assert np.isnan(O.e4m3_decode(np.array([0x7F, 0xFF], dtype=np.uint8))).all()
    v = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    fin = v[~np.isnan(v)]
    assert len(fin) == 254 and np.max(np.abs(fin)) == 448.0


def _e4m3_table(O):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], dtype=np.uint8)
    return codes, O.e4m3_decode(codes).astype(np.float64)


def test_e4m3_encode_is_nearest_even_and_saturates(O):
    """Brute force: the code chosen is the nearest finite E4M3 value; at an exact
    midpoint the even mantissa wins; beyond 448 the value clamps to 448."""
    codes, vals = _e4m3_table(O)
    rng = np.random.default_rng(60)
    x = np.concatenate([rng.normal(0, 40, 4000), rng.uniform(-2.0 ** -6, 2.0 ** -6, 500),
                        [500.0, -1e6, 464.0, 449.0]])
    # midpoints between neighbouring positive values
    pos = np.sort(vals[vals > 0])
    mids = (pos[:-1] + pos[1:]) / 2
    x = np.concatenate([x, mids, -mids]).astype(np.float32)
    got = O.e4m3_encode(x)
    gv = O.e4m3_decode(got).astype(np.float64)
    for xi, g, gc in zip(x.astype(np.float64), gv, got):
        if abs(xi) >= 448.0:
            assert g == np.sign(xi) * 448.0
            continue
        d = np.abs(vals - xi)
        best = np.min(d)
        assert abs(g - xi) == best, (xi, g)
        ties = codes[d == best]
        if len(ties) > 1:
            assert (int(gc) & 1) == 0, (xi, hex(int(gc)))


def test_e4m3_encode_round_trips_every_code(O):
    codes, vals = _e4m3_table(O)
    assert np.array_equal(O.e4m3_encode(vals.astype(np.float32)), codes)


def test_mx_scale_rule_and_bounds(O):
    """Block amax in [2^k, 2^(k+1)) gives scale 2^(k-8): the scaled block maximum
    lands in [256, 512) and encodes to 256..448 (clamped above 448); every element
    is within half a spacing of its scaled value."""
    rng = np.random.default_rng(61)
    n = (rng.normal(0, 1, (6, 256)) * np.exp2(rng.integers(-20, 20, (6, 1)))).astype(np.float32)
    n[2, 64:128] = 0.0
    q, s = O.mx_quant_rows(n)
    assert q.shape == (6, 256) and s.shape == (6, 4)
    nb = n.reshape(6, 4, 64).astype(np.float64)
    for t in range(6):
        for b in range(4):
            blk = nb[t, b]
            amax = np.max(np.abs(blk))
            if amax == 0:
                assert s[t, b] == 0 and not q[t, 64 * b:64 * b + 64].any()
                continue
            k = int(np.floor(np.log2(amax)))
            assert int(s[t, b]) == k - 8 + 127
            X = 2.0 ** (k - 8)
            dec = O.e4m3_decode(q[t, 64 * b:64 * b + 64]).astype(np.float64)
            assert 256.0 <= np.max(np.abs(dec)) <= 448.0
            scaled = blk / X
            spacing = np.exp2(np.maximum(np.floor(np.log2(np.maximum(np.abs(scaled), 1e-300))), -6) - 3)
            err = np.abs(dec - scaled)
            ok = (err <= spacing / 2) | ((np.abs(scaled) > 448.0) & (np.abs(dec) == 448.0))
            assert ok.all()


def test_mx_scaled_mm_exact_small_case(O):
    """Exact rational sum of the scaled E4M3 products, rounded once to fp32."""
    rng = np.random.default_rng(62)
    T, N, K = 3, 4, 128
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    qx, qw = rng.choice(finite, (T, K)), rng.choice(finite, (N, K))
    sx, sw = rng.integers(110, 140, (T, 2)).astype(np.uint8), rng.integers(110, 140, (N, 2)).astype(np.uint8)
    y = O.mx_scaled_mm(qx, sx, qw, sw)
    xf, wf = O.e4m3_decode(qx), O.e4m3_decode(qw)
    for t in range(T):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                b = k // 64
                acc += (Fraction(float(xf[t, k])) * Fraction(float(wf[n, k]))
                        * Fraction(2) ** (int(sx[t, b]) - 127) * Fraction(2) ** (int(sw[n, b]) - 127))
            assert y[t, n] == fraction_to_f32(acc), (t, n)


def test_mx_scaled_mm_scale_acts_on_its_64_block(O):
    """Raising one weight block's scale by one doubles exactly that block's share."""
    rng = np.random.default_rng(63)
    qx = O.e4m3_encode(rng.normal(0, 4, (2, 192)).astype(np.float32))
    qw = O.e4m3_encode(rng.normal(0, 4, (3, 192)).astype(np.float32))
    sx = np.full((2, 3), 127, np.uint8)
    sw = np.full((3, 3), 127, np.uint8)
    y0 = O.mx_scaled_mm(qx, sx, qw, sw).astype(np.float64)
    sw2 = sw.copy()
    sw2[:, 1] += 1
    y1 = O.mx_scaled_mm(qx, sx, qw, sw2).astype(np.float64)
    blk = O.e4m3_decode(qx)[:, 64:128].astype(np.float64) @ O.e4m3_decode(qw)[:, 64:128].astype(np.float64).T
    assert np.allclose(y1 - y0, blk, rtol=1e-6, atol=1e-6 * np.abs(y0).max())


def test_rmsnorm_linear_mxfp8_composes(O):
    case = synthetic.norm_linear_case(4, 128, 8, seed=64)
    x, g = bits(case["x"]), bits(case["gamma"])
    rng = np.random.default_rng(65)
    qw = O.e4m3_encode(rng.normal(0, 8, (8, 128)).astype(np.float32))
    sw = np.full((8, 2), 120, np.uint8)
    out = O.rmsnorm_linear_mxfp8(x, g, 1e-6, qw, sw)
    n, r = O.rms_norm_rows(x, g, 1e-6)
    q, s = O.mx_quant_rows(n)
    assert np.array_equal(out["q"], q) and np.array_equal(out["x_scale"], s) and np.array_equal(out["rstd"], r)
    assert np.array_equal(out["y32"], O.mx_scaled_mm(q, s, qw, sw))
