"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Acceptance rules (spec tolerances; readings of the pages as in the
oracle):
  * rstd: within 8 fp32 ulps of the oracle's own rstd;
  * bf16 outputs: |y - y_ref| <= 1e-2 * (|y_ref| + 1e-2), y_ref from the oracle
    evaluated with the device's rstd, so that both sides feed identical bf16
    normed rows to the projection;
  * int8: xq and x_scale bit-exact against the oracle's quantisation of the
    rows normed with the device's rstd; int32 accumulators bit-exact against
    the int64 GEMM of the device's xq; the fp32 dequant within 1e-5 relative
    of the oracle's dequant of those accumulators;
  * fp32 weights (no bf16 cast): |y - y_ref| <= 1e-5 * max(|y_ref|, rms(y_ref));
  * every path is deterministic: two runs give identical bits.
Every output row is checked, at full size too, in the launch configuration the
benchmark times.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle as O
import rmsnorm_linear_projection_amd as rnl
import synthetic
from tests._util import bits, f32, golden_cases, ulp_diff

pytestmark = pytest.mark.gpu

EPS = 1e-6


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    rnl.load_library()
    yield
    torch.cuda.synchronize()


@pytest.fixture
def variant(monkeypatch):
    def set_(v):
        if v is None:
            monkeypatch.delenv("RNL_VARIANT", raising=False)
        else:
            monkeypatch.setenv("RNL_VARIANT", v)
    return set_


def dev(t):
    return None if t is None else t.cuda()


def assert_bf16_close(y, y_ref, what):
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    err = np.abs(y - y_ref)
    bound = 1e-2 * (np.abs(y_ref) + 1e-2)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; "
                           f"worst err {err.max():.3g} at {np.unravel_index(np.argmax(err - bound), err.shape)}")


def assert_bf16_two_roundings(y, y_ref, what):
    """End-to-end bound for a bf16 value normed from a bf16 intermediate that the oracle forms on its own (the
    chain's q_a): that input may differ from the oracle's by one bf16 ulp (at most 2^-7 relative) where its fp32
    accumulation sits next to a rounding boundary; the norm carries the relative difference through and both sides
    round once more to bf16 (at most 2^-8 relative each), so |y - y_ref| <= 2^-6 (|y_ref| + 1e-2)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    err = np.abs(y - y_ref)
    bad = err > 2.0 ** -6 * (np.abs(y_ref) + 1e-2)
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} outside 2^-6 (|y_ref| + 1e-2); worst {err.max():.3g}"


def assert_rstd(rstd_gpu, rstd_ref, what, ulps=8):
    d = ulp_diff(rstd_gpu, rstd_ref)
    assert d.max() <= ulps, f"{what}: rstd off by {int(d.max())} ulps"


# ---------------------------------------------------------------------------
# bf16 path (norm pre-pass, then the weight-streaming kernel for T <= 16 or the
# tiled GEMM)
# ---------------------------------------------------------------------------
def run_bf16(case, out_dtype=torch.bfloat16):
    x, g, W = dev(case["x"]), dev(case["gamma"]), dev(case["W"])
    T = x.shape[0]
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    y = rnl.rmsnorm_linear_bf16(x, g, EPS, W, out_dtype=out_dtype, rstd_out=rstd)
    torch.cuda.synchronize()
    return y.cpu(), rstd.cpu().numpy()


def check_bf16_case(case, rows=None, out_dtype=torch.bfloat16):
    y, rstd = run_bf16(case, out_dtype)
    T = case["x"].shape[0]
    rows = np.arange(T) if rows is None else rows
    xb = bits(case["x"])[rows]
    gb = None if case["gamma"] is None else bits(case["gamma"])
    Wb = bits(case["W"])
    _, rstd_own = O.rms_norm_rows(xb, gb, EPS)
    assert_rstd(rstd[rows], rstd_own, case.name)
    y32, ybf, _ = O.rmsnorm_linear_bf16(xb, gb, EPS, Wb, rstd=rstd[rows])
    assert_bf16_close(f32(y)[rows], y32, case.name)
    return y


BF16_SMALL = [
    (8, 256, 128),  # bf16 RMSNorm + Linear, T=8 K=256 N=128
    (1, 4096, 64),
    (16, 512, 48),
    (3, 72, 5),  # K tail inside a 32-wide step, ragged N
    (5, 64, 1),
    (16, 8, 17),  # K = 8, the smallest
    (17, 256, 130),
    (300, 1032, 200),  # K tail of a 64-wide k-step
    (129, 64, 33),
    (16, 8200, 40),  # weight streaming with long rows, K tail
    (9, 20480, 24),
    (16, 4096, 24576),  # 32 weight rows per workgroup, three workgroups per CU
    (2, 2048, 200),
    (1, 8200, 40),  # norm fused into the weight streaming: a row longer than one load batch
    (2, 12296, 100),  # the same with two rows and a K tail
    (4, 8192, 200),  # four normed rows filling the 64 KiB LDS budget exactly
    (4, 64, 9),  # two k-steps: two of the four wavefronts have no part of K
    (8, 4096, 200),  # eight rows of 4096: 64 KiB of normed rows, the fused norm's largest
    # one token: whole weight rows per wavefront, each K bucket of the chunk count
    (1, 8, 1),
    (1, 512, 2049),  # one chunk per lane, two rows per wavefront, the last wavefront one row
    (1, 520, 300),  # two chunks, K tail
    (1, 2048, 30001),  # four chunks, six rows per wavefront, ragged last wavefront
    (1, 4104, 333),  # sixteen chunks (nine used), K tail
    (1, 8192, 100),  # the longest row it takes
    (1, 4096, 6144),  # pre-attention QKV shape, one decode token
    # a few tokens: the fused MFMA kernel (T <= 4) or the pre-pass and weight streaming
    (2, 4096, 6144),
    (3, 1024, 3000),  # ragged N
    (6, 512, 5000),
    (8, 1024, 2049),
    (7, 1032, 77),  # K tail
    # two tokens in the whole-row kernel: a K tail, a ragged last wavefront with several rows each
    (2, 520, 300),
    (2, 4104, 333),
    (2, 2048, 30001),
    # 5..16 tokens with the norm fused (every row requested at once, normed rows within 64 KiB): the
    # smallest K and 1, 2, 4 and 8 chunks per lane (the last with a K tail)
    (5, 8, 3),
    (10, 1024, 6144),
    (16, 2048, 300),
    (12, 2056, 777),
    # past 64 KiB of normed rows: pre-pass + weight streaming
    (13, 4096, 1),
    (16, 4088, 100),
    (16, 4104, 40),
]


@pytest.mark.parametrize("T,K,N", BF16_SMALL)
@pytest.mark.parametrize("gamma", [True, False])
@pytest.mark.parametrize("force", [None, "gemm"])
def test_bf16_small(T, K, N, gamma, force, variant):
    variant(force)
    check_bf16_case(synthetic.norm_linear_case(T, K, N, seed=T + K + N, gamma=gamma))


@pytest.mark.parametrize("T,K,N", [(8, 256, 128), (300, 1032, 200), (1, 64, 7), (2, 520, 300), (16, 4096, 200)])
def test_bf16_fp32_output(T, K, N):
    check_bf16_case(synthetic.norm_linear_case(T, K, N, seed=5), out_dtype=torch.float32)


@pytest.mark.parametrize("T,K,N", [
    (4000, 264, 6100),  # 256 x 192 tiles, ragged M, N and K
    (2000, 136, 4000),  # 256 x 128 tiles, ragged M, N and K
])
def test_bf16_large_tiles_ragged(T, K, N):
    case = synthetic.norm_linear_case(T, K, N, seed=11)
    check_bf16_case(case)


@pytest.mark.parametrize("scale", [0.0, 1024.0, 1.0 / 4096])
@pytest.mark.parametrize("K", [4096, 7168])
def test_bf16_single_token_scaled(scale, K):
    """One token (the whole-row kernel): a zero row gives y = 0 and rstd = 1/sqrt(eps); scaled rows keep parity."""
    case = synthetic.norm_linear_case(1, K, 130, seed=K)
    case.tensors["x"] = (case.tensors["x"].float() * scale).to(torch.bfloat16)
    y = check_bf16_case(case)
    if scale == 0.0:
        assert (f32(y) == 0).all()


def test_bf16_single_token_no_gamma_fp32_output():
    check_bf16_case(synthetic.norm_linear_case(1, 2056, 517, seed=9, gamma=False), out_dtype=torch.float32)


def test_bf16_zero_and_scaled_rows():
    case = synthetic.norm_linear_case(40, 512, 96, seed=3)
    x = case.tensors["x"].clone()
    x[3] = 0
    x[7] = (x[7].float() * 1024).to(torch.bfloat16)
    x[9] = (x[9].float() / 4096).to(torch.bfloat16)
    case.tensors["x"] = x
    y = check_bf16_case(case)
    assert (f32(y)[3] == 0).all()


@pytest.mark.parametrize("T", [4096, 1, 16])
def test_bf16_preattn_qkv_full_size(T):
    """Pre-attention norm + fused QKV projection, K=4096, N=6144, at full size."""
    case = synthetic.preattn_qkv(T)
    y1 = check_bf16_case(case)
    y2, _ = run_bf16(case)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), "not deterministic"


# ---------------------------------------------------------------------------
# int8 W8A8 path
# ---------------------------------------------------------------------------
def run_int8(case, out_dtype):
    x, g, Wq, ws = dev(case["x"]), dev(case["gamma"]), dev(case["Wq"]), dev(case["w_scale"])
    T, K = x.shape
    xq = torch.empty((T, K), dtype=torch.int8, device="cuda")
    xs = torch.empty(T, dtype=torch.float32, device="cuda")
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    y = rnl.rmsnorm_linear_int8(x, g, EPS, Wq, ws, out_dtype=out_dtype, xq_out=xq, x_scale_out=xs, rstd_out=rstd)
    torch.cuda.synchronize()
    return y.cpu(), xq.cpu().numpy(), xs.cpu().numpy(), rstd.cpu().numpy()


def check_int8_case(case, rows=None):
    T = case["x"].shape[0]
    rows = np.arange(T) if rows is None else rows
    xb = bits(case["x"])[rows]
    gb = None if case["gamma"] is None else bits(case["gamma"])
    Wq = case["Wq"].numpy()
    wsc = case["w_scale"].numpy()

    acc, xq, xs, rstd = run_int8(case, torch.int32)
    _, rstd_own = O.rms_norm_rows(xb, gb, EPS)
    assert_rstd(rstd[rows], rstd_own, case.name)
    n, _ = O.rms_norm_rows(xb, gb, EPS, rstd=rstd[rows])
    q_ref, xs_ref, _ = O.quant_rows(n)
    assert np.array_equal(xq[rows], q_ref), f"{case.name}: xq not bit-exact ({int((xq[rows] != q_ref).sum())} differ)"
    assert np.array_equal(xs[rows], xs_ref), f"{case.name}: x_scale not bit-exact"
    acc_ref = O.int8_gemm(xq[rows], Wq)
    assert np.array_equal(acc.numpy()[rows].astype(np.int64), acc_ref), f"{case.name}: int32 acc not bit-exact"

    yf, xq2, xs2, _ = run_int8(case, torch.float32)
    assert np.array_equal(xq2, xq) and np.array_equal(xs2, xs)
    y_ref = O.dequant(acc_ref, xs_ref, wsc)
    rel = np.abs(yf.numpy()[rows] - y_ref) / np.maximum(np.abs(y_ref), 1e-30)
    assert (rel <= 1e-5).all(), f"{case.name}: fp32 dequant off by {rel.max():.3g}"

    yb, _, _, _ = run_int8(case, torch.bfloat16)
    assert_bf16_close(f32(yb)[rows], y_ref, case.name)
    return yb


INT8_SMALL = [
    (37, 256, 72),
    (1, 64, 16),
    (16, 128, 130),
    (130, 4112, 100),  # K tail of a 128-byte k-step
    (3, 16, 3),
]


@pytest.mark.parametrize("T,K,N", INT8_SMALL)
@pytest.mark.parametrize("gamma", [True, False])
def test_int8_small(T, K, N, gamma):
    check_int8_case(synthetic.int8_case(T, K, N, seed=T * 3 + N, gamma=gamma))


def test_int8_tiles_ragged():
    case = synthetic.int8_case(2000, 144, 4000, seed=17)  # 256 x 128 tiles
    check_int8_case(case)


def test_int8_zero_row():
    case = synthetic.int8_case(20, 256, 40, seed=2)
    x = case.tensors["x"].clone()
    x[4] = 0
    case.tensors["x"] = x
    yb = check_int8_case(case)
    assert (f32(yb)[4] == 0).all()


def xq_mismatch_own_rstd(case, xq):
    """End-to-end codes against the oracle's quantisation with its own rstd (informational).  The device's rstd
    may differ from the oracle's by a few ulps (a different fp32 summation order), which moves fl(n * s) by far
    less than one unit; a code can then only differ by one, where that product sits within the shift of a .5 tie.
    Returns (count of differing codes, largest difference)."""
    gb = None if case["gamma"] is None else bits(case["gamma"])
    n_own, _ = O.rms_norm_rows(bits(case["x"]), gb, EPS)
    q_own, _, _ = O.quant_rows(n_own)
    d = np.abs(xq.astype(np.int16) - q_own.astype(np.int16))
    return int((d != 0).sum()), int(d.max())


def test_int8_w8a8_full_size(record_property):
    """INT8 W8A8 norm + linear, T=2048, K=4096, N=4096, every row."""
    case = synthetic.int8_w8a8()
    y1 = check_int8_case(case)
    y2, xq, _, _ = run_int8(case, torch.bfloat16)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), "not deterministic"
    count, worst = xq_mismatch_own_rstd(case, xq)
    record_property("xq_mismatch_vs_oracle_own_rstd", count)
    print(f"int8 W8A8: {count} of {xq.size} codes differ from the oracle's own-rstd quantisation (max |diff| {worst})")
    assert worst <= 1


# ---------------------------------------------------------------------------
# fp32 weights: the large-reduction split-K path
# ---------------------------------------------------------------------------
def check_fp32w_case(case, out_dtype=torch.float32):
    y, rstd = run_bf16(case, out_dtype)
    xb = bits(case["x"])
    gb = None if case["gamma"] is None else bits(case["gamma"])
    W = case["W"].numpy()
    _, rstd_own = O.rms_norm_rows(xb, gb, EPS)
    assert_rstd(rstd, rstd_own, case.name)
    y_ref, _ = O.rmsnorm_linear_fp32w(xb, gb, EPS, W, rstd=rstd)
    if out_dtype == torch.float32:
        scale = max(float(np.sqrt(np.mean(y_ref.astype(np.float64) ** 2))), 1e-30)
        err = np.abs(y.numpy().astype(np.float64) - y_ref)
        bound = 1e-5 * np.maximum(np.abs(y_ref), scale)
        assert (err <= bound).all(), f"{case.name}: max err {err.max():.3g} (rms {scale:.3g})"
    else:
        assert_bf16_close(f32(y), y_ref, case.name)
    return y


@pytest.mark.parametrize("T,K,N,gamma", [
    (3, 64, 5, False),
    (70, 4104, 33, False),  # > 64 tokens, > 32 columns, K tail
    (16, 1024, 24, True),
    (130, 256, 64, True),
])
def test_fp32w_small(T, K, N, gamma):
    check_fp32w_case(synthetic.norm_linear_case(T, K, N, seed=T + N, gamma=gamma, w_dtype="fp32"))


def test_fp32w_bf16_output():
    check_fp32w_case(synthetic.norm_linear_case(20, 512, 24, seed=1, gamma=False, w_dtype="fp32"),
                     out_dtype=torch.bfloat16)


@pytest.mark.parametrize("T,K,N", [(3, 1 << 20, 24), (2, (1 << 20) - 8, 8)])
def test_max_k(T, K, N):
    """The largest K the bf16 entry point accepts, with bf16 and with fp32 weights."""
    check_bf16_case(synthetic.norm_linear_case(T, K, N, seed=5))
    check_fp32w_case(synthetic.norm_linear_case(T, K, N, seed=6, gamma=False, w_dtype="fp32"))


def test_int8_max_k():
    """The largest K for which an int32 accumulator cannot overflow (a multiple of 16)."""
    check_int8_case(synthetic.int8_case(2, 133136, 16, seed=7))


def test_skinny_fp32_full_size():
    """Large-reduction tiny-width norm + linear, T=512, K=28672, N=24, fp32 W."""
    case = synthetic.skinny_fp32()
    y1 = check_fp32w_case(case)
    y2, _ = run_bf16(case, torch.float32)
    assert torch.equal(y1, y2), "not deterministic"


# ---------------------------------------------------------------------------
# q_a -> norm -> q_b chain
# ---------------------------------------------------------------------------
def run_chain(case):
    x, Wa, g, Wb = (dev(case[k]) for k in ("x", "W_a", "gamma", "W_b"))
    T, R = x.shape[0], Wa.shape[0]
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    qa = torch.empty((T, R), dtype=torch.bfloat16, device="cuda")
    y, qr = rnl.norm_proj_chain(x, Wa, g, EPS, Wb, rstd_out=rstd, qa_out=qa)
    torch.cuda.synchronize()
    return y.cpu(), qr.cpu(), qa.cpu(), rstd.cpu().numpy()


def check_normed_stage(rows_in, gamma_bits, rstd, out_bits, what):
    """The norm step of the chain on the device's own input rows (bf16 bits):
    rstd within 8 ulps of the oracle's rstd of those rows, and the normed bf16
    rows bit-exact given the device's rstd."""
    _, r_own = O.rms_norm_rows(rows_in, gamma_bits, EPS)
    assert_rstd(rstd, r_own, what)
    n, _ = O.rms_norm_rows(rows_in, gamma_bits, EPS, rstd=rstd)
    want = O.f32_to_bf16_bits(n)
    bad = out_bits != want
    assert not bad.any(), f"{what}: {int(bad.sum())} normed values not bit-exact given the device's input and rstd"


def check_chain_case(case):
    y, qr, qa, rstd = run_chain(case)
    xb = bits(case["x"])
    Wa, Wb = bits(case["W_a"]), bits(case["W_b"])
    gb = None if case["gamma"] is None else bits(case["gamma"])
    # stage 1: q_a is a bf16 output of an fp32 accumulation of x . W_a^T
    qab = bits(qa)
    assert_bf16_close(O.bf16_bits_to_f32(qab), O.project_bf16(O.bf16_bits_to_f32(xb), Wa), case.name + " q_a")
    # the norm on the device's q_a (AT-10 page section 5: q_a -> rms_norm -> x gamma -> bf16 = qr)
    check_normed_stage(qab, gb, rstd, bits(qr), case.name + " qr")
    # stage 2 from the device's qr: identical bf16 inputs
    assert_bf16_close(f32(y), O.project_bf16(O.bf16_bits_to_f32(bits(qr)), Wb), case.name + " y")
    # end to end against the oracle's own stage 1
    ref = O.norm_proj_chain(xb, Wa, gb, EPS, Wb)
    assert_bf16_two_roundings(f32(qr), O.bf16_bits_to_f32(ref["qr"]), case.name + " qr end to end")
    return y


@pytest.mark.parametrize("T,K,R,N,gamma", [
    (37, 256, 64, 80, True),
    (5, 128, 48, 30, False),
    (300, 520, 136, 260, True),
    (64, 4096, 128, 64, True),  # stage 1 split over K (4 slices)
    (50, 2056, 72, 33, False),  # split over K with a K tail
    (4, 7168, 1536, 520, True),  # few tokens: both stages stream their weights
    (16, 1032, 264, 6143, False),
])
def test_chain_small(T, K, R, N, gamma):
    check_chain_case(synthetic.chain_case(T, K, R, N, seed=T + R, gamma=gamma))


def test_mla_q_chain_full_size():
    """Low-rank query chain x[1024,7168] -> W_a[1536,7168] -> norm -> W_b[24576,1536], every row."""
    case = synthetic.mla_q_chain()
    y1 = check_chain_case(case)
    y2 = run_chain(case)[0]
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), "not deterministic"


# ---------------------------------------------------------------------------
# the atoms: AT-03 RMSNorm, AT-03 + AT-05 quant, AT-09 Linear (BF16, INT8)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,K", [(7, 64), (130, 4104), (3, 20480)])
def test_atom_rms_norm_bf16(T, K):
    case = synthetic.norm_linear_case(T, K, 1, seed=T + K)
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    y = rnl.rms_norm_bf16(dev(case["x"]), dev(case["gamma"]), EPS, rstd_out=rstd)
    torch.cuda.synchronize()
    xb, gb = bits(case["x"]), bits(case["gamma"])
    r = rstd.cpu().numpy()
    _, r_own = O.rms_norm_rows(xb, gb, EPS)
    assert_rstd(r, r_own, "rms_norm_bf16")
    n, _ = O.rms_norm_rows(xb, gb, EPS, rstd=r)
    assert np.array_equal(bits(y.cpu()), O.f32_to_bf16_bits(n)), "normed rows not bit-exact given rstd"


@pytest.mark.parametrize("T,K", [(9, 64), (65, 4112)])
def test_atom_rms_norm_quant_int8(T, K):
    case = synthetic.int8_case(T, K, 1, seed=T)
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    xq, xs = rnl.rms_norm_quant_int8(dev(case["x"]), dev(case["gamma"]), EPS, rstd_out=rstd)
    torch.cuda.synchronize()
    n, _ = O.rms_norm_rows(bits(case["x"]), bits(case["gamma"]), EPS, rstd=rstd.cpu().numpy())
    q, s, _ = O.quant_rows(n)
    assert np.array_equal(xq.cpu().numpy(), q) and np.array_equal(xs.cpu().numpy(), s)


@pytest.mark.parametrize("reps,T", [
    (2, 4),      # K = 16: a wavefront per row
    (512, 4),    # K = 4096, few rows: a workgroup per row
    (512, 300),  # K = 4096, 300 rows: a wavefront per row
])
def test_atom_quant_int8_golden_ties(reps, T):
    """The hand-derived rows of tests/golden/int8_quant_ties.txt (eps = 0, rstd = 1, s = 64 exactly, so n * s
    lands on exact .5 ties), each row repeated `reps` times along K and the rows cycled to T: the device's codes
    and x_scale must be the fixture's, whatever the kernel."""
    golden = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "int8_quant_ties.txt")
    for c in golden_cases(golden):
        x = np.tile(np.array(c["x"], dtype=np.float32), (1, reps))
        q = np.tile(np.array(c["q"], dtype=np.int8), (1, reps))
        xs = np.array(c["x_scale"], dtype=np.float32)
        pick = np.arange(T) % x.shape[0]
        g = np.tile(np.array(c["gamma"], dtype=np.float32), reps)
        xd = torch.from_numpy(x[pick]).to(torch.bfloat16).cuda()
        gd = torch.from_numpy(g).to(torch.bfloat16).cuda()
        assert np.array_equal(f32(xd.cpu()), x[pick]) and np.array_equal(f32(gd.cpu()), g), "fixture not bf16-exact"
        xq, x_scale = rnl.rms_norm_quant_int8(xd, gd, c["eps"])
        torch.cuda.synchronize()
        assert np.array_equal(xq.cpu().numpy(), q[pick]), f"{c['name']}: codes differ"
        assert np.array_equal(x_scale.cpu().numpy(), xs[pick]), f"{c['name']}: x_scale differs"


@pytest.mark.parametrize("M,K,N", [(33, 72, 17), (300, 1032, 200), (4000, 264, 6100)])
def test_atom_linear_bf16(M, K, N):
    a = synthetic.normal((M, K), 1.0, 3, 11)
    W = synthetic.normal((N, K), 1.0 / np.sqrt(K), 3, 12)
    y = rnl.linear_bf16(dev(a), dev(W), out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = O.project_bf16(O.bf16_bits_to_f32(bits(a)), bits(W))
    assert_bf16_close(f32(y), ref, "linear_bf16")


@pytest.mark.parametrize("M,K,N", [
    (1, 4096, 6144),  # 24 weight rows per workgroup (two MFMA row blocks)
    (16, 4104, 6143),  # K tail of a 32-wide step, ragged N
    (5, 264, 100),
    (16, 1032, 1536),
    (2, 64, 24576),
    (7, 8, 3),
])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_atom_linear_bf16_few_rows(M, K, N, out_dtype):
    a = synthetic.normal((M, K), 1.0, 5, 11)
    W = synthetic.normal((N, K), 1.0 / np.sqrt(K), 5, 12)
    y = rnl.linear_bf16(dev(a), dev(W), out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref = O.project_bf16(O.bf16_bits_to_f32(bits(a)), bits(W))
    assert_bf16_close(f32(y), ref, "linear_bf16 few rows")
    y2 = rnl.linear_bf16(dev(a), dev(W), out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "not deterministic"


@pytest.mark.parametrize("M,K,N", [(33, 64, 17), (257, 4112, 130)])
def test_atom_linear_int8(M, K, N):
    q = synthetic.int8_uniform((M, K), 4, 1)
    W = synthetic.int8_uniform((N, K), 4, 2)
    xs = synthetic.uniform((M,), 1e-3, 1e-2, 4, 3, dtype=torch.float32)
    ws = synthetic.uniform((N,), 1e-3, 1e-2, 4, 4, dtype=torch.float32)
    acc = rnl.linear_int8(dev(q), dev(xs), dev(W), dev(ws), out_dtype=torch.int32)
    y = rnl.linear_int8(dev(q), dev(xs), dev(W), dev(ws), out_dtype=torch.float32)
    torch.cuda.synchronize()
    acc_ref = O.int8_gemm(q.numpy(), W.numpy())
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), acc_ref)
    y_ref = O.dequant(acc_ref, xs.numpy(), ws.numpy())
    assert np.array_equal(y.cpu().numpy(), y_ref)


def test_atom_linear_int8_large_tiles():
    """Enough 256 x 192 tiles for one per CU (eight-wavefront workgroups), ragged in M and N: sampled rows of
    the int32 accumulators and of the dequantised output, bit for bit."""
    M, K, N = 4100, 144, 3080
    q = synthetic.int8_uniform((M, K), 6, 1)
    W = synthetic.int8_uniform((N, K), 6, 2)
    xs = synthetic.uniform((M,), 1e-3, 1e-2, 6, 3, dtype=torch.float32)
    ws = synthetic.uniform((N,), 1e-3, 1e-2, 6, 4, dtype=torch.float32)
    acc = rnl.linear_int8(dev(q), dev(xs), dev(W), dev(ws), out_dtype=torch.int32)
    y = rnl.linear_int8(dev(q), dev(xs), dev(W), dev(ws), out_dtype=torch.float32)
    torch.cuda.synchronize()
    acc_ref = O.int8_gemm(q.numpy(), W.numpy())
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), acc_ref)
    assert np.array_equal(y.cpu().numpy(), O.dequant(acc_ref, xs.numpy(), ws.numpy()))


# ---------------------------------------------------------------------------
# residual add before the norm: x_add bit-exact against the oracle's add, then
# the same checks as the paths without the add, on x_add; and the call must
# give the same bits as the call without the add made on the device's x_add
# ---------------------------------------------------------------------------
def run_add_bf16(case, out_dtype=torch.bfloat16):
    x, r, g, W = dev(case["x"]), dev(case["residual"]), dev(case["gamma"]), dev(case["W"])
    T = x.shape[0]
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    y, xa = rnl.add_rmsnorm_linear_bf16(x, r, g, EPS, W, out_dtype=out_dtype, rstd_out=rstd)
    torch.cuda.synchronize()
    return y.cpu(), xa.cpu(), rstd.cpu().numpy()


def check_add_bf16_case(case, rows=None, out_dtype=torch.bfloat16):
    y, xa, rstd = run_add_bf16(case, out_dtype)
    T = case["x"].shape[0]
    rows = np.arange(T) if rows is None else rows
    xb, rb = bits(case["x"])[rows], bits(case["residual"])[rows]
    gb = None if case["gamma"] is None else bits(case["gamma"])
    xa_ref = O.add_residual(xb, rb)
    assert np.array_equal(bits(xa)[rows], xa_ref), \
        f"{case.name}: x_add not bit-exact ({int((bits(xa)[rows] != xa_ref).sum())} differ)"
    _, rstd_own = O.rms_norm_rows(xa_ref, gb, EPS)
    assert_rstd(rstd[rows], rstd_own, case.name)
    if case["W"].dtype == torch.float32:
        _, y_ref, _ = O.add_rmsnorm_linear_fp32w(xb, rb, gb, EPS, case["W"].numpy(), rstd=rstd[rows])
        if out_dtype == torch.float32:
            scale = max(float(np.sqrt(np.mean(y_ref.astype(np.float64) ** 2))), 1e-30)
            err = np.abs(y.numpy()[rows].astype(np.float64) - y_ref)
            assert (err <= 1e-5 * np.maximum(np.abs(y_ref), scale)).all(), f"{case.name}: max err {err.max():.3g}"
        else:
            assert_bf16_close(f32(y)[rows], y_ref, case.name)
    else:
        _, y32, _, _ = O.add_rmsnorm_linear_bf16(xb, rb, gb, EPS, bits(case["W"]), rstd=rstd[rows])
        assert_bf16_close(f32(y)[rows], y32, case.name)
    # the add path computes exactly the plain path on x_add
    y_plain = rnl.rmsnorm_linear_bf16(xa.cuda(), dev(case["gamma"]), EPS, dev(case["W"]), out_dtype=out_dtype)
    assert torch.equal(y_plain.cpu().view(torch.uint8), y.view(torch.uint8)), f"{case.name}: differs from plain path"
    return y


ADD_BF16 = [
    (1, 4096, 6144),   # one and two tokens: the whole-row kernel adds the residual itself
    (2, 520, 300),
    (1, 8192, 70),
    (8, 256, 128),     # weight streaming, one wavefront per row
    (16, 4104, 40),
    (300, 1032, 200),  # tiled GEMM, ragged tiles
    (5, 12296, 40),    # rows held in registers across a workgroup
    (40, 20488, 100),  # rows re-read for each pass
    (3, 72, 5),
]


@pytest.mark.parametrize("T,K,N", ADD_BF16)
@pytest.mark.parametrize("gamma", [True, False])
def test_add_bf16_small(T, K, N, gamma):
    base = synthetic.norm_linear_case(T, K, N, seed=T + 2 * N, gamma=gamma)
    check_add_bf16_case(synthetic.with_residual(base, seed=T + 2 * N))


def test_add_bf16_fp32_output():
    case = synthetic.with_residual(synthetic.norm_linear_case(17, 256, 130, seed=4), seed=4)
    check_add_bf16_case(case, out_dtype=torch.float32)


def test_add_bf16_cancelling_residual():
    # residual = -x on some rows: x_add is exactly zero there, and so is y
    case = synthetic.with_residual(synthetic.norm_linear_case(24, 512, 64, seed=8), seed=8)
    r = case.tensors["residual"].clone()
    r[2] = -case["x"][2]
    r[5] = 0
    case.tensors["residual"] = r
    y = check_add_bf16_case(case)
    assert (f32(y)[2] == 0).all()


@pytest.mark.parametrize("T,K,N,gamma", [(70, 4104, 33, False), (16, 28672, 24, True), (3, 64, 5, False)])
def test_add_fp32w(T, K, N, gamma):
    base = synthetic.norm_linear_case(T, K, N, seed=T + N, gamma=gamma, w_dtype="fp32")
    check_add_bf16_case(synthetic.with_residual(base, seed=T + N), out_dtype=torch.float32)


@pytest.mark.parametrize("T", [4096, 16])
def test_add_preattn_qkv_full_size(T):
    """Residual add -> pre-attention norm -> fused QKV projection, K=4096, N=6144, at full size."""
    case = synthetic.preattn_qkv_add(T)
    y1 = check_add_bf16_case(case)
    y2, _, _ = run_add_bf16(case)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), "not deterministic"


def run_add_int8(case, out_dtype):
    x, r, g = dev(case["x"]), dev(case["residual"]), dev(case["gamma"])
    Wq, ws = dev(case["Wq"]), dev(case["w_scale"])
    T, K = x.shape
    xq = torch.empty((T, K), dtype=torch.int8, device="cuda")
    xs = torch.empty(T, dtype=torch.float32, device="cuda")
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    y, xa = rnl.add_rmsnorm_linear_int8(x, r, g, EPS, Wq, ws, out_dtype=out_dtype, xq_out=xq, x_scale_out=xs,
                                        rstd_out=rstd)
    torch.cuda.synchronize()
    return y.cpu(), xa.cpu(), xq.cpu().numpy(), xs.cpu().numpy(), rstd.cpu().numpy()


def check_add_int8_case(case, rows=None):
    T = case["x"].shape[0]
    rows = np.arange(T) if rows is None else rows
    xb, rb = bits(case["x"])[rows], bits(case["residual"])[rows]
    gb = None if case["gamma"] is None else bits(case["gamma"])
    Wq, wsc = case["Wq"].numpy(), case["w_scale"].numpy()

    acc, xa, xq, xs, rstd = run_add_int8(case, torch.int32)
    xa_ref = O.add_residual(xb, rb)
    assert np.array_equal(bits(xa)[rows], xa_ref), f"{case.name}: x_add not bit-exact"
    _, rstd_own = O.rms_norm_rows(xa_ref, gb, EPS)
    assert_rstd(rstd[rows], rstd_own, case.name)
    ref = O.add_rmsnorm_linear_int8(xb, rb, gb, EPS, Wq, wsc, rstd=rstd[rows])
    assert np.array_equal(ref["x_add"], xa_ref)
    assert np.array_equal(xq[rows], ref["q"]), f"{case.name}: xq not bit-exact"
    assert np.array_equal(xs[rows], ref["x_scale"]), f"{case.name}: x_scale not bit-exact"
    assert np.array_equal(acc.numpy()[rows].astype(np.int64), ref["acc"]), f"{case.name}: int32 acc not bit-exact"

    yf, _, _, _, _ = run_add_int8(case, torch.float32)
    rel = np.abs(yf.numpy()[rows] - ref["y32"]) / np.maximum(np.abs(ref["y32"]), 1e-30)
    assert (rel <= 1e-5).all(), f"{case.name}: fp32 dequant off by {rel.max():.3g}"
    yb, _, _, _, _ = run_add_int8(case, torch.bfloat16)
    assert_bf16_close(f32(yb)[rows], ref["y32"], case.name)
    y_plain = rnl.rmsnorm_linear_int8(xa.cuda(), dev(case["gamma"]), EPS, dev(case["Wq"]), dev(case["w_scale"]))
    assert torch.equal(y_plain.cpu().view(torch.int16), yb.view(torch.int16)), f"{case.name}: differs from plain path"


@pytest.mark.parametrize("T,K,N,gamma", [
    (37, 256, 72, True),
    (130, 4112, 100, False),  # K tail of a 128-byte k-step
    (9, 12304, 40, True),     # rows held in registers across a workgroup
    (4, 20480, 16, False),    # rows re-read for each pass
])
def test_add_int8(T, K, N, gamma):
    base = synthetic.int8_case(T, K, N, seed=T + N, gamma=gamma)
    check_add_int8_case(synthetic.with_residual(base, seed=T + N))


def test_add_int8_w8a8_full_size():
    """Residual add, then INT8 W8A8 norm + linear, T=2048, K=4096, N=4096, at full size."""
    case = synthetic.with_residual(synthetic.int8_w8a8())
    check_add_int8_case(case)


# ---------------------------------------------------------------------------
# per-head stage after the projection: per-head RMSNorm (+ RoPE).  The heads
# are bit-exact against the oracle given the device's head rstd; the rstd is
# within 8 ulps of the oracle's own.
# ---------------------------------------------------------------------------
def _np(t):
    return None if t is None else t.numpy()


@pytest.mark.parametrize("T,ld,col0,H,D", [
    (5, 64, 0, 4, 16),
    (7, 256, 64, 3, 64),
    (33, 6144, 0, 40, 128),    # query and key heads of the pre-attention layout
    (3, 24576, 0, 128, 192),   # 24 lanes per head, padded to 32
    (2, 1536, 512, 2, 512),    # one head per wavefront
    (1, 136, 8, 1, 128),
    (4, 512, 16, 5, 48),       # 3 chunk pairs per head: groups of 4 lanes, one idle
    (3, 400, 0, 5, 80),        # 5 chunk pairs per head: groups of 8 lanes, three idle
    (6, 96, 32, 2, 32),        # 2 chunk pairs per head
])
@pytest.mark.parametrize("gamma,rope,inplace", [(True, True, True), (False, True, False), (True, False, False),
                                                (False, False, True)])
def test_head_norm_atom(T, ld, col0, H, D, gamma, rope, inplace):
    seed = T + H + D
    y = synthetic.normal((T, ld), 2.0, seed, 1)
    g = synthetic.uniform((D,), 0.5, 1.5, seed, 2) if gamma else None
    c, s = synthetic.rope_tables(T, D // 2, seed) if rope else (None, None)
    yd = y.cuda()
    rstd = torch.empty((T, H), dtype=torch.float32, device="cuda")
    if inplace:
        out = rnl.head_rms_norm_bf16(yd, col0, H, D, dev(g), EPS, dev(c), dev(s), rstd_out=rstd)
    else:
        out = torch.full_like(yd, 7.0)
        rnl.head_rms_norm_bf16(yd, col0, H, D, dev(g), EPS, dev(c), dev(s), out=out, rstd_out=rstd)
    torch.cuda.synchronize()
    r = rstd.cpu().numpy()
    yb, gb = bits(y), (None if g is None else bits(g))
    _, r_own = O.head_rms_norm(yb, col0, H, D, gb, EPS, _np(c), _np(s))
    assert_rstd(r, r_own, f"heads T{T} D{D}")
    ref, _ = O.head_rms_norm(yb, col0, H, D, gb, EPS, _np(c), _np(s), rstd=r)
    ob = bits(out.cpu())
    heads = slice(col0, col0 + H * D)
    bad = ob[:, heads] != ref[:, heads]
    assert not bad.any(), f"{int(bad.sum())} head values differ"
    outside = np.ones(ld, dtype=bool)
    outside[heads] = False
    if inplace:
        assert np.array_equal(ob[:, outside], yb[:, outside])
    else:
        assert (f32(out)[:, outside] == 7.0).all(), "columns outside the heads were written"


def run_preattn(case, rows=None):
    t = {k: dev(v) for k, v in case.tensors.items()}
    d = case.dims
    T, Hq, Hkv, D = d["T"], d["Hq"], d["Hkv"], d["D"]
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    hr = torch.empty((T, Hq + Hkv), dtype=torch.float32, device="cuda")
    y, xa = rnl.preattn_qkv_bf16(t["x"], t["gamma"], EPS, t["W"], Hq, Hkv, D, t["gamma_q"], t["gamma_k"], EPS,
                                 t["cos"], t["sin"], residual=t.get("residual"), rstd_out=rstd, head_rstd_out=hr)
    # the projection alone, through the same kernels, on what the norm read
    p = rnl.rmsnorm_linear_bf16(xa if xa is not None else t["x"], t["gamma"], EPS, t["W"])
    torch.cuda.synchronize()
    return y.cpu(), (None if xa is None else xa.cpu()), p.cpu(), rstd.cpu().numpy(), hr.cpu().numpy()


def check_preattn_case(case, rows=None):
    y, xa, p, rstd, hr = run_preattn(case)
    d = case.dims
    T, Hq, Hkv, D = d["T"], d["Hq"], d["Hkv"], d["D"]
    rows = np.arange(T) if rows is None else rows
    qk = slice(0, (Hq + Hkv) * D)
    v = slice((Hq + Hkv) * D, (Hq + 2 * Hkv) * D)
    c = None if case["cos"] is None else case["cos"].numpy()[rows]
    s = None if case["sin"] is None else case["sin"].numpy()[rows]
    gq = None if case["gamma_q"] is None else bits(case["gamma_q"])
    gk = None if case["gamma_k"] is None else bits(case["gamma_k"])
    yb, pb = bits(y)[rows], bits(p)[rows]
    # value heads are the projection; query / key heads the head stage of it, bit for bit
    assert np.array_equal(yb[:, v], pb[:, v]), f"{case.name}: value heads differ from the projection"
    hq, _ = O.head_rms_norm(pb, 0, Hq, D, gq, EPS, c, s, rstd=hr[rows, :Hq])
    hk, _ = O.head_rms_norm(hq, Hq * D, Hkv, D, gk, EPS, c, s, rstd=hr[rows, Hq:])
    assert np.array_equal(yb[:, qk], hk[:, qk]), f"{case.name}: {int((yb[:, qk] != hk[:, qk]).sum())} head values differ"
    _, hq_own = O.head_rms_norm(pb, 0, Hq, D, gq, EPS)
    _, hk_own = O.head_rms_norm(pb, Hq * D, Hkv, D, gk, EPS)
    assert_rstd(hr[rows], np.concatenate([hq_own, hk_own], axis=1), case.name)
    # end to end against the oracle's own projection (device input rstd)
    xb = bits(case["x"])[rows]
    rb = None if "residual" not in case.tensors else bits(case["residual"])[rows]
    ref = O.preattn_qkv(xb, rb, bits(case["gamma"]), EPS, bits(case["W"]), Hq, Hkv, D, gq, gk, EPS, c, s,
                        rstd=rstd[rows])
    if rb is not None:
        assert np.array_equal(bits(xa)[rows], ref["x_add"]), f"{case.name}: x_add not bit-exact"
    assert_rstd(rstd[rows], O.rms_norm_rows(ref["x_add"] if rb is not None else xb, bits(case["gamma"]), EPS)[1],
                case.name)
    yf, rf = O.bf16_bits_to_f32(yb).astype(np.float64), O.bf16_bits_to_f32(ref["y"]).astype(np.float64)
    err = np.abs(yf[:, qk] - rf[:, qk])
    assert (err <= (np.abs(rf[:, qk]) + 1.0) / 64).all(), f"{case.name}: head values off by {err.max():.3g}"
    assert_bf16_close(yf[:, v], ref["y32"][:, v], case.name)
    return y


@pytest.mark.parametrize("T,K,Hq,Hkv,D,residual,rope,head_gamma", [
    (8, 256, 4, 2, 64, False, True, True),
    (8, 256, 4, 2, 64, True, False, False),
    (2, 256, 4, 2, 64, False, True, True),     # two tokens: the whole-row kernel
    (1, 4096, 32, 8, 128, True, True, True),   # one decode token with the residual add, in the whole-row kernel
    (2, 520, 4, 2, 64, True, True, True),
    (16, 512, 4, 2, 64, False, True, True),    # sixteen tokens: the norm fused into the weight streaming
    (40, 1032, 6, 1, 128, True, True, True),   # tiled GEMM, ragged tiles
    (3, 64, 2, 0, 16, False, True, False),     # no key / value heads
    (20, 512, 3, 3, 192, False, True, True),
])
def test_preattn_small(T, K, Hq, Hkv, D, residual, rope, head_gamma):
    case = synthetic.preattn_case(T, K, Hq, Hkv, D, seed=T + Hq, residual=residual, rope=rope,
                                  head_gamma=head_gamma)
    check_preattn_case(case)


@pytest.mark.parametrize("T,K,Hq,Hkv,residual,rope,head_gamma,force_gemm", [
    (300, 520, 3, 1, False, True, True, False),    # two column tiles, the second holding two heads; ragged rows
    (130, 256, 2, 0, False, False, False, False),  # query heads only, no rotation, no head gammas
    (257, 1024, 4, 2, True, True, False, False),   # residual add, key heads without a gamma
    (40, 1032, 6, 1, True, True, True, False),
    (8, 256, 1, 1, False, True, True, True),       # eight tokens on the tiled GEMM (RNL_VARIANT=gemm)
    (4096, 4096, 32, 8, True, True, True, False),  # the pre-attention block
])
def test_preattn_head_epilogue(variant, T, K, Hq, Hkv, residual, rope, head_gamma, force_gemm):
    """Heads of 128 on the tiled GEMM: the per-head stage in the GEMM's epilogue against the oracle, and
    bit for bit against the separate per-head pass (RNL_VARIANT=prepass)."""
    case = synthetic.preattn_case(T, K, Hq, Hkv, 128, seed=T + 7 * Hq, residual=residual, rope=rope,
                                  head_gamma=head_gamma)
    variant("gemm" if force_gemm else None)
    y = check_preattn_case(case)
    _, _, _, rstd, hr = run_preattn(case)
    variant("prepass")
    y2, _, _, rstd2, hr2 = run_preattn(case)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "epilogue and separate pass differ"
    assert np.array_equal(hr, hr2) and np.array_equal(rstd, rstd2)


@pytest.mark.parametrize("M,K,Hq,Hkv,rope,head_gamma", [
    (4096, 4096, 32, 8, True, True),   # the pre-attention block's projection (the epilogue)
    (300, 520, 3, 1, True, False),     # the epilogue, ragged rows and a two-head column tile
    (12, 256, 2, 1, False, True),      # few rows: projection, then the per-head pass
])
def test_linear_heads(M, K, Hq, Hkv, rope, head_gamma):
    """The projection with the per-head stage equals the projection followed by the standalone per-head stage,
    bit for bit, rstd included."""
    case = synthetic.preattn_case(M, K, Hq, Hkv, 128, seed=M + K, rope=rope, head_gamma=head_gamma)
    t = {k: dev(v) for k, v in case.tensors.items()}
    a = rnl.rms_norm_bf16(t["x"], t["gamma"], EPS)
    hr = torch.empty((M, Hq + Hkv), dtype=torch.float32, device="cuda")
    y = rnl.linear_heads_bf16(a, t["W"], Hq, Hkv, 128, t["gamma_q"], t["gamma_k"], EPS, t["cos"], t["sin"],
                              head_rstd_out=hr)
    p = rnl.linear_bf16(a, t["W"])
    rq = torch.empty((M, Hq), dtype=torch.float32, device="cuda")
    rk = torch.empty((M, max(Hkv, 1)), dtype=torch.float32, device="cuda")
    q = rnl.head_rms_norm_bf16(p.clone(), 0, Hq, 128, t["gamma_q"], EPS, t["cos"], t["sin"], rstd_out=rq)
    if Hkv:
        q = rnl.head_rms_norm_bf16(q, Hq * 128, Hkv, 128, t["gamma_k"], EPS, t["cos"], t["sin"], rstd_out=rk)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), q.view(torch.int16)), f"{int((y != q).sum())} values differ"
    assert torch.equal(hr[:, :Hq], rq) and (Hkv == 0 or torch.equal(hr[:, Hq:], rk))


@pytest.mark.parametrize("T", [4096, 16])
def test_preattn_block_full_size(T):
    """Residual add -> norm -> fused QKV -> per-head norm -> RoPE, K=4096, 32 + 8 + 8 heads of 128."""
    case = synthetic.preattn_block(T)
    y1 = check_preattn_case(case)
    y2 = run_preattn(case)[0]
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), "not deterministic"


# ---------------------------------------------------------------------------
# MLA prolog: query chain + KV branch with one stage-1 pass over x (stacked
# weight).  Stage 1 is an fp32 accumulation rounded to bf16 on both sides, so
# qr, kv and their rstd are compared with the bf16 / relative bounds of the
# chain; y is checked from the device's own qr.
# ---------------------------------------------------------------------------
def run_mla(case):
    x, Wa, Wkv, gq, gkv, Wb = (dev(case[k]) for k in ("x", "W_a", "W_kv", "gamma", "gamma_ckv", "W_b"))
    T, R, Rkv = x.shape[0], Wa.shape[0], Wkv.shape[0]
    W_akv = torch.cat([Wa, Wkv], dim=0).contiguous()
    rq = torch.empty(T, dtype=torch.float32, device="cuda")
    rkv = torch.empty(T, dtype=torch.float32, device="cuda")
    qakv = torch.empty((T, R + Rkv), dtype=torch.bfloat16, device="cuda")
    y, qr, kv = rnl.mla_prolog_bf16(x, W_akv, R, gq, gkv, EPS, Wb, rstd_q_out=rq, rstd_kv_out=rkv, qakv_out=qakv)
    torch.cuda.synchronize()
    return y.cpu(), qr.cpu(), kv.cpu(), rq.cpu().numpy(), rkv.cpu().numpy(), qakv.cpu()


def check_mla_case(case):
    y, qr, kv, rq, rkv, qakv = run_mla(case)
    R = case["W_a"].shape[0]
    xb = bits(case["x"])
    gq = None if case["gamma"] is None else bits(case["gamma"])
    gkv = None if case["gamma_ckv"] is None else bits(case["gamma_ckv"])
    # stage 1 ([q_a | kv], one pass over x): bf16 outputs of fp32 accumulations
    sb = bits(qakv)
    W_akv = np.concatenate([bits(case["W_a"]), bits(case["W_kv"])], axis=0)
    assert_bf16_close(O.bf16_bits_to_f32(sb), O.project_bf16(O.bf16_bits_to_f32(xb), W_akv), case.name + " [q_a | kv]")
    # both norms on the device's stage-1 rows
    check_normed_stage(np.ascontiguousarray(sb[:, :R]), gq, rq, bits(qr), case.name + " qr")
    check_normed_stage(np.ascontiguousarray(sb[:, R:]), gkv, rkv, bits(kv), case.name + " kv")
    # stage 2 from the device's qr
    assert_bf16_close(f32(y), O.project_bf16(O.bf16_bits_to_f32(bits(qr)), bits(case["W_b"])), case.name + " y")
    # end to end against the oracle's own stage 1
    ref = O.mla_prolog(xb, bits(case["W_a"]), gq, EPS, bits(case["W_b"]), bits(case["W_kv"]), gkv)
    assert_bf16_two_roundings(f32(qr), O.bf16_bits_to_f32(ref["qr"]), case.name + " qr end to end")
    assert_bf16_two_roundings(f32(kv), O.bf16_bits_to_f32(ref["kv_out"]), case.name + " kv end to end")
    return y, kv


@pytest.mark.parametrize("T,K,R,Rkv,N,gamma", [
    (37, 256, 64, 32, 80, True),
    (64, 4096, 128, 64, 64, True),      # stage 1 split over K
    (50, 2056, 72, 40, 33, False),      # split with a K tail, ragged R + Rkv
    (4, 7168, 1536, 512, 520, True),    # few tokens: both stages stream their weights
    (300, 520, 136, 16, 260, True),
])
def test_mla_prolog_small(T, K, R, Rkv, N, gamma):
    check_mla_case(synthetic.mla_case(T, K, R, Rkv, N, seed=T + Rkv, gamma=gamma))


def test_mla_prolog_full_size():
    """Query chain + KV branch, T=1024, K=7168, R=1536, Rkv=512, N=24576, every row."""
    case = synthetic.mla_prolog()
    y1, kv1 = check_mla_case(case)
    y2, _, kv2, _, _, _ = run_mla(case)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)) and torch.equal(kv1.view(torch.int16),
                                                                                   kv2.view(torch.int16))


# ---------------------------------------------------------------------------
# MXFP8: E4M3 codes and E8M0 scales of the normed rows bit-exact against the
# oracle (given the device's rstd); the scaled product against the oracle's
# exact sum on the device's own codes.  The scaled MFMA sums its 128 exact
# products per instruction in a wide fixed-point adder rather than as a
# correctly rounded fp32 sum, so the fp32 output is held to a bound relative to
# the sum of the magnitudes of the scaled products.
# ---------------------------------------------------------------------------
def mx_abs_sum(xq, xs, wq, ws):
    xa = np.abs(O.e4m3_decode(xq).astype(np.float64)) * np.repeat(O.e8m0_decode(xs), 64, axis=1)
    wa = np.abs(O.e4m3_decode(wq).astype(np.float64)) * np.repeat(O.e8m0_decode(ws), 64, axis=1)
    return xa @ wa.T


MX_STEP = 128    # products per scaled MFMA (one k-step)
MX_ALIGN = 14    # bits the step's sum keeps below its largest product (truncation width of the model)


def mx_step_max(q, s):
    """Per row and k-step, the largest |scaled value| of an MX operand: [rows, ceil(K/128)]."""
    a = np.abs(O.e4m3_decode(q).astype(np.float64)) * np.repeat(O.e8m0_decode(s), 64, axis=1)
    pad = (-a.shape[1]) % MX_STEP
    a = np.pad(a, ((0, 0), (0, pad)))
    return a.reshape(a.shape[0], -1, MX_STEP).max(axis=2)


def assert_mx_close(y, y_ref, s_abs, step_max, what, K, bf16=False):
    """The scaled product against the oracle's exact sum of the same codes.

    Model of the scaled MFMA: the products are exact (two E4M3 significands and two
    power-of-two scales); one instruction adds the 128 products of a k-step with
    every product truncated to MX_ALIGN bits below the step's largest product, and
    the result is rounded once into the fp32 accumulator.  Per k-step s the error is
    then below 128 * 2^-MX_ALIGN * max_s|t| + 2^-24 |acc_s|, with |acc_s| <= sum|t|;
    step_max[i, j] = sum_s max_s|x| max_s|w| >= sum_s max_s|t|.  y_ref is the exact sum
    rounded to fp32 (2^-24 |y|); a bf16 output rounds once more to nearest (half a bf16
    ulp: 2^-8 relative, 8 significant bits)."""
    steps = -(-K // MX_STEP)
    y_ref = np.asarray(y_ref, np.float64)
    err = np.abs(np.asarray(y, np.float64) - y_ref)
    acc = MX_STEP * 2.0 ** -MX_ALIGN * step_max + steps * 2.0 ** -24 * s_abs + 2.0 ** -24 * np.abs(y_ref)
    bound = acc * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(y_ref) if bf16 else acc
    bad = err > bound
    worst = float(np.max(err / np.maximum(bound, 1e-300)))
    print(f"{what}: worst err/bound {worst:.3g}")
    assert not bad.any(), f"{what}: {int(bad.sum())} outside; worst err/bound {worst:.3g}"


@pytest.mark.parametrize("T,K", [(5, 64), (9, 4160), (33, 8192), (3, 20480), (130, 256)])
@pytest.mark.parametrize("gamma", [True, False])
def test_mx_quant_atom(T, K, gamma):
    case = synthetic.mxfp8_case(T, K, 8, seed=T + K, gamma=gamma)
    x = case.tensors["x"].clone()
    x[T // 2] = 0                                              # all-zero row: scale 2^-127, codes 0
    x[0, :64] = (x[0, :64].float() * 2.0 ** -100).to(torch.bfloat16)  # a tiny block
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    xq, xs = rnl.rms_norm_quant_mxfp8(x.cuda(), dev(case["gamma"]), EPS, rstd_out=rstd)
    torch.cuda.synchronize()
    r = rstd.cpu().numpy()
    xb = bits(x)
    gb = None if case["gamma"] is None else bits(case["gamma"])
    assert_rstd(r, O.rms_norm_rows(xb, gb, EPS)[1], f"mx T{T} K{K}")
    n, _ = O.rms_norm_rows(xb, gb, EPS, rstd=r)
    q_ref, s_ref = O.mx_quant_rows(n)
    assert np.array_equal(xs.cpu().numpy(), s_ref), f"scales differ at {np.argwhere(xs.cpu().numpy() != s_ref)[:4]}"
    bad = xq.cpu().numpy() != q_ref
    assert not bad.any(), f"{int(bad.sum())} codes differ, first at {np.argwhere(bad)[:4]}"


@pytest.mark.parametrize("M,K,N", [(16, 128, 16), (37, 4160, 100), (300, 1024, 520), (1000, 512, 3000),
                                   (40, 8256, 72),     # scales staged in three chunks, K not a multiple of 1024
                                   (260, 12288, 200)])  # three full chunks
def test_linear_mxfp8_atom(M, K, N):
    """The scaled GEMM on random MX operands (full E4M3 range in the activations)."""
    xq = synthetic.e4m3_codes((M, K), 40.0, M + K, 20)
    xs = synthetic.e8m0_codes((M, K // 64), 120, 134, M + K, 21)
    wq = synthetic.e4m3_codes((N, K), 8.0, M + K, 22)
    ws = synthetic.e8m0_codes((N, K // 64), 117, 119, M + K, 23)
    y = rnl.linear_mxfp8(xq.cuda(), xs.cuda(), wq.cuda(), ws.cuda(), out_dtype=torch.float32)
    yb = rnl.linear_mxfp8(xq.cuda(), xs.cuda(), wq.cuda(), ws.cuda())
    torch.cuda.synchronize()
    q, s, w, t = xq.numpy(), xs.numpy(), wq.numpy(), ws.numpy()
    y_ref = O.mx_scaled_mm(q, s, w, t).astype(np.float64)
    s_abs = mx_abs_sum(q, s, w, t)
    sm = mx_step_max(q, s) @ mx_step_max(w, t).T
    assert_mx_close(y.cpu().numpy(), y_ref, s_abs, sm, f"mx gemm {M}x{K}x{N}", K)
    assert_mx_close(f32(yb), y_ref, s_abs, sm, f"mx gemm bf16 {M}x{K}x{N}", K, bf16=True)


@pytest.mark.parametrize("M,K,N", [(37, 4160, 100), (300, 8256, 200), (260, 12288, 520), (4096, 4096, 6144)])
def test_linear_mxfp8_exact_when_representable(M, K, N):
    """Operands whose every partial sum is exactly representable in fp32 leave the
    accumulation no room to round, so the scaled product must equal the oracle's
    exact sum bit for bit (and its bf16 output the nearest-even rounding of it).

    Values: integers in [-4, 4] in both operands, activation scales 2^0..2^4 and
    weight scales 2^-2..2^0 drawn per 64-block, so every product is a multiple of
    2^-2 of magnitude at most 2^8 and every partial sum over K <= 12288 stays below
    2^24 units of 2^-2.  A wrong 64-block scale, a k index that pairs the wrong
    products or a block read from the wrong row changes the sum by whole units."""
    xq = synthetic.e4m3_int_codes((M, K), 4, M + K, 30)
    xs = synthetic.e8m0_codes((M, K // 64), 127, 131, M + K, 31)
    wq = synthetic.e4m3_int_codes((N, K), 4, M + K, 32)
    ws = synthetic.e8m0_codes((N, K // 64), 125, 127, M + K, 33)
    y = rnl.linear_mxfp8(xq.cuda(), xs.cuda(), wq.cuda(), ws.cuda(), out_dtype=torch.float32)
    yb = rnl.linear_mxfp8(xq.cuda(), xs.cuda(), wq.cuda(), ws.cuda())
    torch.cuda.synchronize()
    # at full size the first and last row of every 128-row block (four of every 256-row tile)
    rows = np.arange(M) if M <= 512 else np.sort(np.concatenate([np.arange(0, M, 128), np.arange(127, M, 128)]))
    q, s = xq.numpy()[rows], xs.numpy()[rows]
    y_ref = O.mx_scaled_mm(q, s, wq.numpy(), ws.numpy())
    # the exact sum is an fp32 value: its fp64 evaluation equals its fp32 rounding
    assert np.array_equal(y_ref.astype(np.float64), (O.e4m3_decode(q).astype(np.float64) * np.repeat(
        O.e8m0_decode(s), 64, axis=1)) @ (O.e4m3_decode(wq.numpy()).astype(np.float64) * np.repeat(
            O.e8m0_decode(ws.numpy()), 64, axis=1)).T)
    got = y.cpu().numpy()[rows]
    bad = got.view(np.uint32) != y_ref.view(np.uint32)
    assert not bad.any(), f"{int(bad.sum())} of {bad.size} differ, first at {np.argwhere(bad)[:4]}"
    gotb = yb.cpu().view(torch.int16).numpy().view(np.uint16)[rows]
    assert np.array_equal(gotb, O.f32_to_bf16_bits(y_ref))


def test_linear_mxfp8_two_term_sums_round_once():
    """A k-step holding two non-zero products returns their exact sum rounded once to
    fp32, wherever the small product sits in the step and whatever its block scale:
    the products are exact and nothing below the largest one is lost before the one
    rounding.  (Random steps with many products deviate more; that is the truncation
    the tolerance of the scaled product models.)"""
    cases = []
    for j in (1, 15, 16, 17, 31, 32, 48, 63, 64, 65, 79, 80, 96, 112, 127):
        for code in (0x01, 0x08, 0x18, 0x28, 0x3F):            # 2^-9 (subnormal), 2^-6, 2^-4, 2^-2, 1.875
            for sh in ((0,) if j < 64 else (10, 14, 18, 20, 22, 24, 26)):
                cases.append((j, code, sh))
    M = len(cases)
    xq = torch.zeros((M, 128), dtype=torch.uint8)
    xs = torch.full((M, 2), 127, dtype=torch.uint8)
    for r, (j, code, sh) in enumerate(cases):
        xq[r, 0] = 0x38                                        # 1.0 at k = 0, scale 2^0
        xq[r, j] = code | (0x80 if r % 2 else 0)                # every other case subtracts
        if j >= 64:
            xs[r, 1] = 127 - sh
    wq = torch.full((16, 128), 0x38, dtype=torch.uint8)
    ws = torch.full((16, 2), 127, dtype=torch.uint8)
    y = rnl.linear_mxfp8(xq.cuda(), xs.cuda(), wq.cuda(), ws.cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    y_ref = O.mx_scaled_mm(xq.numpy(), xs.numpy(), wq.numpy(), ws.numpy())
    got = y.cpu().numpy()
    bad = got.view(np.uint32) != y_ref.view(np.uint32)
    assert not bad.any(), [cases[i] for i in np.argwhere(bad.any(axis=1)).ravel()[:6]]


def run_mx(case, out_dtype):
    x, g, Wq, ws = dev(case["x"]), dev(case["gamma"]), dev(case["Wq"]), dev(case["w_scale"])
    T, K = x.shape
    xq = torch.empty((T, K), dtype=torch.uint8, device="cuda")
    xs = torch.empty((T, K // 64), dtype=torch.uint8, device="cuda")
    rstd = torch.empty(T, dtype=torch.float32, device="cuda")
    y = rnl.rmsnorm_linear_mxfp8(x, g, EPS, Wq, ws, out_dtype=out_dtype, xq_out=xq, x_scale_out=xs, rstd_out=rstd)
    torch.cuda.synchronize()
    return y.cpu(), xq.cpu().numpy(), xs.cpu().numpy(), rstd.cpu().numpy()


def check_mx_case(case, rows=None):
    T = case["x"].shape[0]
    rows = np.arange(T) if rows is None else rows
    xb = bits(case["x"])[rows]
    gb = None if case["gamma"] is None else bits(case["gamma"])
    wq, ws = case["Wq"].numpy(), case["w_scale"].numpy()
    y, xq, xs, rstd = run_mx(case, torch.float32)
    assert_rstd(rstd[rows], O.rms_norm_rows(xb, gb, EPS)[1], case.name)
    ref = O.rmsnorm_linear_mxfp8(xb, gb, EPS, wq, ws, rstd=rstd[rows])
    assert np.array_equal(xq[rows], ref["q"]), f"{case.name}: codes differ"
    assert np.array_equal(xs[rows], ref["x_scale"]), f"{case.name}: scales differ"
    s_abs = mx_abs_sum(ref["q"], ref["x_scale"], wq, ws)
    sm = mx_step_max(ref["q"], ref["x_scale"]) @ mx_step_max(wq, ws).T
    K = xb.shape[1]
    assert_mx_close(y.numpy()[rows], ref["y32"].astype(np.float64), s_abs, sm, case.name, K)
    yb, xq2, xs2, _ = run_mx(case, torch.bfloat16)
    assert np.array_equal(xq2, xq) and np.array_equal(xs2, xs)
    assert_mx_close(f32(yb)[rows], ref["y32"].astype(np.float64), s_abs, sm, case.name + " bf16", K, bf16=True)
    return yb


@pytest.mark.parametrize("T,K,N,gamma", [(8, 256, 128, True), (37, 4160, 100, False), (300, 1024, 520, True),
                                         (1, 64, 24, True)])
def test_rmsnorm_linear_mxfp8_small(T, K, N, gamma):
    check_mx_case(synthetic.mxfp8_case(T, K, N, seed=T + N, gamma=gamma))


def test_mxfp8_qkv_full_size():
    """Pre-attention norm + fused QKV in MXFP8, T=4096, K=4096, N=6144, at full size."""
    case = synthetic.mxfp8_qkv()
    y1 = check_mx_case(case)
    y2, _, _, _ = run_mx(case, torch.bfloat16)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16)), "not deterministic"
