"""Every entry point on seeded random shapes against the oracle, through the C ABI.

The hand-picked cases of the parity suite cover the workload sizes and the known
boundaries; these draw the sizes at random (fixed seed, so the set is the same on
every run) across the routing boundaries of the library -- one and two tokens,
up to 16 tokens, more; K around the whole-row kernel's 8192 limit; ragged T, N
and K tails; with and without gamma, residual, RoPE; bf16 and fp32 outputs --
and apply the same acceptance rules as the parity suite.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synthetic
from tests.test_gpu_parity import (check_add_bf16_case, check_add_int8_case, check_bf16_case, check_chain_case,
                                   check_fp32w_case, check_int8_case, check_mla_case, check_mx_case,
                                   check_preattn_case)
from tests.test_gpu_parity import test_linear_heads as linear_heads_case

pytestmark = pytest.mark.gpu

_rng = np.random.default_rng(20261203)


def _t():
    """Token counts spread over the kernel families: 1-2, 3-4, 5-16, 17-300."""
    band = _rng.integers(0, 4)
    return int([_rng.integers(1, 3), _rng.integers(3, 5), _rng.integers(5, 17), _rng.integers(17, 301)][band])


def _k(mult, hi=9000):
    return int(_rng.integers(1, hi // mult + 1)) * mult


def _n(hi=700):
    return int(_rng.integers(1, hi + 1))


BF16 = [(_t(), _k(8), _n(), bool(_rng.integers(0, 2)), bool(_rng.integers(0, 2))) for _ in range(14)]
FP32W = [(_t(), _k(8, 20000), _n(64), bool(_rng.integers(0, 2))) for _ in range(5)]
INT8 = [(_t(), _k(16, 6000), _n(), bool(_rng.integers(0, 2))) for _ in range(8)]
ADD = [(_t(), _k(8, 6000), _n(), i % 2 == 1) for i in range(6)]  # alternately bf16 and int8
MX = [(_t(), _k(64, 6000), _n(), bool(_rng.integers(0, 2))) for _ in range(6)]
CHAIN = [(_t(), _k(8, 3000), _k(8, 400), _n(500)) for _ in range(5)]
MLA = [(_t(), _k(8, 3000), _k(8, 300), _k(8, 200), _n(400)) for _ in range(4)]
PREATTN = [(_t(), _k(8, 3000), int(_rng.integers(1, 9)), int(_rng.integers(0, 5)), int(_rng.integers(1, 17)) * 16,
            bool(_rng.integers(0, 2)), bool(_rng.integers(0, 2))) for _ in range(6)]
HEADS = [(int(_rng.integers(17, 600)), _k(8, 3000), int(_rng.integers(1, 9)), int(_rng.integers(0, 5)),
          bool(_rng.integers(0, 2)), bool(_rng.integers(0, 2))) for _ in range(5)]


def _seed(*dims):
    return int(sum(d * (i + 3) for i, d in enumerate(dims)) % 100003)


@pytest.mark.parametrize("T,K,N,gamma,fp32_out", BF16)
def test_bf16(T, K, N, gamma, fp32_out):
    case = synthetic.norm_linear_case(T, K, N, seed=_seed(T, K, N), gamma=gamma)
    check_bf16_case(case, out_dtype=torch.float32 if fp32_out else torch.bfloat16)


@pytest.mark.parametrize("T,K,N,gamma", FP32W)
def test_fp32_weights(T, K, N, gamma):
    check_fp32w_case(synthetic.norm_linear_case(T, K, N, seed=_seed(T, K, N), gamma=gamma, w_dtype="fp32"))


@pytest.mark.parametrize("T,K,N,gamma", INT8)
def test_int8(T, K, N, gamma):
    check_int8_case(synthetic.int8_case(T, K, N, seed=_seed(T, K, N), gamma=gamma))


@pytest.mark.parametrize("T,K,N,int8", ADD)
def test_residual_add(T, K, N, int8):
    if int8:
        K = (K + 15) // 16 * 16
        check_add_int8_case(synthetic.with_residual(synthetic.int8_case(T, K, N, seed=_seed(T, K, N)), seed=T))
    else:
        check_add_bf16_case(synthetic.with_residual(synthetic.norm_linear_case(T, K, N, seed=_seed(T, K, N)), seed=T))


@pytest.mark.parametrize("T,K,N,gamma", MX)
def test_mxfp8(T, K, N, gamma):
    check_mx_case(synthetic.mxfp8_case(T, K, N, seed=_seed(T, K, N), gamma=gamma))


@pytest.mark.parametrize("T,K,R,N", CHAIN)
def test_chain(T, K, R, N):
    check_chain_case(synthetic.chain_case(T, K, R, N, seed=_seed(T, K, R, N)))


@pytest.mark.parametrize("T,K,R,Rkv,N", MLA)
def test_mla_prolog(T, K, R, Rkv, N):
    check_mla_case(synthetic.mla_case(T, K, R, Rkv, N, seed=_seed(T, K, R, Rkv, N)))


@pytest.mark.parametrize("T,K,Hq,Hkv,D,residual,rope", PREATTN)
def test_preattn_block(T, K, Hq, Hkv, D, residual, rope):
    check_preattn_case(synthetic.preattn_case(T, K, Hq, Hkv, D, seed=_seed(T, K, Hq, Hkv, D), residual=residual,
                                              rope=rope))


@pytest.mark.parametrize("M,K,Hq,Hkv,rope,head_gamma", HEADS)
def test_linear_heads_random(M, K, Hq, Hkv, rope, head_gamma):
    """Heads of 128 on the tiled GEMM (more than 16 rows): the per-head epilogue against the projection and the
    standalone per-head stage, bit for bit."""
    linear_heads_case(M, K, Hq, Hkv, rope, head_gamma)
