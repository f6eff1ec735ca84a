"""The seeded input generators (CPU): what the workload recipe states about them.

Both the HIP path and the oracle take their inputs from ``synthetic``; these
checks hold it to its stated recipe -- each tensor reproducible from (seed,
stream), independent of which other tensors a case draws, with the stated
distributions and ranges -- so that a change there cannot silently alter every
parity case at once.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import synthetic


def test_draws_are_reproducible_and_streams_independent():
    a = synthetic.norm_linear_case(37, 512, 96, seed=5)
    b = synthetic.norm_linear_case(37, 512, 96, seed=5)
    for k in ("x", "gamma", "W"):
        assert torch.equal(a[k], b[k]), k
    # another role's tensor (gamma dropped, W resized) leaves x unchanged
    c = synthetic.norm_linear_case(37, 512, 200, seed=5, gamma=False)
    assert torch.equal(a["x"], c["x"])
    # another seed changes every tensor
    d = synthetic.norm_linear_case(37, 512, 96, seed=6)
    assert not torch.equal(a["x"], d["x"]) and not torch.equal(a["W"], d["W"])


def test_the_residual_and_heads_do_not_shift_the_base_tensors():
    base = synthetic.norm_linear_case(16, 256, 128, seed=3)
    res = synthetic.with_residual(synthetic.norm_linear_case(16, 256, 128, seed=3), seed=3)
    assert torch.equal(base["x"], res["x"]) and torch.equal(base["W"], res["W"])
    assert res["residual"].shape == base["x"].shape and not torch.equal(res["residual"], base["x"])


def test_distributions_follow_the_recipe():
    K = 4096
    case = synthetic.norm_linear_case(256, K, 512, seed=0)
    x = case["x"].float()
    w = case["W"].float()
    g = case["gamma"].float()
    assert abs(float(x.mean())) < 0.01 and abs(float(x.std()) - 1.0) < 0.01
    assert abs(float(w.std()) * math.sqrt(K) - 1.0) < 0.01  # std 1/sqrt(K)
    assert float(g.min()) >= 0.5 and float(g.max()) <= 1.5
    assert x.dtype == torch.float32 and case["x"].dtype == torch.bfloat16


def test_int8_weights_and_scales():
    case = synthetic.int8_case(4, 2048, 256, seed=1)
    q = case["Wq"].numpy().astype(np.int32)
    assert q.min() >= -127 and q.max() <= 127, "-128 is never drawn"
    assert q.min() == -127 and q.max() == 127
    s = case["w_scale"].numpy()
    assert s.dtype == np.float32 and float(s.min()) >= 1e-3 and float(s.max()) <= 1e-2


def test_normal_on_device_is_deterministic():
    a = synthetic.normal_on_device((300, 64), 0.5, seed=7, stream=2, device="cpu")
    b = synthetic.normal_on_device((300, 64), 0.5, seed=7, stream=2, device="cpu")
    c = synthetic.normal_on_device((300, 64), 0.5, seed=7, stream=3, device="cpu")
    assert a.dtype == torch.bfloat16 and a.shape == (300, 64)
    assert torch.equal(a, b) and not torch.equal(a, c)
    assert abs(float(a.float().std()) - 0.5) < 0.02


@pytest.mark.parametrize("T,half", [(5, 8), (64, 64)])
def test_rope_tables(T, half):
    c, s = synthetic.rope_tables(T, half, seed=2)
    assert c.shape == (T, half) and s.shape == (T, half) and c.dtype == torch.float32
    # cos and sin of the same angles
    assert torch.allclose(c * c + s * s, torch.ones_like(c), atol=1e-6)
