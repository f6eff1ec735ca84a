"""The allocation-free entry point (rmsnorm_linear_bf16_noalloc) through the C
ABI: its outputs equal those of rmsnorm_linear_bf16 (same kernels, caller
workspace) bit for bit, on two calls in a row, the second with a smaller input,
for each kernel family that uses scratch (the norm pre-pass + tiled GEMM, the
pre-pass + weight streaming, the fp32-weight split-K path) and for the
whole-row kernel that uses none; sizes beyond the scratch are rejected."""
from __future__ import annotations

import pytest
import torch

import rmsnorm_linear_projection_amd as rnl
import synthetic

pytestmark = pytest.mark.gpu

EPS = 1e-6


def dev(t):
    return None if t is None else t.cuda()


def both(case, out_dtype):
    """(y, rstd) of the workspace entry point and of the allocation-free one."""
    x, g, W = dev(case["x"]), dev(case["gamma"]), dev(case["W"])
    T, N = x.shape[0], W.shape[0]
    r1 = torch.empty(T, dtype=torch.float32, device="cuda")
    y1 = rnl.rmsnorm_linear_bf16(x, g, EPS, W, out_dtype=out_dtype, rstd_out=r1)
    y2 = torch.full((T, N), float("nan"), dtype=out_dtype, device="cuda")
    r2 = torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    rnl.rmsnorm_linear_bf16_noalloc(x, g, EPS, W, y2, rstd_out=r2)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before, "the allocation-free call allocated through torch"
    return y1.cpu(), r1.cpu(), y2.cpu(), r2.cpu()


def same_bits(a, b):
    return torch.equal(a.view(torch.uint8), b.view(torch.uint8))


@pytest.mark.parametrize("big,small,w_dtype,out_dtype", [
    ((4096, 4096, 6144), (300, 1032, 200), "bf16", torch.bfloat16),  # pre-pass + tiled GEMM, 32 MiB of scratch
    ((16, 4096, 6144), (8, 256, 128), "bf16", torch.bfloat16),      # pre-pass + weight streaming
    ((512, 28672, 24), (70, 4104, 33), "fp32", torch.float32),       # fp32 weights: split-K partials
    ((2, 4096, 6144), (1, 520, 300), "bf16", torch.float32),         # whole-row kernel (no scratch used)
])
def test_noalloc_matches_workspace_entry_point(big, small, w_dtype, out_dtype):
    for i, (T, K, N) in enumerate((big, small)):
        case = synthetic.norm_linear_case(T, K, N, seed=T + K + N + i, gamma=(w_dtype == "bf16"), w_dtype=w_dtype)
        y1, r1, y2, r2 = both(case, out_dtype)
        assert same_bits(y1, y2), f"call {i} ({T}, {K}, {N}): outputs differ from rmsnorm_linear_bf16"
        assert same_bits(r1, r2), f"call {i} ({T}, {K}, {N}): rstd differs"


def test_noalloc_rejects_sizes_beyond_scratch():
    cap = rnl.noalloc_scratch_bytes()
    assert cap == 32 << 20
    T, K = 4097, 4096  # T * K * 2 bytes of normed rows: just over the scratch
    x = torch.zeros((T, K), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((8, K), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, 8), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rnl.RnlError) as e:
        rnl.rmsnorm_linear_bf16_noalloc(x, None, EPS, W, y)
    assert e.value.status == -6  # RNL_ERR_WORKSPACE
