"""CPU oracle for the fused RMSNorm -> Linear projection.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the entry
script and the ``cpu_baseline`` leg of the benchmark may import this package.
The product path never calls it and never falls back to it.

The oracle is plain C (``oracle/c/rnl_oracle.c``, loops with double
accumulation, built by ``oracle/build_oracle.py``), reached through the
functions below (``oracle/c_oracle.py``).  ``oracle.numpy_ref`` is a second,
independent implementation of the same definitions in numpy, kept as a
cross-check: every pin runs against both.  Neither shares code with the HIP
path.
"""
from . import rmsnorm_linear as numpy_ref  # noqa: F401
from . import c_oracle as c  # noqa: F401
from .c_oracle import (  # noqa: F401
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    rms_norm_rows,
    rms_norm_rows_mla_order,
    rms_norm_rows_golden_div,
    project_bf16,
    project_fp32,
    quant_rows,
    quant_values,
    int8_gemm,
    int8_gemm_int64,
    dequant,
    rmsnorm_linear_bf16,
    rmsnorm_linear_fp32w,
    rmsnorm_linear_int8,
    norm_proj_chain,
    add_residual,
    add_rmsnorm_linear_bf16,
    add_rmsnorm_linear_fp32w,
    add_rmsnorm_linear_int8,
    rope_rotate_half,
    head_rms_norm,
    preattn_qkv,
    mla_prolog,
    e4m3_decode,
    e4m3_encode,
    e8m0_decode,
    mx_quant_rows,
    mx_scaled_mm,
    rmsnorm_linear_mxfp8,
    set_threads,
    threads,
    cpu_count,
)
