"""CPU oracle for the fused RMSNorm -> Linear projection.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check of the entry
script and the ``cpu_baseline`` leg of the benchmark may import this package.
The product path never calls it and never falls back to it.

Plain numpy, slow and obviously correct; it shares no code with the HIP path.
See ``oracle/rmsnorm_linear.py`` for the definitions and their citations.
"""
from .rmsnorm_linear import (  # noqa: F401
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    rms_norm_rows,
    rstd_variant_a,
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
)
