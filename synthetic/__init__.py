"""Seeded synthetic inputs for the fused RMSNorm -> Linear projection workloads.

This module only draws random tensors.  It holds none of the arithmetic of the
method (no norm, no quantisation, no contraction): the HIP path and the CPU
oracle both take their inputs from here and from nowhere else.

Every tensor comes from its own CPU ``torch.Generator`` seeded from
``(seed, stream)``, so a tensor does not change when another one is added or
resized.  Float draws are made in fp32 and stored through torch's own bf16
conversion; int8 weights are drawn uniformly from [-127, 127].

Distributions follow the workload statements: activations x ~ N(0, 1) bf16,
gamma ~ U(0.5, 1.5) bf16, weights W[N, K] ~ N(0, std = 1/sqrt(K)), int8
weights uniform in [-127, 127] with per-output-channel fp32 scales
U(1e-3, 1e-2), eps = 1e-6.  The pages (AT-10 "RMSNorm + Linear (Fused)" and
SK-03 "Linear Projection (Norm->MatMul)") print no dataset; dense iid values
with no sparsity or outliers stand in for the model activations their
operators see.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

EPS = 1e-6

# stream ids: one per tensor role, so that adding a tensor never shifts another
_S_X, _S_GAMMA, _S_W, _S_WSCALE, _S_WA, _S_WB, _S_RES = 1, 2, 3, 4, 5, 6, 7
_S_GQ, _S_GK, _S_ANGLE, _S_WKV, _S_GKV, _S_WSC = 8, 9, 10, 11, 12, 13


def _gen(seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed((int(seed) * 1_000_003 + int(stream)) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def normal(shape, std: float, seed: int, stream: int, dtype=torch.bfloat16) -> torch.Tensor:
    """N(0, std^2) draws, made in fp32 and stored as ``dtype`` (CPU tensor)."""
    t = torch.randn(tuple(shape), generator=_gen(seed, stream), dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype).contiguous()


def normal_on_device(shape, std: float, seed: int, stream: int, device="cuda", dtype=torch.bfloat16) -> torch.Tensor:
    """N(0, std^2) draws made on ``device`` by that device's own torch generator (seeded from ``(seed, stream)``
    like the host draws), in fp32 slabs of at most 2^28 values, each stored as ``dtype``: for operands of several
    GB, too large to draw on the host in a test.  A given (shape, seed, stream) gives the same tensor every time
    on a given device; it is not the host draw of the same arguments."""
    shape = tuple(int(d) for d in shape)
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + int(stream)) & 0x7FFF_FFFF_FFFF_FFFF)
    out = torch.empty(shape, dtype=dtype, device=device)
    row = math.prod(shape[1:])
    slab = max(1, (1 << 28) // max(row, 1))
    for r0 in range(0, shape[0], slab):
        r1 = min(shape[0], r0 + slab)
        t = torch.randn((r1 - r0,) + shape[1:], generator=g, dtype=torch.float32, device=device)
        if std != 1.0:
            t.mul_(std)
        out[r0:r1].copy_(t)
    return out


def uniform(shape, lo: float, hi: float, seed: int, stream: int, dtype=torch.bfloat16) -> torch.Tensor:
    """U(lo, hi) draws, made in fp32 and stored as ``dtype`` (CPU tensor)."""
    t = torch.rand(tuple(shape), generator=_gen(seed, stream), dtype=torch.float32)
    t.mul_(hi - lo).add_(lo)
    return t.to(dtype).contiguous()


def int8_uniform(shape, seed: int, stream: int) -> torch.Tensor:
    """Integers uniform in [-127, 127] as int8 (-128 is never drawn)."""
    return torch.randint(-127, 128, tuple(shape), generator=_gen(seed, stream), dtype=torch.int8)


@dataclass
class Case:
    """One workload instance: CPU tensors plus scalar arguments."""

    name: str
    tensors: dict = field(default_factory=dict)
    eps: float = EPS
    dims: dict = field(default_factory=dict)

    def __getitem__(self, k):
        return self.tensors[k]


def norm_linear_case(T: int, K: int, N: int, seed: int = 0, gamma: bool = True,
                     w_dtype: str = "bf16", name: str | None = None) -> Case:
    """x[T,K] bf16, optional gamma[K] bf16, W[N,K] (bf16 or fp32)."""
    wdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[w_dtype]
    t = {
        "x": normal((T, K), 1.0, seed, _S_X),
        "gamma": uniform((K,), 0.5, 1.5, seed, _S_GAMMA) if gamma else None,
        "W": normal((N, K), 1.0 / math.sqrt(K), seed, _S_W, dtype=wdt),
    }
    return Case(name or f"norm_linear_T{T}_K{K}_N{N}_{w_dtype}", t, EPS, {"T": T, "K": K, "N": N})


def int8_case(T: int, K: int, N: int, seed: int = 0, gamma: bool = True, name: str | None = None) -> Case:
    """x[T,K] bf16, optional gamma[K] bf16, Wq[N,K] int8 in [-127,127], w_scale[N] fp32."""
    t = {
        "x": normal((T, K), 1.0, seed, _S_X),
        "gamma": uniform((K,), 0.5, 1.5, seed, _S_GAMMA) if gamma else None,
        "Wq": int8_uniform((N, K), seed, _S_W),
        "w_scale": uniform((N,), 1e-3, 1e-2, seed, _S_WSCALE, dtype=torch.float32),
    }
    return Case(name or f"int8_T{T}_K{K}_N{N}", t, EPS, {"T": T, "K": K, "N": N})


def with_residual(case: Case, seed: int = 0, std: float = 2.0) -> Case:
    """Adds residual[T,K] bf16 ~ N(0, std^2) (the residual stream the layer input
    is added to before the norm); the other tensors are unchanged."""
    T, K = case["x"].shape
    t = dict(case.tensors)
    t["residual"] = normal((T, K), std, seed, _S_RES)
    return Case(case.name.replace("_T", "_add_T", 1), t, case.eps, dict(case.dims))


def rope_tables(T: int, half: int, seed: int = 0):
    """cos and sin [T, half] fp32 of angles drawn uniformly in [0, 2 pi): the
    rotation tables a caller hands to the rotary embedding (random angles stand
    in for positions times frequencies)."""
    phi = uniform((T, half), 0.0, 2.0 * math.pi, seed, _S_ANGLE, dtype=torch.float32)
    return torch.cos(phi).contiguous(), torch.sin(phi).contiguous()


def preattn_case(T: int, K: int, Hq: int, Hkv: int, D: int, seed: int = 0, residual: bool = False,
                 rope: bool = True, head_gamma: bool = True, name: str | None = None) -> Case:
    """Pre-attention block: x[T,K] bf16, gamma[K], fused QKV weight W[(Hq+2Hkv)D, K],
    head-norm scales gamma_q, gamma_k [D] ~ U(0.5, 1.5), optional residual, and
    rotation tables cos/sin [T, D/2]."""
    N = (Hq + 2 * Hkv) * D
    case = norm_linear_case(T, K, N, seed, name=name or f"preattn_T{T}_K{K}_Hq{Hq}_Hkv{Hkv}_D{D}")
    t = case.tensors
    t["gamma_q"] = uniform((D,), 0.5, 1.5, seed, _S_GQ) if head_gamma else None
    t["gamma_k"] = uniform((D,), 0.5, 1.5, seed, _S_GK) if head_gamma else None
    t["cos"], t["sin"] = rope_tables(T, D // 2, seed) if rope else (None, None)
    case.dims.update({"Hq": Hq, "Hkv": Hkv, "D": D})
    if residual:
        t["residual"] = normal((T, K), 2.0, seed, _S_RES)
    return case


def e4m3_codes(shape, std: float, seed: int, stream: int) -> torch.Tensor:
    """E4M3 bytes of N(0, std^2) draws (torch's float8_e4m3fn conversion), as uint8."""
    t = torch.randn(tuple(shape), generator=_gen(seed, stream), dtype=torch.float32)
    return (t * std).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()


def e4m3_int_codes(shape, vmax: int, seed: int, stream: int) -> torch.Tensor:
    """E4M3 bytes of integers uniform in [-vmax, vmax] (vmax <= 16, so every value is
    exactly representable), as uint8."""
    assert 0 < vmax <= 16
    t = torch.randint(-vmax, vmax + 1, tuple(shape), generator=_gen(seed, stream), dtype=torch.int32)
    return t.to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()


def e8m0_codes(shape, lo: int, hi: int, seed: int, stream: int) -> torch.Tensor:
    """E8M0 scale bytes uniform in [lo, hi] (scale 2^(code - 127)), as uint8."""
    return torch.randint(lo, hi + 1, tuple(shape), generator=_gen(seed, stream), dtype=torch.int32).to(torch.uint8)


def mxfp8_case(T: int, K: int, N: int, seed: int = 0, gamma: bool = True, name: str | None = None) -> Case:
    """x[T,K] bf16, optional gamma[K], MXFP8 weight Wq[N,K] (E4M3 of N(0, 8^2)) with
    E8M0 scales w_scale[N, K/64] in 2^-10 .. 2^-8, so that a weight value has a
    standard deviation near 1/sqrt(4096)."""
    t = {
        "x": normal((T, K), 1.0, seed, _S_X),
        "gamma": uniform((K,), 0.5, 1.5, seed, _S_GAMMA) if gamma else None,
        "Wq": e4m3_codes((N, K), 8.0, seed, _S_W),
        "w_scale": e8m0_codes((N, K // 64), 117, 119, seed, _S_WSC),
    }
    return Case(name or f"mxfp8_T{T}_K{K}_N{N}", t, EPS, {"T": T, "K": K, "N": N})


def chain_case(T: int, K: int, R: int, N: int, seed: int = 0, gamma: bool = True,
               name: str | None = None) -> Case:
    """x[T,K] -> W_a[R,K] -> RMSNorm(R, gamma) -> W_b[N,R]; all bf16."""
    t = {
        "x": normal((T, K), 1.0, seed, _S_X),
        "W_a": normal((R, K), 1.0 / math.sqrt(K), seed, _S_WA),
        "gamma": uniform((R,), 0.5, 1.5, seed, _S_GAMMA) if gamma else None,
        "W_b": normal((N, R), 1.0 / math.sqrt(R), seed, _S_WB),
    }
    return Case(name or f"chain_T{T}_K{K}_R{R}_N{N}", t, EPS, {"T": T, "K": K, "R": R, "N": N})


def mla_case(T: int, K: int, R: int, Rkv: int, N: int, seed: int = 0, gamma: bool = True,
             name: str | None = None) -> Case:
    """The chain of chain_case plus the KV branch: W_kv[Rkv, K] ~ N(0, 1/K), gamma_ckv[Rkv]."""
    case = chain_case(T, K, R, N, seed, gamma, name=name or f"mla_T{T}_K{K}_R{R}_Rkv{Rkv}_N{N}")
    case.tensors["W_kv"] = normal((Rkv, K), 1.0 / math.sqrt(K), seed, _S_WKV)
    case.tensors["gamma_ckv"] = uniform((Rkv,), 0.5, 1.5, seed, _S_GKV) if gamma else None
    case.dims["Rkv"] = Rkv
    return case


# The five workloads, by what they are.
def small_norm_linear(seed: int = 0) -> Case:
    """bf16 RMSNorm + Linear, T=8 tokens, K=256, N=128."""
    return norm_linear_case(8, 256, 128, seed, name="norm_linear_bf16_T8_K256_N128")


def preattn_qkv(T: int = 4096, seed: int = 0) -> Case:
    """Pre-attention norm + fused QKV projection, K=4096, N=6144 (Q 4096 + K 1024 + V 1024)."""
    return norm_linear_case(T, 4096, 6144, seed, name=f"preattn_qkv_bf16_T{T}_K4096_N6144")


def preattn_qkv_add(T: int = 4096, seed: int = 0) -> Case:
    """Residual add -> pre-attention norm -> fused QKV projection, K=4096, N=6144."""
    return with_residual(preattn_qkv(T, seed), seed)


def preattn_block(T: int = 4096, seed: int = 0) -> Case:
    """Residual add -> norm -> fused QKV (32 query heads, 8 key/value heads of 128)
    -> per-head norm of Q and K -> RoPE; K = 4096, N = 6144."""
    return preattn_case(T, 4096, 32, 8, 128, seed, residual=True, name=f"preattn_block_T{T}_K4096_Hq32_Hkv8_D128")


def int8_w8a8(seed: int = 0) -> Case:
    """INT8 W8A8 norm + linear, T=2048, K=4096, N=4096."""
    return int8_case(2048, 4096, 4096, seed, name="int8_w8a8_T2048_K4096_N4096")


def mla_q_chain(seed: int = 0) -> Case:
    """Low-rank query chain x[1024,7168] -> W_a[1536,7168] -> norm -> W_b[24576,1536]."""
    return chain_case(1024, 7168, 1536, 24576, seed, name="mla_q_chain_T1024_K7168_R1536_N24576")


def mxfp8_qkv(T: int = 4096, seed: int = 0) -> Case:
    """Pre-attention norm + fused QKV projection in MXFP8, K=4096, N=6144."""
    return mxfp8_case(T, 4096, 6144, seed, name=f"mxfp8_qkv_T{T}_K4096_N6144")


def mla_prolog(seed: int = 0) -> Case:
    """Low-rank query chain plus the KV branch (kv_lora_rank 512) on the same x."""
    return mla_case(1024, 7168, 1536, 512, 24576, seed, name="mla_prolog_T1024_K7168_R1536_Rkv512_N24576")


def skinny_fp32(seed: int = 0) -> Case:
    """Large-reduction tiny-width norm + linear, no gamma, T=512, K=28672, N=24, fp32 W."""
    return norm_linear_case(512, 28672, 24, seed, gamma=False, w_dtype="fp32",
                            name="skinny_fp32_T512_K28672_N24")
