"""Small test helpers: tensor <-> numpy bit views and ulp distances."""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 CPU tensor -> uint16 bit patterns."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().to(torch.float32).numpy()


def bf16_from_bits(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def ulp_diff(a, b) -> np.ndarray:
    """Distance in units of fp32 ulps between finite fp32 arrays (ordered ints)."""
    ia = np.asarray(a, dtype=np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, dtype=np.float32).view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def fraction_to_f32(fr: Fraction) -> np.float32:
    """Correctly rounded (nearest, ties to even) fp32 of an exact rational.

    Written from the definition of binary32: 24 significant bits, normal
    exponents only (the tests never reach subnormals or overflow)."""
    if fr == 0:
        return np.float32(0.0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # find e with 2^e <= a < 2^(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    scale = Fraction(2) ** (e - 23)
    m = a / scale  # in [2^23, 2^24)
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return np.float32(sign * float(fl * scale))
