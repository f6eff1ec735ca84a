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


def parse_fraction(tok: str) -> float:
    """A fixture value written as an exact decimal or as p/q."""
    if "/" in tok:
        a, b = tok.split("/")
        return float(Fraction(a) / Fraction(b))
    return float(tok)


def golden_cases(path: str) -> list[dict]:
    """Cases of a tests/golden fixture: "case <name>" opens a case; "K", "eps",
    "gamma" and per-row "x", "q", "x_scale" lines follow."""
    cases, cur = [], None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        if key == "case":
            cur = {"name": vals[0], "x": [], "q": [], "x_scale": []}
            cases.append(cur)
        elif key == "K":
            cur[key] = int(vals[0])
        elif key == "eps":
            cur[key] = float(vals[0])
        elif key == "gamma":
            cur[key] = [parse_fraction(v) for v in vals]
        elif key in ("x", "q"):
            cur[key].append([parse_fraction(v) for v in vals])
        elif key == "x_scale":
            cur[key].append(parse_fraction(vals[0]))
    return cases
