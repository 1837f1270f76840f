"""Exact-arithmetic helpers for the oracle pins (test code only).

Rounding here is written independently of the oracle's C code: it works on
Python ``Fraction`` values with integer floor/compare steps, while the oracle
uses frexp/nearbyint on binary64.
"""
from fractions import Fraction

import numpy as np
import torch

BF16 = dict(p=8, emin=-126, maxfinite=Fraction(2 ** 8 - 1, 2 ** 7) * Fraction(2) ** 127)
F16 = dict(p=11, emin=-14, maxfinite=Fraction(65504))


def floor_log2(a: Fraction) -> int:
    """floor(log2(a)) for a > 0, exactly."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def rne(x: Fraction, p: int, emin: int, maxfinite: Fraction):
    """Round x to the nearest value with p significant bits (ties to even);
    returns a Fraction, or +-inf as float when the rounded value overflows."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = max(floor_log2(a), emin)
    q = Fraction(2) ** (e - (p - 1))
    t = a / q
    n = t.numerator // t.denominator
    r = t - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = n * q
    # Overflow: anything that rounds above the largest finite value.
    if v > maxfinite:
        return sign * float("inf")
    return sign * v


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 through torch's own conversion."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.double().numpy()


def f16_values(bits: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(bits).view(np.float16).astype(np.float64)


def e4m3_values(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.uint8)).view(torch.float8_e4m3fn)
    return t.double().numpy()


def as_fraction(v) -> Fraction:
    return Fraction(float(v))
