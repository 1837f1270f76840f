"""The block-scale quantiser that makes the FP8 workload's inputs.

Per row and per 128 K elements: the scale 2^e is the smallest power of two
with absmax <= 448 * 2^e, stored as the e8m0 byte e + 127, and each element is
x * 2^-e rounded to the nearest e4m3fn value.  Checked here by its defining
inequalities, against exact rational rounding, and on the degenerate blocks.
"""
from fractions import Fraction

import numpy as np
import torch

import workloads
from _exact import e4m3_values

E4M3 = dict(p=4, emin=-6)


def _rne_e4m3(x: Fraction) -> Fraction:
    """Exact-rational round-to-nearest-even onto the e4m3fn grid (|x| <= 448)."""
    if x == 0:
        return Fraction(0)
    s = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, E4M3["emin"])
    q = Fraction(2) ** (e - 3)
    t = a / q
    n = t.numerator // t.denominator
    r = t - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return s * n * q


def test_scale_is_minimal_power_of_two():
    g = workloads.generator(0)
    x = workloads.randn_f32((64, 1024), g) * torch.logspace(-6, 6, 64)[:, None]
    q, s = workloads.quantize_mxfp8(x)
    absmax = x.view(64, 8, 128).abs().amax(2).double().numpy()
    e = s.astype(np.int64) - 127
    assert np.all(absmax * 2.0 ** -e <= 448.0)
    assert np.all(absmax * 2.0 ** -(e - 1) > 448.0)


def test_elements_are_rounded_once_to_e4m3():
    g = workloads.generator(1)
    x = workloads.randn_f32((8, 384), g)
    q, s = workloads.quantize_mxfp8(x)
    qv = e4m3_values(q)
    for r in range(8):
        for k in range(384):
            e = int(s[r, k // 128]) - 127
            y = Fraction(float(x[r, k])) * Fraction(2) ** -e
            assert Fraction(float(qv[r, k])) == _rne_e4m3(y)


def test_zero_block_and_exact_powers():
    x = torch.zeros(2, 256)
    x[1, 128:] = 448.0          # absmax exactly 448 -> e = 0
    x[1, 0] = 449.0             # just above -> e = 1
    q, s = workloads.quantize_mxfp8(x)
    assert s[0, 0] == 0 and s[0, 1] == 0 and np.all(q[0] == 0)
    assert s[1, 1] == 127 and s[1, 0] == 128


def test_ragged_K_pads_the_last_block():
    g = workloads.generator(2)
    x = workloads.randn_f32((3, 200), g)
    q, s = workloads.quantize_mxfp8(x)
    assert q.shape == (3, 200) and s.shape == (3, 2)
    absmax = x[:, 128:].abs().amax(1).double().numpy()
    e = s[:, 1].astype(np.int64) - 127
    assert np.all(absmax * 2.0 ** -e <= 448) and np.all(absmax * 2.0 ** -(e - 1) > 448)


def test_workload_scale_range():
    """N(0,1) data: block absmax lies in about [1.6, 5.3], so e is -8..-6."""
    x = workloads.make_inputs("mxfp8_nt_4096")
    for s in (x["sA"], x["sB"]):
        e = s.astype(np.int64) - 127
        assert e.min() >= -8 and e.max() <= -6
