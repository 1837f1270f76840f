"""Pins of the oracle's e4m3fn encoder and block-scale quantiser.

The quantiser makes the block-scaled GEMM's operands: per row and per 128 K
elements (Blackwell TCGEN05 GEMM tutorial, "进阶" (Advanced): scale
granularity 128 along K) the scale 2^e is the smallest power of two with
absmax <= 448 * 2^e, stored as the e8m0 byte e + 127, and each element is
x * 2^-e rounded once to e4m3fn.  Pinned here against exact rational
rounding, torch's own float8_e4m3fn cast (a library routine), the defining
inequalities, and the degenerate blocks.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads
from _exact import e4m3_values, floor_log2

E4M3_MAX = 448


def rne_e4m3(x: Fraction) -> Fraction:
    """Round to the e4m3fn grid (4 significant bits, emin -6), ties to even."""
    if x == 0:
        return Fraction(0)
    s = -1 if x < 0 else 1
    a = abs(x)
    e = max(floor_log2(a), -6)
    step = Fraction(2) ** (e - 3)
    t = a / step
    n = t.numerator // t.denominator
    r = t - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return s * n * step


def finite_e4m3_bytes():
    return np.array([b for b in range(256) if b & 0x7F != 0x7F], np.uint8)


# --- the encoder ------------------------------------------------------------------

def test_encode_e4m3fn_round_trips_every_finite_pattern():
    b = finite_e4m3_bytes()
    v = e4m3_values(b)
    got = oracle.encode_e4m3fn(v)
    # -0.0 keeps its sign bit; every other pattern comes back as itself.
    assert np.array_equal(got, b)


def test_encode_e4m3fn_halfway_points_round_to_even():
    vals = sorted(set(float(v) for v in e4m3_values(finite_e4m3_bytes()) if v >= 0))
    mids = [(Fraction(a) + Fraction(b)) / 2 for a, b in zip(vals, vals[1:])]
    got = e4m3_values(oracle.encode_e4m3fn(np.array([float(m) for m in mids])))
    for m, g in zip(mids, got):
        assert Fraction(float(g)) == rne_e4m3(m), m


def test_encode_e4m3fn_matches_exact_rounding_on_random_values():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(4000) * np.exp2(rng.integers(-12, 9, 4000))
    x = np.clip(x, -E4M3_MAX, E4M3_MAX)
    got = e4m3_values(oracle.encode_e4m3fn(x))
    for xi, g in zip(x, got):
        assert Fraction(float(g)) == rne_e4m3(Fraction(float(xi)))


def test_encode_e4m3fn_matches_torch_cast():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-10, 8, 20000))).astype(np.float32)
    x = np.clip(x, -E4M3_MAX, E4M3_MAX)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode_e4m3fn(x.astype(np.float64)), ref)


# --- the quantiser ------------------------------------------------------------------

def test_quantise_matches_the_torch_based_input_recipe():
    """workloads.quantize_mxfp8 (frexp on numpy + torch's float8 cast) is an
    independent implementation of the same rule."""
    g = workloads.generator(3)
    x = workloads.randn_f32((48, 1000), g) * torch.logspace(-30, 30, 48)[:, None]
    q_ref, s_ref = workloads.quantize_mxfp8(x)
    q, s = oracle.quantize_mxfp8(x.numpy())
    assert np.array_equal(s, s_ref)
    assert np.array_equal(q, q_ref)


def test_quantise_scale_is_the_smallest_fitting_power_of_two():
    g = workloads.generator(4)
    x = (workloads.randn_f32((32, 512), g) * torch.logspace(-8, 8, 32)[:, None]).numpy()
    q, s = oracle.quantize_mxfp8(x)
    absmax = np.abs(x.astype(np.float64)).reshape(32, 4, 128).max(2)
    e = s.astype(np.int64) - 127
    assert np.all(absmax <= 448.0 * np.exp2(e))
    assert np.all(absmax > 448.0 * np.exp2(e - 1))


def test_quantise_elements_are_one_rounding_of_the_scaled_value():
    g = workloads.generator(5)
    x = (workloads.randn_f32((6, 256), g) * 37.0).numpy()
    q, s = oracle.quantize_mxfp8(x)
    qv = e4m3_values(q)
    for r in range(6):
        for k in range(256):
            e = int(s[r, k // 128]) - 127
            assert Fraction(float(qv[r, k])) == rne_e4m3(Fraction(float(x[r, k])) * Fraction(2) ** -e)


@pytest.mark.parametrize("k", [-20, 0, 5, 100])
def test_quantise_scale_boundaries(k):
    """absmax exactly 448 * 2^k gives e = k and the byte 0x7e for that
    element; one binary32 ulp more gives e = k + 1."""
    top = np.float32(448.0 * 2.0 ** k)
    above = np.nextafter(top, np.float32(np.inf))
    x = np.zeros((2, 128), np.float32)
    x[0, 7], x[1, 7] = top, above
    x[:, 0] = top / 4
    q, s = oracle.quantize_mxfp8(x)
    assert s[0, 0] == k + 127 and q[0, 7] == 0x7E and q[0, 0] == 0x6E  # 112 = 1.75 * 2^6
    assert s[1, 0] == k + 128


def test_quantise_degenerate_blocks():
    K = 144  # two blocks, the second of 16 elements
    x = np.zeros((4, K), np.float32)
    x[1, 130] = -3.0                     # only the short block is non-zero
    x[2, :] = np.float32(2.0 ** -149)    # binary32 subnormals: e clamps at -127
    x[3, 5] = np.float32(-448.0)
    q, s = oracle.quantize_mxfp8(x)
    # All-zero blocks: byte 0 (e = -127) and zero elements.
    assert list(s[0]) == [0, 0] and not q[0].any()
    # 3 <= 448 * 2^-7 = 3.5 but > 448 * 2^-8: e = -7, and -3 * 2^7 = -384 is exact.
    assert s[1, 0] == 0 and s[1, 1] == 127 - 7
    assert e4m3_values(q[1, 130:131])[0] == -384.0
    # 2^-149 * 2^127 = 2^-22 is below half the smallest e4m3fn subnormal (2^-10).
    assert list(s[2]) == [0, 0] and not q[2].any()
    # |-448| = 448 * 2^0: e = 0, byte 0x7e with the sign bit.
    assert s[3, 0] == 127 and q[3, 5] == 0xFE and s[3, 1] == 0


def test_quantise_negative_values_mirror_positive():
    g = workloads.generator(7)
    x = (workloads.randn_f32((8, 300), g) * 5).numpy()
    q1, s1 = oracle.quantize_mxfp8(x)
    q2, s2 = oracle.quantize_mxfp8(-x)
    assert np.array_equal(s1, s2)
    nz = q1 & 0x7F != 0
    assert np.array_equal(q2[nz], q1[nz] ^ 0x80)
