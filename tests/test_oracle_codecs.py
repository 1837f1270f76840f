"""Pins for the oracle's codecs (bit pattern <-> binary64).

Decoders are checked exhaustively against library conversions (torch for
bf16 and e4m3fn, numpy for fp16) and against the closed form for e8m0.
Encoders (binary64 -> bf16/fp16, round to nearest even) are checked against
numpy's direct double->half rounding, torch's float->bf16 rounding on
binary32 inputs, and an exact-rational rounding written independently in
``_exact.py`` -- including halfway cases and the double-rounding traps just
next to them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from _exact import BF16, F16, bf16_values, e4m3_values, f16_values, rne

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

ALL16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
ALL8 = np.arange(256, dtype=np.uint16).astype(np.uint8)


def _same(a, b):
    return np.array_equal(a, b, equal_nan=True)


def test_decode_bf16_exhaustive_vs_torch():
    assert _same(oracle.decode_bf16(ALL16), bf16_values(ALL16))


def test_decode_f16_exhaustive_vs_numpy():
    assert _same(oracle.decode_f16(ALL16), f16_values(ALL16))


def test_decode_e4m3fn_exhaustive_vs_torch():
    got = oracle.decode_e4m3fn(ALL8)
    assert _same(got, e4m3_values(ALL8))
    # OCP E4M3: largest finite 448, smallest subnormal 2^-9, only S.1111.111 NaN.
    assert np.nanmax(got) == 448.0 and got[0x7E] == 448.0
    assert got[0x01] == 2.0 ** -9
    assert np.isnan(got).sum() == 2 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def test_decode_e8m0_closed_form():
    got = oracle.decode_e8m0(ALL8)
    for e in range(255):
        assert got[e] == math.ldexp(1.0, e - 127)
    assert np.isnan(got[255])
    if hasattr(torch, "float8_e8m0fnu"):
        t = torch.from_numpy(ALL8[:255].copy()).view(torch.float8_e8m0fnu).double().numpy()
        assert np.array_equal(got[:255], t)


@pytest.mark.parametrize("enc,dec", [(oracle.encode_bf16, bf16_values),
                                     (oracle.encode_f16, f16_values)])
def test_encode_round_trips_every_pattern(enc, dec):
    vals = dec(ALL16)
    finite = np.isfinite(vals)
    assert np.array_equal(enc(vals[finite]), ALL16[finite])
    # Infinities keep their sign; NaN stays NaN.
    back = dec(enc(vals[~finite]))
    assert _same(back, vals[~finite])


def _wide_doubles(n, seed):
    rng = np.random.default_rng(seed)
    mant = rng.uniform(1.0, 2.0, n)
    exps = rng.integers(-140, 130, n)
    sign = rng.choice([-1.0, 1.0], n)
    return sign * np.ldexp(mant, exps)


def test_encode_f16_matches_numpy_direct_rounding():
    x = np.concatenate([_wide_doubles(200000, 0) / 2.0 ** 100,  # many in the f16 range
                        np.random.default_rng(1).normal(size=100000),
                        np.array([65504.0, 65519.99, 65520.0, 2.0 ** -25,
                                  2.0 ** -25 * 1.0000001, 2.0 ** -24 * 1.5, 0.0, -0.0])])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.encode_f16(x), ref)


def test_encode_bf16_matches_torch_on_binary32_inputs():
    x32 = _wide_doubles(200000, 2).astype(np.float32)
    x32 = x32[np.isfinite(x32)]
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.encode_bf16(x32.astype(np.float64)), ref)


@pytest.mark.parametrize("fmt,dec,enc", [(BF16, bf16_values, oracle.encode_bf16),
                                         (F16, f16_values, oracle.encode_f16)])
def test_encode_halfway_and_double_rounding_traps(fmt, dec, enc):
    """Midpoints between neighbours round to the even one; the binary64
    neighbours of a midpoint round away from it (a binary64 -> binary32 ->
    16-bit path would get these wrong)."""
    vals = dec(ALL16)
    pos = np.where(np.isfinite(vals) & ((ALL16 & 0x8000) == 0))[0]
    order = pos[np.argsort(vals[pos], kind="stable")]
    v = vals[order]
    keep = np.diff(v) > 0
    lo, hi = v[:-1][keep], v[1:][keep]
    lo_bits, hi_bits = ALL16[order][:-1][keep], ALL16[order][1:][keep]
    mid = (lo + hi) / 2.0                      # exact in binary64
    even = np.where((lo_bits & 1) == 0, lo_bits, hi_bits)
    assert np.array_equal(enc(mid), even)
    assert np.array_equal(enc(np.nextafter(mid, 0.0)), lo_bits)
    assert np.array_equal(enc(np.nextafter(mid, np.inf)), hi_bits)
    # The same for negatives.
    assert np.array_equal(enc(-mid), even | 0x8000)


@pytest.mark.parametrize("fmt,dec,enc", [(BF16, bf16_values, oracle.encode_bf16),
                                         (F16, f16_values, oracle.encode_f16)])
def test_encode_matches_exact_rational_rounding(fmt, dec, enc):
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.normal(size=3000) * 10.0 ** rng.integers(-8, 6, 3000),
                        _wide_doubles(2000, 4)])
    got = dec(enc(x))
    for xi, gi in zip(x, got):
        want = rne(Fraction(float(xi)), **fmt)
        if isinstance(want, float):
            assert gi == want
        else:
            assert Fraction(float(gi)) == want, (xi, gi, want)


def test_bf16_of_closed_form_integers():
    # 5000 is not a bf16 value: the grid at 2^12 has spacing 2^5, and
    # 5000 / 32 = 156.25 rounds to 156, so 5000 -> 4992.
    assert bf16_values(oracle.encode_bf16([5000.0]))[0] == 4992.0
    for k in (256, 1024, 4096, 8192):
        j = k.bit_length() - 1
        assert oracle.encode_bf16([float(k)])[0] == (127 + j) << 7
        assert oracle.encode_f16([float(k)])[0] == ((15 + j) << 10 if j < 16 else 0x7C00)
