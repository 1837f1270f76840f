"""Pins of the oracle's block-scaled FP4 (MXFP4) GEMM and of its input recipe.

E2M1 elements, two per byte (element 2i in the low nibble of byte i), one
e8m0 scale per 32 K elements.  Every product of two scaled E2M1 values is a
power of two times a small integer, so the binary64 sums here are exact:
the oracle must equal exact rational arithmetic written independently here
(with its own unpacking of the nibbles), bit for bit.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads
from _exact import bf16_values, rne, BF16


def e2m1_exact(code: int) -> Fraction:
    """The OCP E2M1 value of a 4-bit code, from its definition."""
    s = -1 if code & 8 else 1
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        return s * Fraction(m, 2)
    return s * Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))


def unpack(q: np.ndarray, K: int) -> np.ndarray:
    """Packed bytes (R, K/2) -> codes (R, K): low nibble first."""
    out = np.empty((q.shape[0], K), np.int64)
    out[:, 0::2] = q & 15
    out[:, 1::2] = q >> 4
    return out


def exact_gemm(qA, qB, sA, sB, K):
    a, b = unpack(qA, K), unpack(qB, K)
    M, N = a.shape[0], b.shape[0]
    C = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += (e2m1_exact(int(a[m, k])) * Fraction(2) ** (int(sA[m, k // 32]) - 127) *
                        e2m1_exact(int(b[n, k])) * Fraction(2) ** (int(sB[n, k // 32]) - 127))
            C[m][n] = acc
    return C


def test_decode_every_code():
    codes = np.arange(16, dtype=np.uint8)
    got = oracle.decode_e2m1(codes)
    assert [Fraction(float(v)) for v in got] == [e2m1_exact(c) for c in range(16)]
    assert sorted(set(abs(float(v)) for v in got)) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (3, 2, 64), (5, 4, 96), (2, 7, 160)])
def test_brute_force_exact(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    qA = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    qB = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sA = rng.integers(120, 135, (M, K // 32), dtype=np.uint8)
    sB = rng.integers(120, 135, (N, K // 32), dtype=np.uint8)
    C, C64 = oracle.gemm_mxfp4_nt(qA, qB, sA, sB, want_f64=True)
    ref = exact_gemm(qA, qB, sA, sB, K)
    for m in range(M):
        for n in range(N):
            assert Fraction(float(C64[m, n])) == ref[m][n]
            want = rne(ref[m][n], BF16["p"], BF16["emin"], BF16["maxfinite"])
            assert Fraction(float(bf16_values(C[m:m + 1, n:n + 1])[0, 0])) == want


def test_element_order_inside_a_byte():
    """A code in the low nibble of byte 0 is element 0, in the high nibble
    element 1: paired with a B that is non-zero only at element 1, only the
    high nibble contributes."""
    qA = np.zeros((1, 16), np.uint8)
    qB = np.zeros((1, 16), np.uint8)
    qA[0, 0] = 0x2 | (0x6 << 4)      # element 0 = 1.0, element 1 = 4.0
    qB[0, 0] = 0x4 << 4              # element 1 = 2.0, element 0 = 0
    s = np.full((1, 1), 127, np.uint8)
    _, C64 = oracle.gemm_mxfp4_nt(qA, qB, s, s, want_f64=True)
    assert C64[0, 0] == 8.0


def test_scale_applies_per_32_elements():
    K = 64
    qA = np.full((1, K // 2), 0x22, np.uint8)   # every element 1.0
    qB = np.full((1, K // 2), 0x22, np.uint8)
    sA = np.array([[127, 129]], np.uint8)       # 2^0 for k < 32, 2^2 above
    sB = np.array([[126, 127]], np.uint8)       # 2^-1, then 2^0
    _, C64 = oracle.gemm_mxfp4_nt(qA, qB, sA, sB, want_f64=True)
    assert C64[0, 0] == 32 * 0.5 + 32 * 4.0


def test_all_ones_gives_K():
    for K in (32, 256, 4096):
        q = np.full((2, K // 2), 0x22, np.uint8)
        s = np.full((2, K // 32), 127, np.uint8)
        C, C64 = oracle.gemm_mxfp4_nt(q, q, s, s, want_f64=True)
        assert np.all(C64 == K)


def test_transpose_invariant_bitwise():
    x = workloads.make_random("mxfp4_nt", 24, 40, 128, seed=3)
    C1 = oracle.gemm_mxfp4_nt(x["qA"], x["qB"], x["sA"], x["sB"])
    C2 = oracle.gemm_mxfp4_nt(x["qB"], x["qA"], x["sB"], x["sA"])
    assert np.array_equal(C1.T, C2)


def test_sampled_equals_full_and_exact_at_workload_size():
    w = workloads.WORKLOADS["mxfp4_nt_4096"]
    x = workloads.make_inputs(w)
    rows, cols = workloads.sample_positions(w.M, w.N, 6, seed=3)
    out, out64 = oracle.gemm_mxfp4_nt_at(x["qA"], x["qB"], x["sA"], x["sB"], rows, cols, want_f64=True)
    a, b = unpack(x["qA"][rows], w.K), unpack(x["qB"][cols], w.K)
    vals = np.array([float(e2m1_exact(c)) for c in range(16)])
    for p in range(rows.size):
        sa = np.repeat(np.exp2(x["sA"][rows[p]].astype(np.float64) - 127), 32)
        sb = np.repeat(np.exp2(x["sB"][cols[p]].astype(np.float64) - 127), 32)
        terms = [Fraction(float(t)) for t in vals[a[p]] * sa * vals[b[p]] * sb]
        assert Fraction(float(out64[p])) == sum(terms, Fraction(0))


def test_input_recipe_scale_is_minimal_and_rounding_is_exact():
    g = workloads.generator(8)
    x = workloads.randn_f32((16, 256), g) * torch.logspace(-6, 6, 16)[:, None]
    q, s = workloads.quantize_mxfp4(x)
    codes = unpack(q, 256)
    e = s.astype(np.int64) - 127
    absmax = np.abs(x.double().numpy()).reshape(16, 8, 32).max(2)
    assert np.all(absmax <= 6.0 * np.exp2(e)) and np.all(absmax > 6.0 * np.exp2(e - 1))
    grid = [e2m1_exact(c) for c in range(8)]
    for r in range(16):
        for k in range(0, 256, 7):
            y = Fraction(float(x[r, k])) * Fraction(2) ** -int(e[r, k // 32])
            got = e2m1_exact(int(codes[r, k]))
            # nearest magnitude, ties to the even code
            a = abs(y)
            best = min(range(8), key=lambda c: (abs(grid[c] - a), c % 2))
            assert abs(got) == grid[best] and (got == 0 or (got < 0) == (y < 0))
