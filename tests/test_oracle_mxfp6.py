"""Pins of the oracle's block-scaled FP6 (MXFP6) GEMM and of its input recipe.

FP6 elements of one type (OCP E2M3 or E3M2) packed densely, element k at bits
6k .. 6k+5 of the row read as a little-endian bit string; one e8m0 scale per
32 K elements.  Every product of two scaled FP6 values is a power of two
times a small integer; with the scale ranges used here the binary64 sums are
exact, so the oracle must equal exact rational arithmetic written
independently here (with its own decoding and its own unpacking), bit for bit.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads
from _exact import bf16_values, rne, BF16

FORMATS = {"e2m3": (2, 1), "e3m2": (3, 3)}   # exponent bits, bias


def fp6_exact(code: int, fmt: str) -> Fraction:
    """The OCP FP6 value of a 6-bit code, from its definition."""
    ebits, bias = FORMATS[fmt]
    mbits = 5 - ebits
    s = -1 if code & 32 else 1
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    if e == 0:
        return s * Fraction(m, 1 << mbits) * Fraction(2) ** (1 - bias)
    return s * (1 + Fraction(m, 1 << mbits)) * Fraction(2) ** (e - bias)


def unpack(q: np.ndarray, K: int) -> np.ndarray:
    """Packed rows -> codes, through one big little-endian integer per row."""
    out = np.empty((q.shape[0], K), np.int64)
    for r in range(q.shape[0]):
        v = int.from_bytes(bytes(q[r]), "little")
        for k in range(K):
            out[r, k] = (v >> (6 * k)) & 63
    return out


def exact_gemm(qA, qB, sA, sB, K, fmt):
    a, b = unpack(qA, K), unpack(qB, K)
    M, N = a.shape[0], b.shape[0]
    C = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += (fp6_exact(int(a[m, k]), fmt) * Fraction(2) ** (int(sA[m, k // 32]) - 127) *
                        fp6_exact(int(b[n, k]), fmt) * Fraction(2) ** (int(sB[n, k // 32]) - 127))
            C[m][n] = acc
    return C


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_decode_every_code(fmt):
    codes = np.arange(64, dtype=np.uint8)
    got = oracle.decode_fp6(codes, fmt)
    assert [Fraction(float(v)) for v in got] == [fp6_exact(c, fmt) for c in range(64)]


def test_named_values():
    e2m3 = oracle.decode_fp6(np.arange(32, dtype=np.uint8), "e2m3")
    e3m2 = oracle.decode_fp6(np.arange(32, dtype=np.uint8), "e3m2")
    assert e2m3.max() == 7.5 and e2m3[1] == 0.125 and e2m3[8] == 1.0
    assert e3m2.max() == 28.0 and e3m2[1] == 0.0625 and e3m2[12] == 1.0
    # 32 distinct non-negative magnitudes, increasing with the code.
    assert np.all(np.diff(e2m3) > 0) and np.all(np.diff(e3m2) > 0)


def test_unpack_bit_order():
    rng = np.random.default_rng(4)
    q = rng.integers(0, 256, (5, 48), dtype=np.uint8)     # K = 64
    assert np.array_equal(oracle.unpack_fp6(q, 64), unpack(q, 64))
    codes = rng.integers(0, 64, (3, 96))
    assert np.array_equal(oracle.unpack_fp6(workloads.pack_fp6(codes), 96), codes)


def test_element_order_inside_the_bytes():
    """Element 0 is the low 6 bits of byte 0; element 1 the top 2 bits of
    byte 0 and the low 4 of byte 1: a B that is non-zero only at element 1
    picks out A's element 1."""
    K = 32
    qA = np.zeros((1, 24), np.uint8)
    qB = np.zeros((1, 24), np.uint8)
    one, two = 8, 16                       # E2M3 codes of 1.0 and 2.0
    bitsA = one | (two << 6)               # element 0 = 1.0, element 1 = 2.0
    qA[0, 0], qA[0, 1] = bitsA & 255, bitsA >> 8
    bitsB = one << 6                       # element 1 = 1.0
    qB[0, 0], qB[0, 1] = bitsB & 255, bitsB >> 8
    s = np.full((1, 1), 127, np.uint8)
    _, C64 = oracle.gemm_mxfp6_nt(qA, qB, s, s, "e2m3", K=K, want_f64=True)
    assert C64[0, 0] == 2.0


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (3, 2, 64), (2, 5, 96), (2, 3, 160)])
def test_brute_force_exact(fmt, M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K + len(fmt))
    qA = rng.integers(0, 256, (M, K // 4 * 3), dtype=np.uint8)
    qB = rng.integers(0, 256, (N, K // 4 * 3), dtype=np.uint8)
    sA = rng.integers(124, 131, (M, K // 32), dtype=np.uint8)
    sB = rng.integers(124, 131, (N, K // 32), dtype=np.uint8)
    C, C64 = oracle.gemm_mxfp6_nt(qA, qB, sA, sB, fmt, want_f64=True)
    ref = exact_gemm(qA, qB, sA, sB, K, fmt)
    for m in range(M):
        for n in range(N):
            assert Fraction(float(C64[m, n])) == ref[m][n]
            want = rne(ref[m][n], BF16["p"], BF16["emin"], BF16["maxfinite"])
            assert Fraction(float(bf16_values(C[m:m + 1, n:n + 1])[0, 0])) == want


def test_scale_applies_per_32_elements():
    K = 64
    codes = np.full((1, K), 8)             # E2M3 1.0 everywhere
    q = workloads.pack_fp6(codes)
    sA = np.array([[127, 129]], np.uint8)  # 2^0 for k < 32, 2^2 above
    sB = np.array([[126, 127]], np.uint8)  # 2^-1, then 2^0
    _, C64 = oracle.gemm_mxfp6_nt(q, q, sA, sB, "e2m3", want_f64=True)
    assert C64[0, 0] == 32 * 0.5 + 32 * 4.0


@pytest.mark.parametrize("fmt,one", [("e2m3", 8), ("e3m2", 12)])
def test_all_ones_gives_K(fmt, one):
    for K in (32, 256, 4096):
        q = workloads.pack_fp6(np.full((2, K), one))
        s = np.full((2, K // 32), 127, np.uint8)
        _, C64 = oracle.gemm_mxfp6_nt(q, q, s, s, fmt, want_f64=True)
        assert np.all(C64 == K)


def test_formats_differ_on_the_same_bits():
    x = workloads.make_random("mxfp6_e2m3_nt", 8, 8, 64, seed=2)
    c1 = oracle.gemm_mxfp6_nt(x["qA"], x["qB"], x["sA"], x["sB"], "e2m3")
    c2 = oracle.gemm_mxfp6_nt(x["qA"], x["qB"], x["sA"], x["sB"], "e3m2")
    assert not np.array_equal(c1, c2)


@pytest.mark.parametrize("kind", ["mxfp6_e2m3_nt", "mxfp6_e3m2_nt"])
def test_transpose_invariant_bitwise(kind):
    x = workloads.make_random(kind, 24, 40, 128, seed=3)
    fmt = workloads.fp6_format(kind)
    C1 = oracle.gemm_mxfp6_nt(x["qA"], x["qB"], x["sA"], x["sB"], fmt)
    C2 = oracle.gemm_mxfp6_nt(x["qB"], x["qA"], x["sB"], x["sA"], fmt)
    assert np.array_equal(C1.T, C2)


def test_sampled_equals_full_and_exact_at_workload_size():
    w = workloads.WORKLOADS["mxfp6_e2m3_nt_4096"]
    x = workloads.make_inputs(w)
    rows, cols = workloads.sample_positions(w.M, w.N, 4, seed=3)
    out, out64 = oracle.gemm_mxfp6_nt_at(x["qA"], x["qB"], x["sA"], x["sB"], rows, cols, "e2m3", want_f64=True)
    vals = [fp6_exact(c, "e2m3") for c in range(64)]
    for p in range(rows.size):
        a = unpack(x["qA"][rows[p]:rows[p] + 1], w.K)[0]
        b = unpack(x["qB"][cols[p]:cols[p] + 1], w.K)[0]
        total = Fraction(0)
        for k in range(w.K):
            total += (vals[a[k]] * Fraction(2) ** (int(x["sA"][rows[p], k // 32]) - 127) *
                      vals[b[k]] * Fraction(2) ** (int(x["sB"][cols[p], k // 32]) - 127))
        assert Fraction(float(out64[p])) == total
    full = oracle.gemm_mxfp6_nt(x["qA"][rows[:6]], x["qB"][cols[:6]], x["sA"][rows[:6]], x["sB"][cols[:6]], "e2m3")
    assert np.array_equal(np.diag(full), out[:6])


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2"])
def test_input_recipe_scale_is_minimal_and_rounding_is_exact(fmt):
    vmax = {"e2m3": Fraction(15, 2), "e3m2": Fraction(28)}[fmt]
    g = workloads.generator(8)
    x = workloads.randn_f32((16, 256), g) * torch.logspace(-6, 6, 16)[:, None]
    q, s = workloads.quantize_mxfp6(x, fmt)
    codes = unpack(q, 256)
    e = s.astype(np.int64) - 127
    for r in range(16):
        for blk in range(8):
            absmax = max(abs(Fraction(float(v))) for v in x[r, 32 * blk:32 * blk + 32])
            assert absmax <= vmax * Fraction(2) ** int(e[r, blk])
            assert absmax > vmax * Fraction(2) ** int(e[r, blk] - 1)
    grid = [fp6_exact(c, fmt) for c in range(32)]
    for r in range(16):
        for k in range(0, 256, 5):
            y = Fraction(float(x[r, k])) * Fraction(2) ** -int(e[r, k // 32])
            got = fp6_exact(int(codes[r, k]), fmt)
            best = min(range(32), key=lambda c: (abs(grid[c] - abs(y)), c % 2))
            assert abs(got) == grid[best] and (got == 0 or (got < 0) == (y < 0))


@pytest.mark.parametrize("kind", ["mxfp6_e2m3_nt", "mxfp6_e3m2_nt"])
def test_integer_inputs_are_exact(kind):
    x = workloads.make_integer(kind, 6, 5, 96, seed=1)
    fmt = workloads.fp6_format(kind)
    vals = oracle.decode_fp6(oracle.unpack_fp6(x["qA"], 96), fmt)
    assert set(np.unique(vals)) <= {-2.0, -1.0, 0.0, 1.0, 2.0}
    _, C64 = oracle.gemm_mxfp6_nt(x["qA"], x["qB"], x["sA"], x["sB"], fmt, want_f64=True)
    a = vals.reshape(6, 96)
    b = oracle.decode_fp6(oracle.unpack_fp6(x["qB"], 96), fmt).reshape(5, 96)
    assert np.array_equal(C64, a @ b.T)
