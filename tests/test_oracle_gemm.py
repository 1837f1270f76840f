"""Pins for the oracle GEMMs against things other than the oracle itself.

* closed forms: all-ones inputs give K (rounded once), identity operands
  reproduce the other operand, K = 1 is one rounded product;
* brute force with exact rationals on tiny, non-square shapes (catches a
  dropped term, a wrong sign, a transposed operand or a wrong index);
* invariants: (A.B^T)^T = B.A^T and (A.B)^T = B^T.A^T bit for bit;
* library cross-check: numpy float64 matmul, rounded independently, agrees
  at the workloads' shapes;
* the sampled (one output at a time) entry points equal the full ones;
* block-scaled FP8: exact rational sums, the scale index k/128 per row,
  the e8m0 bias, and scale factoring (one more exponent doubles C exactly);
* IEEE special values: infinities and NaN in the inputs, and a finite sum
  past the output format's largest value.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads
from _exact import BF16, F16, bf16_values, e4m3_values, f16_values, rne

BF16_ONE, F16_ONE = 0x3F80, 0x3C00


def _bf16(x):
    return workloads.to_bits(torch.as_tensor(np.asarray(x, np.float32)).bfloat16())


def _f16(x):
    return workloads.to_bits(torch.as_tensor(np.asarray(x, np.float32)).half())


# --- closed forms --------------------------------------------------------------

@pytest.mark.parametrize("K", [1, 7, 256, 1024, 5000, 8192])
def test_all_ones_gives_K(K):
    M, N = 3, 5
    want_bf16 = rne(Fraction(K), **BF16)
    c = oracle.gemm_bf16_nt(np.full((M, K), BF16_ONE, np.uint16),
                            np.full((N, K), BF16_ONE, np.uint16))
    assert np.all(bf16_values(c) == float(want_bf16))
    c = oracle.gemm_f16_nn(np.full((M, K), F16_ONE, np.uint16),
                           np.full((K, N), F16_ONE, np.uint16))
    assert np.all(f16_values(c) == float(rne(Fraction(K), **F16)))
    if K in (256, 1024, 8192):
        assert float(want_bf16) == K


def test_identity_operands():
    rng = np.random.default_rng(0)
    n = 37
    eye = _bf16(np.eye(n))
    X = _bf16(rng.normal(size=(n, n)))
    # NT with A = I: C[m][n] = B[n][m]   -> C = B^T
    assert np.array_equal(oracle.gemm_bf16_nt(eye, X), X.T)
    # NT with B = I: C = A
    assert np.array_equal(oracle.gemm_bf16_nt(X, eye), X)
    eye16 = _f16(np.eye(n))
    Y = _f16(rng.normal(size=(n, n)))
    assert np.array_equal(oracle.gemm_f16_nn(eye16, Y), Y)     # A = I -> C = B
    assert np.array_equal(oracle.gemm_f16_nn(Y, eye16), Y)     # B = I -> C = A


def test_K1_is_one_rounded_product():
    rng = np.random.default_rng(1)
    A = _bf16(rng.normal(size=(9, 1)))
    B = _bf16(rng.normal(size=(11, 1)))
    c = bf16_values(oracle.gemm_bf16_nt(A, B))
    a, b = bf16_values(A)[:, 0], bf16_values(B)[:, 0]
    for i in range(9):
        for j in range(11):
            assert Fraction(c[i, j]) == rne(Fraction(a[i]) * Fraction(b[j]), **BF16)


# --- brute force with exact rationals --------------------------------------------

SHAPES = [(1, 1, 1), (2, 3, 5), (5, 3, 2), (3, 8, 17), (17, 5, 33), (8, 33, 3), (33, 17, 8)]


def _exact_nt(a, b):
    M, K = a.shape
    N = b.shape[0]
    fa = [[Fraction(float(v)) for v in row] for row in a]
    fb = [[Fraction(float(v)) for v in row] for row in b]
    return [[sum((fa[m][k] * fb[n][k] for k in range(K)), Fraction(0)) for n in range(N)]
            for m in range(M)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("ints", [True, False])
def test_bf16_nt_brute_force(M, N, K, ints):
    rng = np.random.default_rng(M * 10000 + N * 100 + K)
    if ints:
        A, B = _bf16(rng.integers(-4, 5, (M, K))), _bf16(rng.integers(-4, 5, (N, K)))
    else:
        A, B = _bf16(rng.normal(size=(M, K))), _bf16(rng.normal(size=(N, K)))
    C, C64 = oracle.gemm_bf16_nt(A, B, want_f64=True)
    exact = _exact_nt(bf16_values(A), bf16_values(B))
    cv = bf16_values(C)
    a, b = bf16_values(A), bf16_values(B)
    for m in range(M):
        for n in range(N):
            # The binary64 sum is within the recursive-summation bound of the
            # exact sum (exact for these small integer or bf16 products) ...
            bound = K * 2.0 ** -53 * float(np.abs(a[m]) @ np.abs(b[n]))
            assert abs(Fraction(C64[m, n]) - exact[m][n]) <= Fraction(bound)
            # ... and the output is that sum rounded once.
            assert Fraction(cv[m, n]) == rne(Fraction(C64[m, n]), **BF16)
            if Fraction(C64[m, n]) == exact[m][n]:
                assert Fraction(cv[m, n]) == rne(exact[m][n], **BF16)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_f16_nn_brute_force(M, N, K):
    rng = np.random.default_rng(7 + M * 10000 + N * 100 + K)
    A, B = _f16(rng.normal(size=(M, K))), _f16(rng.normal(size=(K, N)))
    C, C64 = oracle.gemm_f16_nn(A, B, want_f64=True)
    a, b = f16_values(A), f16_values(B)
    exact = _exact_nt(a, b.T)          # C = A.B with B given K x N
    cv = f16_values(C)
    for m in range(M):
        for n in range(N):
            assert Fraction(C64[m, n]) == exact[m][n]     # fp16 products: exact here
            assert Fraction(cv[m, n]) == rne(exact[m][n], **F16)


def test_nt_is_not_nn():
    """A transposed-operand mistake would make NT equal NN; it must not."""
    rng = np.random.default_rng(5)
    A = _bf16(rng.normal(size=(4, 6)))
    B = _bf16(rng.normal(size=(6, 6)))
    a, b = bf16_values(A), bf16_values(B)
    c = bf16_values(oracle.gemm_bf16_nt(A, B))
    assert np.allclose(c, a @ b.T, rtol=1e-2, atol=1e-2)
    assert not np.allclose(c, a @ b, rtol=1e-2, atol=1e-2)


# --- invariants -------------------------------------------------------------------

def test_transpose_invariants_bitwise():
    rng = np.random.default_rng(2)
    A = _bf16(rng.normal(size=(45, 70)))
    B = _bf16(rng.normal(size=(31, 70)))
    assert np.array_equal(oracle.gemm_bf16_nt(A, B).T, oracle.gemm_bf16_nt(B, A))
    A16 = _f16(rng.normal(size=(45, 70)))
    B16 = _f16(rng.normal(size=(70, 31)))
    assert np.array_equal(oracle.gemm_f16_nn(A16, B16).T,
                          oracle.gemm_f16_nn(np.ascontiguousarray(B16.T),
                                             np.ascontiguousarray(A16.T)))


# --- library cross-check at the workloads' shapes ------------------------------------

def _check_close_to_numpy(C, C64, ref64, enc, dec):
    # Only the summation order differs: binary64 sums agree to ~1e-16 relative.
    assert np.allclose(C64, ref64, rtol=1e-12, atol=1e-12)
    ref_bits = enc(ref64)
    same = np.mean(C == ref_bits)
    assert same >= 0.9999
    # Where they differ, they are neighbours on the output grid.
    diff = C != ref_bits
    if diff.any():
        d = np.abs(dec(C[diff]) - dec(ref_bits[diff]))
        ulp = np.abs(dec(C[diff])) * 2.0 ** -7 + 1e-30
        assert np.all(d <= ulp)


def test_bf16_nt_256_vs_numpy():
    x = workloads.make_inputs("bf16_nt_256")
    C, C64 = oracle.gemm_bf16_nt(x["A"], x["B"], want_f64=True)
    ref = bf16_values(x["A"]) @ bf16_values(x["B"]).T
    _check_close_to_numpy(C, C64, ref, oracle.encode_bf16, bf16_values)


def test_f16_nn_1024_vs_numpy():
    x = workloads.make_inputs("f16_nn_1024")
    C, C64 = oracle.gemm_f16_nn(x["A"], x["B"], want_f64=True)
    ref = f16_values(x["A"]) @ f16_values(x["B"])
    _check_close_to_numpy(C, C64, ref, oracle.encode_f16, f16_values)


@pytest.mark.parametrize("name", ["bf16_nt_4000x3000x5000", "bf16_nt_4096x4096x8192"])
def test_bf16_nt_large_sampled_vs_numpy(name):
    w = workloads.WORKLOADS[name]
    x = workloads.make_inputs(w)
    rows, cols = workloads.sample_positions(w.M, w.N, 200)
    out, out64 = oracle.gemm_bf16_nt_at(x["A"], x["B"], rows, cols, want_f64=True)
    a = bf16_values(x["A"][rows])
    b = bf16_values(x["B"][cols])
    ref = np.einsum("pk,pk->p", a, b)
    _check_close_to_numpy(out, out64, ref, oracle.encode_bf16, bf16_values)


def test_sampled_equals_full():
    rng = np.random.default_rng(9)
    A, B = _bf16(rng.normal(size=(70, 129))), _bf16(rng.normal(size=(50, 129)))
    C = oracle.gemm_bf16_nt(A, B)
    rows, cols = workloads.sample_positions(70, 50, 300)
    assert np.array_equal(oracle.gemm_bf16_nt_at(A, B, rows, cols), C[rows, cols])
    A16, B16 = _f16(rng.normal(size=(70, 129))), _f16(rng.normal(size=(129, 50)))
    C16 = oracle.gemm_f16_nn(A16, B16)
    assert np.array_equal(oracle.gemm_f16_nn_at(A16, B16, rows, cols), C16[rows, cols])
    x = workloads.make_random("mxfp8_nt", 70, 50, 384, seed=3)
    C8 = oracle.gemm_mxfp8_nt(x["qA"], x["qB"], x["sA"], x["sB"])
    assert np.array_equal(
        oracle.gemm_mxfp8_nt_at(x["qA"], x["qB"], x["sA"], x["sB"], rows, cols), C8[rows, cols])


# --- block-scaled FP8 ---------------------------------------------------------------

def _exact_mx(qA, qB, sA, sB):
    M, K = qA.shape
    N = qB.shape[0]
    a, b = e4m3_values(qA), e4m3_values(qB)
    ea, eb = sA.astype(np.int64) - 127, sB.astype(np.int64) - 127
    fa = [[Fraction(float(a[m, k])) * Fraction(2) ** int(ea[m, k // 128]) for k in range(K)]
          for m in range(M)]
    fb = [[Fraction(float(b[n, k])) * Fraction(2) ** int(eb[n, k // 128]) for k in range(K)]
          for n in range(N)]
    return [[sum((fa[m][k] * fb[n][k] for k in range(K)), Fraction(0)) for n in range(N)]
            for m in range(M)]


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 2, 130), (5, 7, 256), (4, 3, 300)])
def test_mxfp8_brute_force_exact(M, N, K):
    x = workloads.make_random("mxfp8_nt", M, N, K, seed=M + N + K)
    # Different scales per 128-block and per row, so a wrong scale index shows.
    rng = np.random.default_rng(K)
    x["sA"] = rng.integers(120, 135, x["sA"].shape).astype(np.uint8)
    x["sB"] = rng.integers(120, 135, x["sB"].shape).astype(np.uint8)
    C, C64 = oracle.gemm_mxfp8_nt(x["qA"], x["qB"], x["sA"], x["sB"], want_f64=True)
    exact = _exact_mx(x["qA"], x["qB"], x["sA"], x["sB"])
    cv = bf16_values(C)
    for m in range(M):
        for n in range(N):
            # Every term is a multiple of a fixed power of two and the sum is
            # far below 2^53 of them, so the binary64 sum is exact.
            assert Fraction(C64[m, n]) == exact[m][n]
            assert Fraction(cv[m, n]) == rne(exact[m][n], **BF16)


def test_mxfp8_all_ones_with_scales_closed_form():
    K = 384
    one = 0x38                             # e4m3fn 1.0: exponent field 7, fraction 0
    assert e4m3_values(np.array([one], np.uint8))[0] == 1.0
    qA = np.full((2, K), one, np.uint8)
    qB = np.full((3, K), one, np.uint8)
    sA = np.array([[127, 128, 129], [100, 127, 150]], np.uint8)
    sB = np.array([[127, 127, 127], [126, 127, 128], [130, 120, 127]], np.uint8)
    _, C64 = oracle.gemm_mxfp8_nt(qA, qB, sA, sB, want_f64=True)
    for m in range(2):
        for n in range(3):
            want = sum(128 * 2.0 ** (int(sA[m, j]) - 127 + int(sB[n, j]) - 127) for j in range(3))
            assert C64[m, n] == want


def test_mxfp8_scale_factoring_doubles_exactly():
    x = workloads.make_random("mxfp8_nt", 16, 12, 512, seed=11)
    _, C64 = oracle.gemm_mxfp8_nt(x["qA"], x["qB"], x["sA"], x["sB"], want_f64=True)
    _, D64 = oracle.gemm_mxfp8_nt(x["qA"], x["qB"], x["sA"] + 1, x["sB"], want_f64=True)
    assert np.array_equal(D64, 2.0 * C64)
    _, E64 = oracle.gemm_mxfp8_nt(x["qA"], x["qB"], x["sA"] + 1, x["sB"] - 1, want_f64=True)
    assert np.array_equal(E64, C64)


def test_mxfp8_unit_scales_reduce_to_integer_gemm():
    x = workloads.make_integer("mxfp8_nt", 20, 24, 256, seed=4)
    _, C64 = oracle.gemm_mxfp8_nt(x["qA"], x["qB"], x["sA"], x["sB"], want_f64=True)
    a = e4m3_values(x["qA"]).astype(np.int64)
    b = e4m3_values(x["qB"]).astype(np.int64)
    assert np.array_equal(C64, (a @ b.T).astype(np.float64))


def test_mxfp8_4096_sampled_exact():
    w = workloads.WORKLOADS["mxfp8_nt_4096"]
    x = workloads.make_inputs(w)
    rows, cols = workloads.sample_positions(w.M, w.N, 40)
    out, out64 = oracle.gemm_mxfp8_nt_at(x["qA"], x["qB"], x["sA"], x["sB"], rows, cols,
                                         want_f64=True)
    a = e4m3_values(x["qA"][rows]) * np.repeat(2.0 ** (x["sA"][rows].astype(np.int64) - 127),
                                               128, axis=1)
    b = e4m3_values(x["qB"][cols]) * np.repeat(2.0 ** (x["sB"][cols].astype(np.int64) - 127),
                                               128, axis=1)
    for p in range(rows.size):
        exact = sum((Fraction(float(u)) * Fraction(float(v)) for u, v in zip(a[p], b[p])),
                    Fraction(0))
        assert Fraction(out64[p]) == exact
        assert Fraction(float(bf16_values(out[p:p + 1])[0])) == rne(exact, **BF16)


# --- IEEE special values -------------------------------------------------------

def test_special_values_follow_ieee():
    """An infinite element makes its outputs infinite with the sign of the
    product (NaN where the other factor is 0); +inf and -inf terms give NaN;
    a NaN element gives NaN; a finite sum past the output format's largest
    value rounds to infinity (fp16: 128 products of 32 * 32 = 131072 >
    65504)."""
    M, N, K = 4, 3, 8
    A = np.ones((M, K), np.float32)
    B = np.ones((N, K), np.float32)
    B[1, 2], B[2, 2] = -1.0, 0.0
    A[0, 2] = np.inf                          # row 0: +inf, -inf, inf * 0 = NaN
    A[1, 4], A[1, 5] = np.inf, -np.inf        # row 1: inf - inf = NaN
    A[2, 6] = np.nan                          # row 2: NaN
    C = bf16_values(oracle.gemm_bf16_nt(_bf16(A), _bf16(B)))
    assert C[0, 0] == np.inf and C[0, 1] == -np.inf and np.isnan(C[0, 2])
    assert np.isnan(C[1]).all() and np.isnan(C[2]).all()
    assert list(C[3]) == [8.0, 6.0, 7.0]      # row 3: finite, B's -1 and 0 at k = 2
    Ah = np.full((2, 128), 32.0, np.float32)
    Ah[1] = -32.0
    Bh = np.full((128, 2), 32.0, np.float32)
    Ch = f16_values(oracle.gemm_f16_nn(_f16(Ah), _f16(Bh)))
    assert (Ch[0] == np.inf).all() and (Ch[1] == -np.inf).all()
    Ch = f16_values(oracle.gemm_f16_nn(_f16(Ah[:, :127]), _f16(Bh[:127])))
    assert (Ch[0] == np.inf).all()            # 130048: still past 65504
    Ch = f16_values(oracle.gemm_f16_nn(_f16(Ah[:, :63]), _f16(Bh[:63])))
    assert (Ch[0] == 64512.0).all()           # 64512 is an fp16 value: no overflow
