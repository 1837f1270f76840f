"""gemm_bf16 / gemm_f16: every operand storage (NN, NT, TN, TT) with row
strides, against the oracle.

The oracle takes op(A) as M x K and op(B) as N x K (bf16) or K x N (fp16);
the tests build those from the stored arrays by transposing and slicing
(data movement only).  Stored rows are padded past their valid length with
NaN, so a kernel that read padding would produce NaN and fail; C is written
inside a larger buffer whose other elements must not change.
"""
import numpy as np
import pytest
import torch

import dense_tiled_gemm_bf16_amd as tg
import oracle
import workloads
from _exact import bf16_values, f16_values

pytestmark = pytest.mark.gpu

RTOL = ATOL = 1e-2
NAN_BITS = {"bf16": 0x7FC0, "f16": 0x7E00}
TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    tg.init()
    yield
    tg.set_tile(0, 0)


def values(dt, bits):
    return bf16_values(bits) if dt == "bf16" else f16_values(bits)


def random_bits(dt, shape, seed, integer):
    g = workloads.generator(seed)
    if integer:
        x = torch.randint(-2, 3, shape, generator=g).to(TORCH_DT[dt])
        return workloads.to_bits(x)
    return workloads.randn_bits(shape, TORCH_DT[dt], g)


def stored(valid_bits, ld, dt):
    """valid (rows x cols) inside rows x ld, padding NaN."""
    rows, cols = valid_bits.shape
    out = np.full((rows, ld), NAN_BITS[dt], np.uint16)
    out[:, :cols] = valid_bits
    return out


def reference(dt, opA, opB):
    """opA M x K, opB K x N (bits) -> oracle output bits."""
    if dt == "bf16":
        return oracle.gemm_bf16_nt(opA, np.ascontiguousarray(opB.T))
    return oracle.gemm_f16_nn(opA, opB)


def run_general(dt, ta, tb, M, N, K, seed, integer, lda_pad=8, ldb_pad=16, ldc_pad=24):
    opA = random_bits(dt, (M, K), seed, integer)
    opB = random_bits(dt, (K, N), seed + 1, integer)
    a_st = opA.T if ta else opA          # as stored
    b_st = opB.T if tb else opB
    lda, ldb, ldc = a_st.shape[1] + lda_pad, b_st.shape[1] + ldb_pad, N + ldc_pad
    A = torch.from_numpy(stored(np.ascontiguousarray(a_st), lda, dt).view(np.int16)).cuda()
    B = torch.from_numpy(stored(np.ascontiguousarray(b_st), ldb, dt).view(np.int16)).cuda()
    guard = 1024
    Cbuf = torch.full((guard + M * ldc + guard,), 0x3C00, dtype=torch.int16, device="cuda")
    C = Cbuf[guard:guard + M * ldc]
    fn = tg.lib().gemm_bf16 if dt == "bf16" else tg.lib().gemm_f16
    print(f"[gpu] gemm_{dt} ta={ta} tb={tb} M={M} N={N} K={K} lda={lda} ldb={ldb} ldc={ldc}", flush=True)
    rc = fn(ta, tb, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), ldc, None)
    assert rc == 0, tg.last_error()
    torch.cuda.synchronize()
    cb = Cbuf.cpu().numpy().view(np.uint16)
    assert np.all(cb[:guard] == 0x3C00) and np.all(cb[guard + M * ldc:] == 0x3C00), "wrote outside C"
    got = cb[guard:guard + M * ldc].reshape(M, ldc)
    assert np.all(got[:, N:] == 0x3C00), "wrote into C's row padding"
    return got[:, :N], reference(dt, opA, opB)


def check(dt, got, ref, integer, what):
    if integer:
        bad = np.argwhere(got != ref)
        assert bad.size == 0, f"{what}: {len(bad)} differ, first {bad[0]}"
    else:
        g, r = values(dt, got), values(dt, ref)
        ok = np.abs(g - r) <= ATOL + RTOL * np.abs(r)
        assert ok.all(), f"{what}: {int((~ok).sum())} outside tolerance, max err {np.nanmax(np.abs(g - r))}"


LAYOUTS = [(0, 0), (0, 1), (1, 0), (1, 1)]


def shapes_for(tb):
    return [(256, 256), (128, 128), (64, 64)] + ([(256, 192)] if tb else [])


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_layouts_every_tile_shape(dt, ta, tb):
    for tm, tn in shapes_for(tb):
        tg.set_tile(tm, tn)
        for (M, N, K) in [(200, 136, 72), (296, 264, 200), (40, 8, 8)]:
            for integer in (True, False):
                got, ref = run_general(dt, ta, tb, M, N, K, seed=M + 3 * N + 7 * K + ta + 2 * tb, integer=integer)
                check(dt, got, ref, integer, f"{dt} ta={ta} tb={tb} tile {tm}x{tn} {M}x{N}x{K} int={integer}")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("ta,tb", LAYOUTS)
def test_layouts_mid_size_auto_tile(dt, ta, tb):
    M, N, K = 776, 520, 1040
    got, ref = run_general(dt, ta, tb, M, N, K, seed=5, integer=False, lda_pad=0, ldb_pad=0, ldc_pad=0)
    check(dt, got, ref, False, f"{dt} ta={ta} tb={tb} {M}x{N}x{K}")


def test_packed_general_matches_the_fixed_entry_points():
    M, N, K = 300, 264, 200
    x = workloads.make_random("bf16_nt", M, N, K, seed=9)
    A = torch.from_numpy(x["A"].view(np.int16)).cuda().view(torch.bfloat16)
    B = torch.from_numpy(x["B"].view(np.int16)).cuda().view(torch.bfloat16)
    c1 = tg.gemm_bf16_nt(A, B)
    c2 = torch.empty_like(c1)
    assert tg.lib().gemm_bf16(0, 1, M, N, K, A.data_ptr(), K, B.data_ptr(), K, c2.data_ptr(), N, None) == 0
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_python_gemm_on_transposed_views(dt):
    M, N, K = 264, 200, 136
    g = workloads.generator(12)
    a = torch.randn(M, K, generator=g).to(TORCH_DT[dt]).cuda()
    b = torch.randn(K, N, generator=g).to(TORCH_DT[dt]).cuda()
    ref = tg.gemm(a, b)
    at = a.t().contiguous().t()        # same values, stored K x M
    bt = b.t().contiguous().t()        # same values, stored N x K
    for x, y in [(at, b), (a, bt), (at, bt)]:
        c = tg.gemm(x, y)
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int16), ref.view(torch.int16))
    opA = workloads.to_bits(a.cpu())
    opB = workloads.to_bits(b.cpu())
    check(dt, workloads.to_bits(ref.cpu()), reference(dt, opA, opB), False, "python gemm")


def test_general_validation_on_device():
    a = torch.zeros(64, 64, dtype=torch.bfloat16, device="cuda")
    c = torch.zeros(64, 64, dtype=torch.bfloat16, device="cuda")
    L = tg.lib()
    assert L.gemm_bf16(2, 0, 64, 64, 64, a.data_ptr(), 64, a.data_ptr(), 64, c.data_ptr(), 64, None) == tg.EINVAL
    assert L.gemm_bf16(0, 0, 64, 64, 64, a.data_ptr(), 32, a.data_ptr(), 64, c.data_ptr(), 64, None) == tg.EINVAL
    assert "lda=32" in tg.last_error()
    assert L.gemm_bf16(0, 0, 64, 64, 64, a.data_ptr(), 68, a.data_ptr(), 64, c.data_ptr(), 64, None) == tg.EALIGN
    tg.set_tile(256, 192)
    assert L.gemm_bf16(0, 0, 64, 64, 64, a.data_ptr(), 64, a.data_ptr(), 64, c.data_ptr(), 64, None) == tg.EINVAL
    assert "no 256x192 tile" in tg.last_error()
