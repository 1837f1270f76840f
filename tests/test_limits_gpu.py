"""The largest operands the library accepts, against the oracle at sampled
outputs.

Buffer offsets are 31-bit, and the host rejects anything whose addressed
span would pass 2^31 bytes.  These tests sit right below each limit, so every
offset the kernels form comes within a few rows of 2^31:

* bf16 NT, MXFP8 NT, MXFP4 NT and MXFP6 NT with the largest K whose
  256-row panel fits (the K-contiguous panels are addressed per 256 rows),
  with a ragged last slice read at the very end of the range (and, for the
  kinds with a kernel for whole slices, K a multiple of the slice too);
* gemm_bf16 with A stored K x M (M-contiguous, addressed as a whole) and
  the largest K whose rows, rounded up to whole slices of 64, fit.

Elements are integers in [-1, 1], drawn on the device from a seeded
generator; every partial sum is then an integer below 2^24, exact in fp32 in
any order, so the sampled outputs must match the oracle bit for bit.  Only
the rows of A and B that the sampled outputs use are copied to the host.
"""
import numpy as np
import pytest
import torch

import dense_tiled_gemm_bf16_amd as tg
import oracle
import workloads

pytestmark = pytest.mark.gpu

LIMIT = 2**31 - 1


@pytest.fixture(autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    tg.init()
    yield
    tg.set_tile(0, 0)
    torch.cuda.empty_cache()


def ints(shape, seed):
    """Seeded integers in [-1, 1] (int8) on the device."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randint(-1, 2, shape, generator=g, device="cuda", dtype=torch.int8)


def e4m3_ints(shape, seed):
    """Seeded e4m3fn bytes of -1, 0 and 1 (0xB8, 0x00, 0x38) on the device."""
    x = ints(shape, seed)
    q = x.abs().to(torch.uint8) * 0x38
    q |= (x < 0).to(torch.uint8) << 7
    return q


def bits16(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def sampled(M, N, count, seed):
    rows, cols = workloads.sample_positions(M, N, count, seed=seed)
    ur, rinv = np.unique(rows, return_inverse=True)
    uc, cinv = np.unique(cols, return_inverse=True)
    return rows, cols, ur, rinv, uc, cinv


@pytest.mark.parametrize("tile", [(0, 0), (256, 256)])
def test_bf16_nt_largest_panel(tile):
    K = (LIMIT // (256 * 2)) // 8 * 8          # 256 * K * 2 < 2^31, K % 8 == 0
    assert 256 * K * 2 <= LIMIT < 256 * (K + 8) * 2 and K % 64 != 0
    M, N = 300, 24                             # a full and a partial row panel
    A = ints((M, K), 1).to(torch.bfloat16)
    B = ints((N, K), 2).to(torch.bfloat16)
    tg.set_tile(*tile)
    print(f"[gpu] gemm_bf16_nt M={M} N={N} K={K} tile={tile}", flush=True)
    C = tg.gemm_bf16_nt(A, B)
    torch.cuda.synchronize()
    rows, cols, ur, rinv, uc, cinv = sampled(M, N, 40, seed=3)
    ref = oracle.gemm_bf16_nt_at(bits16(A[torch.from_numpy(ur).cuda()]), bits16(B[torch.from_numpy(uc).cuda()]),
                                 rinv, cinv)
    got = bits16(C)[rows, cols]
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"{bad.size} of {got.size} differ, first at {(rows[bad[0]], cols[bad[0]])}"


@pytest.mark.parametrize("whole", [False, True])
def test_mxfp8_nt_largest_panel(whole):
    # 256 * K < 2^31 with K % 16 == 0 (a ragged last slice), or K % 128 == 0
    step = 128 if whole else 16
    K = (LIMIT // 256) // step * step
    assert 256 * K <= LIMIT < 256 * (K + step) and (K % 128 == 0) == whole
    M, N = 300, 24
    KB = (K + 127) // 128
    qA = e4m3_ints((M, K), 4)
    qB = e4m3_ints((N, K), 5)
    sA = torch.full((M, KB), 127, dtype=torch.uint8, device="cuda")            # 2^0
    sB = torch.full((N, KB), 127, dtype=torch.uint8, device="cuda")
    print(f"[gpu] gemm_mxfp8_nt M={M} N={N} K={K}", flush=True)
    C = tg.gemm_mxfp8_nt(qA, qB, sA, sB)
    torch.cuda.synchronize()
    rows, cols, ur, rinv, uc, cinv = sampled(M, N, 40, seed=4)
    r, c = torch.from_numpy(ur).cuda(), torch.from_numpy(uc).cuda()
    ref = oracle.gemm_mxfp8_nt_at(qA[r].cpu().numpy(), qB[c].cpu().numpy(), sA[r].cpu().numpy(),
                                  sB[c].cpu().numpy(), rinv, cinv)
    got = bits16(C)[rows, cols]
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"{bad.size} of {got.size} differ, first at {(rows[bad[0]], cols[bad[0]])}"


@pytest.mark.parametrize("tile", [(0, 0), (256, 256), (128, 128)])
def test_m_contiguous_a_largest_k(tile):
    M, N = 1024, 16
    lda = M
    K = LIMIT // (lda * 2) // 64 * 64 - 56     # rounded up to 64 rows it just fits; ragged
    assert (K + 63) // 64 * 64 * lda * 2 <= LIMIT < ((K + 63) // 64 + 1) * 64 * lda * 2 and K % 64 != 0
    A = ints((K, M), 6).to(torch.bfloat16)      # stored K x M
    B = ints((N, K), 7).to(torch.bfloat16)      # stored N x K
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    tg.set_tile(*tile)
    print(f"[gpu] gemm_bf16 ta=1 tb=1 M={M} N={N} K={K} lda={lda} tile={tile}", flush=True)
    rc = tg.lib().gemm_bf16(1, 1, M, N, K, A.data_ptr(), lda, B.data_ptr(), K, C.data_ptr(), N, None)
    assert rc == 0, tg.last_error()
    torch.cuda.synchronize()
    rows, cols, ur, rinv, uc, cinv = sampled(M, N, 40, seed=5)
    opA = A[:, torch.from_numpy(ur).cuda()].t().contiguous()                  # rows of op(A)
    ref = oracle.gemm_bf16_nt_at(bits16(opA), bits16(B[torch.from_numpy(uc).cuda()]), rinv, cinv)
    got = bits16(C)[rows, cols]
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"{bad.size} of {got.size} differ, first at {(rows[bad[0]], cols[bad[0]])}"


def fp4_ints(shape, seed):
    """Seeded E2M1 codes of -1, 0 and 1 (10, 0, 2), two per byte (element 2 i
    in the low nibble), on the device: (R, K) -> (R, K / 2)."""
    x = ints(shape, seed)
    c = x.abs().to(torch.uint8) * 2
    c |= (x < 0).to(torch.uint8) << 3
    c = c.view(shape[0], shape[1] // 2, 2)
    return c[:, :, 0] | (c[:, :, 1] << 4)


def fp6_ints(shape, seed):
    """Seeded E2M3 codes of -1, 0 and 1 (40, 0, 8), four in three bytes
    (element k at bits 6 k .. 6 k + 5), on the device: (R, K) -> (R, 3K / 4)."""
    x = ints(shape, seed)
    c = x.abs().to(torch.int32) * 8
    c |= (x < 0).to(torch.int32) << 5
    del x
    c = c.view(shape[0], shape[1] // 4, 4)
    v = c[:, :, 0] | (c[:, :, 1] << 6) | (c[:, :, 2] << 12) | (c[:, :, 3] << 18)
    del c
    out = torch.stack([v & 255, (v >> 8) & 255, v >> 16], dim=2).to(torch.uint8)
    return out.view(shape[0], shape[1] // 4 * 3)


@pytest.mark.parametrize("whole", [False, True])
def test_mxfp4_nt_largest_panel(whole):
    # 256 * K / 2 < 2^31 with K % 32 == 0 (ragged last slice), or K % 256 == 0
    step = 256 if whole else 32
    K = (LIMIT // 128) // step * step
    assert 256 * (K // 2) <= LIMIT < 256 * ((K + step) // 2) and (K % 256 == 0) == whole
    M, N = 300, 24
    KB = K // 32
    qA, qB = fp4_ints((M, K), 8), fp4_ints((N, K), 9)
    sA = torch.full((M, KB), 127, dtype=torch.uint8, device="cuda")
    sB = torch.full((N, KB), 127, dtype=torch.uint8, device="cuda")
    print(f"[gpu] gemm_mxfp4_nt M={M} N={N} K={K}", flush=True)
    C = tg.gemm_mxfp4_nt(qA, qB, sA, sB)
    torch.cuda.synchronize()
    rows, cols, ur, rinv, uc, cinv = sampled(M, N, 40, seed=6)
    r, c = torch.from_numpy(ur).cuda(), torch.from_numpy(uc).cuda()
    ref = oracle.gemm_mxfp4_nt_at(qA[r].cpu().numpy(), qB[c].cpu().numpy(), sA[r].cpu().numpy(),
                                  sB[c].cpu().numpy(), rinv, cinv, K=K)
    got = bits16(C)[rows, cols]
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"{bad.size} of {got.size} differ, first at {(rows[bad[0]], cols[bad[0]])}"


def test_mxfp6_nt_largest_panel():
    # 256 * 3K/4 < 2^31 with K % 64 == 0, and a ragged last 128-element slice
    K = (LIMIT // 256) * 4 // 3 // 64 * 64 - 64
    assert 256 * (K // 4 * 3) <= LIMIT and K % 128 == 64
    M, N = 300, 24
    KB = K // 32
    qA, qB = fp6_ints((M, K), 10), fp6_ints((N, K), 11)
    sA = torch.full((M, KB), 127, dtype=torch.uint8, device="cuda")
    sB = torch.full((N, KB), 127, dtype=torch.uint8, device="cuda")
    print(f"[gpu] gemm_mxfp6_nt e2m3 M={M} N={N} K={K}", flush=True)
    C = tg.gemm_mxfp6_nt(qA, qB, sA, sB, fmt="e2m3")
    torch.cuda.synchronize()
    rows, cols, ur, rinv, uc, cinv = sampled(M, N, 40, seed=7)
    r, c = torch.from_numpy(ur).cuda(), torch.from_numpy(uc).cuda()
    ref = oracle.gemm_mxfp6_nt_at(qA[r].cpu().numpy(), qB[c].cpu().numpy(), sA[r].cpu().numpy(),
                                  sB[c].cpu().numpy(), rinv, cinv, "e2m3", K=K)
    got = bits16(C)[rows, cols]
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"{bad.size} of {got.size} differ, first at {(rows[bad[0]], cols[bad[0]])}"
