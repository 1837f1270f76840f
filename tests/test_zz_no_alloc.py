"""gemm_bf16_splitk_noalloc, the K split for callers that cannot allocate,
against gemm_bf16_splitk (the same computation with a caller's workspace).

Both run the same kernels on the same inputs, so their outputs must agree
bit for bit; each is also checked against the oracle (random inputs within
rtol = atol = 1e-2, the pages' bound, TileLang SM100 README, "Compilation and
Usage"; integer-valued inputs bit for bit).  Two calls in a row share the
scratch array, the second with a smaller problem, so stale partial sums of
the first call would show up in the second.
"""
import ctypes

import numpy as np
import pytest
import torch

import dense_tiled_gemm_bf16_amd as tg
import oracle
import workloads
from _exact import bf16_values

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    tg.init()


def bits_of(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def call_noalloc(A, B, C, M, N, K, splits):
    stream = torch.cuda.current_stream().cuda_stream
    print(f"[gpu] gemm_bf16_splitk_noalloc M={M} N={N} K={K} splits={splits}", flush=True)
    rc = tg.lib().gemm_bf16_splitk_noalloc(0, 1, M, N, K, A.data_ptr(), K, B.data_ptr(), K, C.data_ptr(), N,
                                           splits, ctypes.c_void_p(stream))
    assert rc == tg.OK, tg.last_error()


def call_workspace(A, B, C, M, N, K, splits):
    need = tg.lib().tgemm_splitk_workspace_bytes(M, N, splits)
    ws = torch.full((max(need, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    rc = tg.lib().gemm_bf16_splitk(0, 1, M, N, K, A.data_ptr(), K, B.data_ptr(), K, C.data_ptr(), N, splits,
                                   ws.data_ptr(), ws.numel() * 4, ctypes.c_void_p(stream))
    assert rc == tg.OK, tg.last_error()


@pytest.mark.parametrize("integer", [False, True])
def test_noalloc_matches_the_workspace_entry_point(integer):
    # The first call fills more of the scratch than the second reads.
    cases = [(512, 512, 4096, 4), (200, 136, 1000, 3), (512, 512, 4096, 0), (136, 72, 520, 2)]
    for M, N, K, splits in cases:
        make = workloads.make_integer if integer else workloads.make_random
        x = make("bf16_nt", M, N, K, seed=M + N + K + splits)
        A, B = dev(x["A"]), dev(x["B"])
        c_noalloc = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        c_ws = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        call_noalloc(A, B, c_noalloc, M, N, K, splits)
        call_workspace(A, B, c_ws, M, N, K, splits)
        torch.cuda.synchronize()
        got, want = bits_of(c_noalloc), bits_of(c_ws)
        assert np.array_equal(got, want), f"{M}x{N}x{K} splits={splits}: {int((got != want).sum())} differ"
        ref = oracle.gemm_bf16_nt(x["A"], x["B"])
        if integer:
            assert np.array_equal(got, ref), f"{M}x{N}x{K}: {int((got != ref).sum())} differ from the oracle"
        else:
            g, r = bf16_values(got), bf16_values(ref)
            bad = ~(np.abs(g - r) <= 1e-2 + 1e-2 * np.abs(r))
            assert not bad.any(), f"{M}x{N}x{K}: {int(bad.sum())} outside rtol=atol=1e-2"


def test_noalloc_rejects_what_the_scratch_cannot_hold():
    M, N, K = 1024, 1024, 256
    A = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
    C = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    rc = tg.lib().gemm_bf16_splitk_noalloc(0, 1, M, N, K, A.data_ptr(), K, B.data_ptr(), K, C.data_ptr(), N, 3,
                                           None)
    assert rc == tg.ETOOBIG and "scratch" in tg.last_error()
    torch.cuda.synchronize()
