"""gemm_mxfp4_nt (block-scaled FP4, one e8m0 scale per 32 K) against the oracle."""
import numpy as np
import pytest
import torch

import dense_tiled_gemm_bf16_amd as tg
import oracle
import workloads
from _exact import bf16_values

pytestmark = pytest.mark.gpu
RTOL = ATOL = 1e-2


@pytest.fixture(autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    tg.init()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def run(x, M, N, K, sA=None, sB=None):
    print(f"[gpu] gemm_mxfp4_nt M={M} N={N} K={K}", flush=True)
    c = tg.gemm_mxfp4_nt(dev(x["qA"]), dev(x["qB"]), sA if sA is not None else dev(x["sA"]),
                         sB if sB is not None else dev(x["sB"]))
    torch.cuda.synchronize()
    return c.cpu().view(torch.int16).numpy().view(np.uint16)


def assert_close(got, ref, what):
    g, r = bf16_values(got), bf16_values(ref)
    ok = np.abs(g - r) <= ATOL + RTOL * np.abs(r)
    assert ok.all(), f"{what}: {int((~ok).sum())} outside tolerance, max err {np.nanmax(np.abs(g - r))}"


def assert_bitwise(got, ref, what):
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{what}: {len(bad)} differ, first {bad[0]}"


def oracle_full(x):
    return oracle.gemm_mxfp4_nt(x["qA"], x["qB"], x["sA"], x["sB"])


# K = 256, 768, 1280, 2560 take the kernel for dword-aligned scale rows (K a
# multiple of 256): one slice, and odd numbers of slices whose last pair of
# slices is half outside K; the others the kernel for any scale rows.
@pytest.mark.parametrize("K", [32, 96, 256, 288, 768, 800, 1280, 2560])
def test_tails(K):
    for M in [1, 31, 257, 300]:
        for N in [8, 56, 264]:
            x = workloads.make_random("mxfp4_nt", M, N, K, seed=M * 7 + N * 3 + K)
            assert_close(run(x, M, N, K), oracle_full(x), f"mxfp4 {M}x{N}x{K}")
            xi = workloads.make_integer("mxfp4_nt", M, N, K, seed=M + N + K)
            assert_bitwise(run(xi, M, N, K), oracle_full(xi), f"mxfp4 int {M}x{N}x{K}")


def test_per_row_and_per_block_scales_bitwise():
    """Integer elements, a different power-of-two scale per row and per
    32-K block: exact in fp32, so bitwise; a wrong lane, row, block or byte
    of the scale mapping shows up here."""
    M, N, K = 300, 264, 544
    x = workloads.make_integer("mxfp4_nt", M, N, K, seed=9)
    rng = np.random.default_rng(3)
    x["sA"] = rng.integers(124, 131, x["sA"].shape).astype(np.uint8)
    x["sB"] = rng.integers(124, 131, x["sB"].shape).astype(np.uint8)
    assert_bitwise(run(x, M, N, K), oracle_full(x), "mxfp4 scales")


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_unaligned_scale_pointers(offset):
    M, N, K = 260, 136, 352          # 11 scale blocks per row: rows start at every byte of a dword
    x = workloads.make_integer("mxfp4_nt", M, N, K, seed=20 + offset)
    rng = np.random.default_rng(offset)
    x["sA"] = rng.integers(125, 130, x["sA"].shape).astype(np.uint8)
    x["sB"] = rng.integers(125, 130, x["sB"].shape).astype(np.uint8)

    def at_offset(bits):
        buf = torch.zeros(bits.size + offset, dtype=torch.uint8, device="cuda")
        buf[offset:] = torch.from_numpy(np.ascontiguousarray(bits).reshape(-1)).cuda()
        return buf[offset:].view(bits.shape)

    assert_bitwise(run(x, M, N, K, at_offset(x["sA"]), at_offset(x["sB"])), oracle_full(x),
                   f"mxfp4 scales at offset {offset}")


@pytest.mark.parametrize("offset", [0, 1, 2])
def test_whole_slices_with_unaligned_scale_pointers(offset):
    """K a multiple of 256 (32 scale blocks per row, whole dwords), the scale
    arrays at offset 0 (the kernel for dword-aligned scale rows) or 1, 2
    bytes past a dword (the kernel for any scale rows, chosen by the host
    for the same K).  Bitwise on integer elements with varied scales."""
    M, N, K = 264, 200, 1024
    x = workloads.make_integer("mxfp4_nt", M, N, K, seed=70 + offset)
    rng = np.random.default_rng(70 + offset)
    x["sA"] = rng.integers(124, 131, x["sA"].shape).astype(np.uint8)
    x["sB"] = rng.integers(124, 131, x["sB"].shape).astype(np.uint8)

    def at_offset(bits):
        buf = torch.zeros(bits.size + 4, dtype=torch.uint8, device="cuda")
        buf[offset:offset + bits.size] = torch.from_numpy(np.ascontiguousarray(bits).reshape(-1)).cuda()
        return buf[offset:offset + bits.size].view(bits.shape)

    assert_bitwise(run(x, M, N, K, at_offset(x["sA"]), at_offset(x["sB"])), oracle_full(x),
                   f"mxfp4 K={K} scales at offset {offset}")


@pytest.mark.parametrize("offset", [0, 1, 3])
def test_unaligned_scales_long_K(offset):
    """75 scale blocks per row (K = 2400), rows starting at every byte of a
    dword: each row's scale bytes are streamed 16 at a time across several
    such pieces.  Bitwise on integer elements."""
    M, N, K = 264, 136, 2400
    x = workloads.make_integer("mxfp4_nt", M, N, K, seed=50 + offset)
    rng = np.random.default_rng(50 + offset)
    x["sA"] = rng.integers(125, 130, x["sA"].shape).astype(np.uint8)
    x["sB"] = rng.integers(125, 130, x["sB"].shape).astype(np.uint8)

    def at_offset(bits):
        buf = torch.zeros(bits.size + offset, dtype=torch.uint8, device="cuda")
        buf[offset:] = torch.from_numpy(np.ascontiguousarray(bits).reshape(-1)).cuda()
        return buf[offset:].view(bits.shape)

    assert_bitwise(run(x, M, N, K, at_offset(x["sA"]), at_offset(x["sB"])), oracle_full(x),
                   f"mxfp4 long K scales at offset {offset}")


@pytest.mark.parametrize("K", [96, 1312])
def test_next_rows_scales_do_not_leak(K):
    """A slice is 8 scale blocks; with K = 96 (3 blocks) or 1312 (41) the
    last slice's other blocks would be the next rows' bytes.  Odd rows of A
    and B get 0xff scales (NaN in the e8m0 format); the products of even
    rows and even columns use none of them and must equal the oracle."""
    M, N = 64, 64
    x = workloads.make_integer("mxfp4_nt", M, N, K, seed=K)
    x["sA"][1::2] = 0xFF
    x["sB"][1::2] = 0xFF
    got = run(x, M, N, K)
    ref = oracle_full(x)
    assert_bitwise(got[::2, ::2], ref[::2, ::2], f"mxfp4 K={K} even rows and columns")


def test_mid_size_full_parity():
    M, N, K = 776, 520, 1024
    x = workloads.make_random("mxfp4_nt", M, N, K, seed=11)
    assert_close(run(x, M, N, K), oracle_full(x), "mxfp4 mid")


def test_workload_sampled_and_integer_bitwise():
    w = workloads.WORKLOADS["mxfp4_nt_4096"]
    x = workloads.make_inputs(w)
    got = run(x, w.M, w.N, w.K)
    rows, cols = workloads.sample_positions(w.M, w.N, 512, seed=5)
    assert_close(got[rows, cols], oracle.gemm_mxfp4_nt_at(x["qA"], x["qB"], x["sA"], x["sB"], rows, cols),
                 "mxfp4 4096^3 sampled")
    xi = workloads.make_integer("mxfp4_nt", w.M, w.N, w.K, seed=1)
    got = run(xi, w.M, w.N, w.K)
    rows, cols = workloads.sample_positions(w.M, w.N, 2000, seed=6)
    assert_bitwise(got[rows, cols], oracle.gemm_mxfp4_nt_at(xi["qA"], xi["qB"], xi["sA"], xi["sB"], rows, cols),
                   "mxfp4 4096^3 integer")


def test_K_zero_writes_zeros():
    M, N = 70, 40
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    e = torch.zeros((M, 0), dtype=torch.uint8, device="cuda")
    f = torch.zeros((N, 0), dtype=torch.uint8, device="cuda")
    tg.gemm_mxfp4_nt(e, f, e, f, out=out)
    torch.cuda.synchronize()
    assert torch.all(out.view(torch.int16) == 0)
