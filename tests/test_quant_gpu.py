"""GPU block-scale quantiser (quantize_mxfp8) against the oracle's, bit for bit.

Both sides implement the same deterministic rule, so scales and elements
must match exactly: random rows over a wide range of magnitudes, ragged K,
scale boundaries, halfway values, binary32 subnormals, the full 4096 x 4096
workload, and the quantiser feeding the block-scaled GEMM.
"""
import numpy as np
import pytest
import torch

import dense_tiled_gemm_bf16_amd as tg
import oracle
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    tg.init()


def gpu_quantize(x: np.ndarray):
    print(f"[gpu] quantize_mxfp8 {x.shape}", flush=True)
    q, s = tg.quantize_mxfp8(torch.from_numpy(np.ascontiguousarray(x)).cuda())
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


def assert_same(x: np.ndarray, what: str):
    q, s = gpu_quantize(x)
    qr, sr = oracle.quantize_mxfp8(x)
    bad_s = np.argwhere(s != sr)
    assert bad_s.size == 0, f"{what}: {len(bad_s)} scales differ, first {bad_s[0]}: {s[tuple(bad_s[0])]} vs {sr[tuple(bad_s[0])]}"
    bad_q = np.argwhere(q != qr)
    assert bad_q.size == 0, (f"{what}: {len(bad_q)} elements differ, first {bad_q[0]}: x={x[tuple(bad_q[0])]!r} "
                             f"gpu {q[tuple(bad_q[0])]:#04x} oracle {qr[tuple(bad_q[0])]:#04x}")


def test_random_rows_over_wide_magnitudes():
    g = workloads.generator(21)
    x = workloads.randn_f32((96, 1024), g) * torch.logspace(-35, 35, 96)[:, None]
    assert_same(x.numpy(), "wide magnitudes")


@pytest.mark.parametrize("K", [16, 112, 128, 144, 400, 512, 528, 1040])
@pytest.mark.parametrize("M", [1, 3, 65])
def test_ragged_shapes(M, K):
    g = workloads.generator(M * 1000 + K)
    x = workloads.randn_f32((M, K), g) * 3.0
    assert_same(x.numpy(), f"{M}x{K}")


def test_scale_boundaries_and_zero_blocks():
    x = np.zeros((8, 512), np.float32)
    for r, k in enumerate([-30, -1, 0, 7, 60, 100]):
        top = np.float32(448.0 * 2.0 ** k)
        x[r, 3] = top                                               # block 0: exactly 448 * 2^k
        x[r, 130] = np.nextafter(top, np.float32(np.inf))            # block 1: one ulp above
        x[r, 260] = -top / 3                                        # block 2: inside
    x[7, 300] = 1.0                                                 # row 7: one non-zero block
    assert_same(x, "boundaries")


def test_halfway_values_round_to_even():
    """Scaled values exactly halfway between e4m3fn neighbours, in the normal
    and subnormal ranges (scale fixed at 2^0 by a 448 in each block)."""
    grid = np.array(sorted(set(torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
                                .double().abs().tolist())), np.float64)
    grid = grid[np.isfinite(grid)]
    mids = (grid[:-1] + grid[1:]) / 2
    mids = np.concatenate([mids, -mids]).astype(np.float32)
    K = 128
    rows = (len(mids) + K - 2) // (K - 1)
    x = np.zeros((rows, K), np.float32)
    x[:, 0] = 448.0
    flat = x[:, 1:].reshape(-1)
    flat[:len(mids)] = mids
    x[:, 1:] = flat.reshape(rows, K - 1)
    assert np.all(mids.astype(np.float64) == np.concatenate([(grid[:-1] + grid[1:]) / 2, -(grid[:-1] + grid[1:]) / 2]))
    assert_same(x, "halfway")


def test_binary32_subnormal_inputs():
    """Blocks whose maximum is a binary32 subnormal: e clamps to -127 and
    x * 2^127 lands in the e4m3fn range, so flushing the inputs would show."""
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((4, 256)) * 2.0 ** -133).astype(np.float32)
    assert np.all(np.abs(x[x != 0]) < np.float32(2.0 ** -126))
    assert_same(x, "subnormal inputs")


def test_full_workload_size():
    w = workloads.WORKLOADS["mxfp8_nt_4096"]
    g = workloads.generator(0)
    x = workloads.randn_f32((w.M, w.K), g)
    assert_same(x.numpy(), "4096 x 4096")


def test_quantiser_feeds_the_block_scaled_gemm():
    """GPU quantiser -> GPU GEMM equals the oracle GEMM of the oracle's
    quantisation (within the GEMM tolerance; the inputs are bit-identical)."""
    M, N, K = 384, 264, 640
    g = workloads.generator(31)
    a = workloads.randn_f32((M, K), g)
    b = workloads.randn_f32((N, K), g)
    qa, sa = tg.quantize_mxfp8(a.cuda())
    qb, sb = tg.quantize_mxfp8(b.cuda())
    c = tg.gemm_mxfp8_nt(qa, qb, sa, sb)
    torch.cuda.synchronize()
    qa_r, sa_r = oracle.quantize_mxfp8(a.numpy())
    qb_r, sb_r = oracle.quantize_mxfp8(b.numpy())
    assert np.array_equal(qa.cpu().numpy(), qa_r) and np.array_equal(sb.cpu().numpy(), sb_r)
    ref = oracle.gemm_mxfp8_nt(qa_r, qb_r, sa_r, sb_r)
    got = c.cpu().view(torch.int16).numpy().view(np.uint16)
    g64 = torch.from_numpy(got.view(np.int16)).view(torch.bfloat16).double().numpy()
    r64 = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.all(np.abs(g64 - r64) <= 1e-2 + 1e-2 * np.abs(r64))
