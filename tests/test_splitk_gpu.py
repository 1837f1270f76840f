"""The K-split entry points (gemm_bf16_splitk, gemm_f16_splitk) against the
oracle.

Each output tile's K slices are divided into contiguous ranges computed by
different workgroups; their fp32 sums are added in range order by a second
kernel.  The result differs from the one-pass kernels only in fp32 summation
order: random inputs are checked within rtol = atol = 1e-2 (the pages' bound,
TileLang SM100 README, "Compilation and Usage"), integer-valued inputs (exact
fp32 sums) bit for bit.  Every operand layout, both split tile shapes, ragged
M, N and K, split counts that do not divide the slices evenly, more splits
than slices, and a workspace full of NaN on entry.
"""
import numpy as np
import pytest
import torch

import dense_tiled_gemm_bf16_amd as tg
import oracle
import workloads
from _exact import bf16_values, f16_values

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    tg.init()


@pytest.fixture
def forced_tile():
    def force(tm, tn):
        tg.set_tile(tm, tn)
    yield force
    tg.set_tile(0, 0)


TDT = {"bf16": torch.bfloat16, "f16": torch.float16}


def values(dt, bits):
    return bf16_values(bits) if dt == "bf16" else f16_values(bits)


def operands(dt, M, N, K, seed, integer):
    """op(A) (M x K) and op(B) (K x N) bit patterns."""
    if integer:
        x = workloads.make_integer("f16_nn" if dt == "f16" else "bf16_nt", M, N, K, seed=seed)
    else:
        x = workloads.make_random("f16_nn" if dt == "f16" else "bf16_nt", M, N, K, seed=seed)
    A = x["A"]
    B = x["B"] if dt == "f16" else np.ascontiguousarray(x["B"].T)   # K x N
    return A, B


def dev(bits, dt):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(TDT[dt]).cuda()


def as_stored(bits, dt, trans):
    """A device view of the op(X) bits stored as given (trans: stored as the
    transpose of a row-major array)."""
    return dev(np.ascontiguousarray(bits.T), dt).t() if trans else dev(bits, dt)


def reference(dt, A, B):
    return oracle.gemm_f16_nn(A, B) if dt == "f16" else oracle.gemm_bf16_nt(A, np.ascontiguousarray(B.T))


def to_bits(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def check(dt, got, ref, integer, what):
    if integer:
        diff = got != ref
        assert not diff.any(), f"{what}: {int(diff.sum())} of {diff.size} differ"
    else:
        g, r = values(dt, got), values(dt, ref)
        bad = ~(np.abs(g - r) <= 1e-2 + 1e-2 * np.abs(r))
        assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} outside rtol=atol=1e-2"


def run_split(dt, ta, tb, A, B, splits, ws_fill=float("nan")):
    M, K = A.shape
    N = B.shape[1]
    a = as_stored(A, dt, ta)      # ta: A stored K x M
    b = as_stored(B, dt, tb)      # tb: B stored N x K
    need = tg.lib().tgemm_splitk_workspace_bytes(M, N, splits)
    ws = torch.full((max(need, 16) // 4,), ws_fill, dtype=torch.float32, device="cuda")
    print(f"[gpu] splitk {dt} ta={ta} tb={tb} M={M} N={N} K={K} splits={splits}", flush=True)
    c = tg.gemm_splitk(a, b, splits=splits, workspace=ws)
    torch.cuda.synchronize()
    return to_bits(c)


LAYOUTS = [(0, 1), (0, 0), (1, 0), (1, 1)]   # NT, NN, TN, TT


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("ta,tb", LAYOUTS, ids=["NT", "NN", "TN", "TT"])
@pytest.mark.parametrize("tile", [(64, 64), (128, 128)])
def test_split_layouts_tiles_ragged(dt, ta, tb, tile, forced_tile):
    forced_tile(*tile)
    for M, N, K, splits in [(200, 264, 1000, 3), (136, 72, 4104, 5), (296, 136, 72, 4), (8, 8, 640, 16)]:
        for integer in (False, True):
            A, B = operands(dt, M, N, K, seed=M + 3 * N + K + splits + integer, integer=integer)
            got = run_split(dt, ta, tb, A, B, splits)
            check(dt, got, reference(dt, A, B), integer, f"{dt} ta={ta} tb={tb} {tile} {M}x{N}x{K} s={splits}")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_auto_split_deep_k(dt):
    """512 x 512 x 4096: 64 tiles of 64 x 64 leave most CUs idle, so the
    automatic choice splits; the result matches the oracle in full."""
    M, N, K = 512, 512, 4096
    for integer in (False, True):
        A, B = operands(dt, M, N, K, seed=17 + integer, integer=integer)
        got = run_split(dt, 0, 1, A, B, 0)
        check(dt, got, reference(dt, A, B), integer, f"{dt} auto split {M}x{N}x{K}")


def test_no_split_matches_gemm():
    """splits = 1 is the one-pass kernel: bit for bit gemm()'s result."""
    M, N, K = 300, 264, 520
    A, B = operands("bf16", M, N, K, seed=5, integer=False)
    got = run_split("bf16", 0, 1, A, B, 1)
    ref = to_bits(tg.gemm(dev(A, "bf16"), dev(np.ascontiguousarray(B.T), "bf16").t()))
    assert np.array_equal(got, ref)


def test_workspace_validation_on_device():
    M, N, K = 64, 64, 256
    a = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((N, K), dtype=torch.bfloat16, device="cuda")
    c = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros(2 * M * N, dtype=torch.float32, device="cuda")
    L = tg.lib()
    small = 2 * M * N * 4
    rc = L.gemm_bf16_splitk(0, 1, M, N, K, a.data_ptr(), K, b.data_ptr(), K, c.data_ptr(), N, 3, ws.data_ptr(),
                            small, None)
    assert rc == tg.EINVAL and "workspace bytes" in tg.last_error()
    rc = L.gemm_bf16_splitk(0, 1, M, N, K, a.data_ptr(), K, b.data_ptr(), K, c.data_ptr(), N, 2,
                            ws.data_ptr() + 4, small - 4, None)
    assert rc == tg.EALIGN
    rc = L.gemm_bf16_splitk(0, 1, M, N, K, a.data_ptr(), K, b.data_ptr(), K, c.data_ptr(), N, 2, c.data_ptr(),
                            small, None)
    assert rc == tg.EINVAL and "overlaps" in tg.last_error()
    rc = L.gemm_bf16_splitk(0, 1, M, N, K, a.data_ptr(), K, b.data_ptr(), K, c.data_ptr(), N, 17, ws.data_ptr(),
                            small, None)
    assert rc == tg.EINVAL
    tg.set_tile(256, 256)
    try:
        rc = L.gemm_bf16_splitk(0, 1, M, N, K, a.data_ptr(), K, b.data_ptr(), K, c.data_ptr(), N, 2,
                                ws.data_ptr(), small, None)
        assert rc == tg.EINVAL and "256x256" in tg.last_error()
    finally:
        tg.set_tile(0, 0)
    torch.cuda.synchronize()


def test_split_calls_replay_from_a_graph():
    """gemm_bf16_splitk and gemm_bf16_splitk_noalloc launch kernels only (no
    memset, no allocation), so a caller may capture them.  A captured pair
    of calls is replayed three times, with eager work and synchronisation
    between the replays; every replay must equal the eager results bit for
    bit, and after A is doubled in place the outputs must double exactly."""
    import ctypes
    M, N, K = 512, 512, 4096
    A, B = operands("bf16", M, N, K, seed=23, integer=False)
    a = dev(A, "bf16")
    b = as_stored(B, "bf16", 1)
    need = tg.lib().tgemm_splitk_workspace_bytes(M, N, 0)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    c1 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    c2 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def calls():
        tg.gemm_splitk(a, b, splits=0, out=c1, workspace=ws)
        s = torch.cuda.current_stream().cuda_stream
        rc = tg.lib().gemm_bf16_splitk_noalloc(0, 1, M, N, K, a.data_ptr(), K, b.data_ptr(), K, c2.data_ptr(), N, 0,
                                               ctypes.c_void_p(s))
        assert rc == tg.OK, tg.last_error()

    print(f"[gpu] splitk graph M={M} N={N} K={K}", flush=True)
    calls()
    torch.cuda.synchronize()
    eager1, eager2 = to_bits(c1), to_bits(c2)
    assert np.array_equal(eager1, eager2)
    check("bf16", eager1, reference("bf16", A, B), False, "eager split")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        c1.fill_(0)
        c2.fill_(0)
        if rep == 2:
            a.mul_(2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want1 = eager1 if rep < 2 else to_bits((torch.from_numpy(eager1.view(np.int16)).view(torch.bfloat16)
                                                 .float() * 2).to(torch.bfloat16))
        assert np.array_equal(to_bits(c1), want1), f"replay {rep}: gemm_bf16_splitk"
        assert np.array_equal(to_bits(c2), want1), f"replay {rep}: gemm_bf16_splitk_noalloc"
