"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Tolerance: |gpu - oracle| <= 1e-2 + 1e-2 |oracle| elementwise on the output
values, NaN failing -- the check the pages themselves apply (TileLang SM100
README, "Compilation and Usage"), here against the binary64 oracle rounded
once to the output type.  On integer-valued inputs every fp32 partial sum
is exact, so there the GPU and the oracle must agree bit for bit.

Every workload is compared in full, at its real size, on random and on
integer-valued inputs; only the maximum-size cases elsewhere are sampled.
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


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    tg.init()


# --- helpers ---------------------------------------------------------------------

def to_dev(bits: np.ndarray, kind: str) -> torch.Tensor:
    if bits.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
        t = t.view(torch.bfloat16 if kind == "bf16" else torch.float16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(bits))
    return t.cuda()


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def run(kind: str, x: dict, M: int, N: int, K: int, out=None, stream=None) -> torch.Tensor:
    print(f"[gpu] {kind} M={M} N={N} K={K}", flush=True)
    if kind == "bf16_nt":
        c = tg.gemm_bf16_nt(to_dev(x["A"], "bf16"), to_dev(x["B"], "bf16"), out=out, stream=stream)
    elif kind == "f16_nn":
        c = tg.gemm_f16_nn(to_dev(x["A"], "f16"), to_dev(x["B"], "f16"), out=out, stream=stream)
    else:
        c = tg.gemm_mxfp8_nt(to_dev(x["qA"], ""), to_dev(x["qB"], ""), to_dev(x["sA"], ""),
                             to_dev(x["sB"], ""), out=out, stream=stream)
    torch.cuda.synchronize()
    return c


def oracle_full(kind, x):
    if kind == "bf16_nt":
        return oracle.gemm_bf16_nt(x["A"], x["B"])
    if kind == "f16_nn":
        return oracle.gemm_f16_nn(x["A"], x["B"])
    return oracle.gemm_mxfp8_nt(x["qA"], x["qB"], x["sA"], x["sB"])


def oracle_at(kind, x, rows, cols):
    if kind == "bf16_nt":
        return oracle.gemm_bf16_nt_at(x["A"], x["B"], rows, cols)
    if kind == "f16_nn":
        return oracle.gemm_f16_nn_at(x["A"], x["B"], rows, cols)
    return oracle.gemm_mxfp8_nt_at(x["qA"], x["qB"], x["sA"], x["sB"], rows, cols)


def values(kind, bits):
    return f16_values(bits) if kind == "f16_nn" else bf16_values(bits)


def assert_close(kind, got_bits, ref_bits, what=""):
    g, r = values(kind, got_bits), values(kind, ref_bits)
    bad = ~(np.abs(g - r) <= ATOL + RTOL * np.abs(r))
    if bad.any():
        idx = np.argwhere(bad)[:8]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside rtol=atol=1e-2; first at "
            f"{[tuple(int(v) for v in i) for i in idx]}: got {g[bad][:8]} want {r[bad][:8]}")


def assert_bitwise(got_bits, ref_bits, what=""):
    diff = got_bits != ref_bits
    if diff.any():
        idx = np.argwhere(diff)[:8]
        raise AssertionError(f"{what}: {int(diff.sum())} of {diff.size} differ; first at "
                             f"{[tuple(int(v) for v in i) for i in idx]}: got {got_bits[diff][:8]} "
                             f"want {ref_bits[diff][:8]}")


# --- the five workloads -----------------------------------------------------------

SMALL = ["bf16_nt_256", "f16_nn_1024"]
LARGE = ["bf16_nt_4096x4096x8192", "bf16_nt_4000x3000x5000", "mxfp8_nt_4096"]


@pytest.mark.parametrize("name", SMALL)
def test_small_workload_full_parity(name):
    w = workloads.WORKLOADS[name]
    x = workloads.make_inputs(w)
    got = to_bits(run(w.kind, x, w.M, w.N, w.K))
    assert_close(w.kind, got, oracle_full(w.kind, x), name)


@pytest.mark.parametrize("name", SMALL)
def test_small_workload_integer_inputs_bitwise(name):
    """Integer-valued inputs: every fp32 partial sum is exact, so every output
    must match the oracle bit for bit."""
    w = workloads.WORKLOADS[name]
    x = workloads.make_integer(w.kind, w.M, w.N, w.K, seed=5)
    assert_bitwise(to_bits(run(w.kind, x, w.M, w.N, w.K)), oracle_full(w.kind, x), name)


# The full-size workloads are compared output by output, in full.  The oracle
# takes tens of seconds per workload on the host's cores, so each comparison
# is split into bands of rows (a test each, sharing one GPU result).
LARGE_BANDS = {"bf16_nt_4096x4096x8192": 2, "bf16_nt_4000x3000x5000": 1, "mxfp8_nt_4096": 4}
LARGE_CASES = [(name, variant, band, LARGE_BANDS[name]) for name in LARGE for variant in ("random", "integer")
               for band in range(LARGE_BANDS[name])]


@pytest.fixture(scope="module")
def large_result():
    """(inputs, GPU output bits) of a full-size workload, random or integer
    inputs; the last one is kept for the next band."""
    cache = {}

    def get(name, variant):
        if (name, variant) not in cache:
            cache.clear()
            w = workloads.WORKLOADS[name]
            x = workloads.make_inputs(w) if variant == "random" else workloads.make_integer(w.kind, w.M, w.N, w.K,
                                                                                          seed=5)
            cache[(name, variant)] = (x, to_bits(run(w.kind, x, w.M, w.N, w.K)))
        return cache[(name, variant)]
    return get


def oracle_rows(kind, x, r0, r1):
    """Rows r0 .. r1 - 1 of the oracle's C: the same function on that band of
    A's rows (and their scales) with all of B."""
    if kind == "bf16_nt":
        return oracle.gemm_bf16_nt(x["A"][r0:r1], x["B"])
    if kind == "f16_nn":
        return oracle.gemm_f16_nn(x["A"][r0:r1], x["B"])
    return oracle.gemm_mxfp8_nt(x["qA"][r0:r1], x["qB"], x["sA"][r0:r1], x["sB"])


@pytest.mark.parametrize("name,variant,band,bands", LARGE_CASES,
                         ids=[f"{n}-{v}-{b}of{nb}" for n, v, b, nb in LARGE_CASES])
def test_large_workload_full_parity(large_result, name, variant, band, bands):
    """Every output of the full-size workloads against the oracle: random
    inputs within the tolerance, integer-valued inputs (exact fp32 sums) bit
    for bit."""
    w = workloads.WORKLOADS[name]
    x, got = large_result(name, variant)
    r0, r1 = band * w.M // bands, (band + 1) * w.M // bands
    ref = oracle_rows(w.kind, x, r0, r1)
    what = f"{name} {variant} rows {r0}..{r1 - 1}"
    if variant == "random":
        assert_close(w.kind, got[r0:r1], ref, what)
        assert np.isfinite(values(w.kind, got[r0:r1])).all()
    else:
        assert_bitwise(got[r0:r1], ref, what)


# --- tails, several tiles, degenerate shapes ------------------------------------------

TAIL_M = [1, 31, 255, 257, 300]
TAIL_N = [8, 56, 264]


@pytest.mark.parametrize("K", [8, 64, 72, 136, 520])
def test_bf16_nt_tails(K):
    for M in TAIL_M:
        for N in TAIL_N:
            x = workloads.make_random("bf16_nt", M, N, K, seed=M * 7 + N * 3 + K)
            assert_close("bf16_nt", to_bits(run("bf16_nt", x, M, N, K)), oracle_full("bf16_nt", x),
                         f"bf16_nt {M}x{N}x{K}")
            xi = workloads.make_integer("bf16_nt", M, N, K, seed=M + N + K)
            assert_bitwise(to_bits(run("bf16_nt", xi, M, N, K)), oracle_full("bf16_nt", xi),
                           f"bf16_nt int {M}x{N}x{K}")


@pytest.mark.parametrize("K", [8, 64, 72, 200])
def test_f16_nn_tails(K):
    for M in TAIL_M:
        for N in TAIL_N:
            x = workloads.make_random("f16_nn", M, N, K, seed=M * 7 + N * 3 + K)
            assert_close("f16_nn", to_bits(run("f16_nn", x, M, N, K)), oracle_full("f16_nn", x),
                         f"f16_nn {M}x{N}x{K}")
            xi = workloads.make_integer("f16_nn", M, N, K, seed=M + N + K)
            assert_bitwise(to_bits(run("f16_nn", xi, M, N, K)), oracle_full("f16_nn", xi),
                           f"f16_nn int {M}x{N}x{K}")


@pytest.mark.parametrize("K", [16, 112, 128, 144, 400])
def test_mxfp8_tails(K):
    for M in TAIL_M:
        for N in TAIL_N:
            x = workloads.make_random("mxfp8_nt", M, N, K, seed=M * 7 + N * 3 + K)
            assert_close("mxfp8_nt", to_bits(run("mxfp8_nt", x, M, N, K)), oracle_full("mxfp8_nt", x),
                         f"mxfp8 {M}x{N}x{K}")
            xi = workloads.make_integer("mxfp8_nt", M, N, K, seed=M + N + K)
            assert_bitwise(to_bits(run("mxfp8_nt", xi, M, N, K)), oracle_full("mxfp8_nt", xi),
                           f"mxfp8 int {M}x{N}x{K}")


def test_mxfp8_per_row_and_per_block_scales_bitwise():
    """Integer elements with a different power-of-two scale per row and per
    128-K block: exact in fp32, so bitwise; a wrong scale lane, row or block
    mapping shows up here."""
    M, N, K = 300, 264, 512
    x = workloads.make_integer("mxfp8_nt", M, N, K, seed=9)
    rng = np.random.default_rng(3)
    x["sA"] = rng.integers(124, 131, x["sA"].shape).astype(np.uint8)
    x["sB"] = rng.integers(124, 131, x["sB"].shape).astype(np.uint8)
    assert_bitwise(to_bits(run("mxfp8_nt", x, M, N, K)), oracle_full("mxfp8_nt", x), "mxfp8 scales")


@pytest.mark.parametrize("slices", [1, 2, 3, 5, 6, 7, 9, 33])
def test_mxfp8_slice_counts_bitwise(slices):
    """K a whole number of 128-element slices (the kernel that checks no
    columns), every count of slices left after the K loop's rounds of four
    (each slice's fragments are read during the one before, each group of
    four slices' scales during the group before), several tiles with a
    ragged N, a different power-of-two scale per row and block: integer
    elements and scales within 2^-2 .. 2^2 keep every fp32 sum exact, so the
    result is compared bit for bit."""
    M, N, K = 264, 520, 128 * slices
    x = workloads.make_integer("mxfp8_nt", M, N, K, seed=70 + slices)
    rng = np.random.default_rng(slices)
    x["sA"] = rng.integers(125, 130, x["sA"].shape).astype(np.uint8)
    x["sB"] = rng.integers(125, 130, x["sB"].shape).astype(np.uint8)
    print(f"[gpu] mxfp8_nt slices={slices} M={M} N={N} K={K}", flush=True)
    assert_bitwise(to_bits(run("mxfp8_nt", x, M, N, K)), oracle_full("mxfp8_nt", x), f"mxfp8 {slices} slices")


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_mxfp8_unaligned_scale_pointers(offset):
    """The scale arrays need no alignment: views starting 1-3 bytes into a
    buffer, with an odd number of scale blocks per row (K = 272, 3 blocks)
    so that rows start at every byte position of a dword.  Integer elements
    and per-row, per-block scales: bitwise."""
    M, N, K = 300, 264, 272
    x = workloads.make_integer("mxfp8_nt", M, N, K, seed=11 + offset)
    rng = np.random.default_rng(offset)
    x["sA"] = rng.integers(124, 131, x["sA"].shape).astype(np.uint8)
    x["sB"] = rng.integers(124, 131, x["sB"].shape).astype(np.uint8)

    def at_offset(bits):
        buf = torch.zeros(bits.size + offset, dtype=torch.uint8, device="cuda")
        buf[offset:] = torch.from_numpy(np.ascontiguousarray(bits).reshape(-1)).cuda()
        view = buf[offset:].view(bits.shape)
        assert view.data_ptr() % 4 == offset % 4
        return view

    print(f"[gpu] mxfp8_nt unaligned scales offset={offset} M={M} N={N} K={K}", flush=True)
    c = tg.gemm_mxfp8_nt(to_dev(x["qA"], ""), to_dev(x["qB"], ""), at_offset(x["sA"]), at_offset(x["sB"]))
    torch.cuda.synchronize()
    assert_bitwise(to_bits(c), oracle_full("mxfp8_nt", x), f"mxfp8 scales at offset {offset}")


@pytest.mark.parametrize("offset", [0, 1, 3])
def test_mxfp8_unaligned_scales_long_K(offset):
    """37 scale blocks per row (K = 4736): the kernel streams each row's
    scale bytes in 16-byte pieces, so a row whose bytes start at any byte of
    a dword is read across several of them.  Bitwise on integer elements."""
    M, N, K = 264, 136, 4736
    x = workloads.make_integer("mxfp8_nt", M, N, K, seed=40 + offset)
    rng = np.random.default_rng(40 + offset)
    x["sA"] = rng.integers(124, 131, x["sA"].shape).astype(np.uint8)
    x["sB"] = rng.integers(124, 131, x["sB"].shape).astype(np.uint8)

    def at_offset(bits):
        buf = torch.zeros(bits.size + offset, dtype=torch.uint8, device="cuda")
        buf[offset:] = torch.from_numpy(np.ascontiguousarray(bits).reshape(-1)).cuda()
        return buf[offset:].view(bits.shape)

    print(f"[gpu] mxfp8_nt long-K unaligned scales offset={offset} M={M} N={N} K={K}", flush=True)
    c = tg.gemm_mxfp8_nt(to_dev(x["qA"], ""), to_dev(x["qB"], ""), at_offset(x["sA"]), at_offset(x["sB"]))
    torch.cuda.synchronize()
    assert_bitwise(to_bits(c), oracle_full("mxfp8_nt", x), f"mxfp8 long K scales at offset {offset}")


def test_mxfp8_next_rows_scales_do_not_leak():
    """K = 768: 6 slices of 128; a scale dword covers 4 slices, so the
    second one's last two bytes would be the next row's.  Odd rows of A and B get 0xff
    scales (NaN in the e8m0 format); the products of even rows and even
    columns use none of them and must equal the oracle bit for bit."""
    M, N, K = 64, 64, 768
    x = workloads.make_integer("mxfp8_nt", M, N, K, seed=31)
    x["sA"][1::2] = 0xFF
    x["sB"][1::2] = 0xFF
    got = to_bits(run("mxfp8_nt", x, M, N, K))
    ref = oracle_full("mxfp8_nt", x)
    assert_bitwise(got[::2, ::2], ref[::2, ::2], "mxfp8 even rows and columns")


@pytest.mark.parametrize("kind", ["bf16_nt", "f16_nn", "mxfp8_nt"])
def test_mid_size_full_parity_several_tiles(kind):
    M, N, K = 776, 520, 1040 if kind != "mxfp8_nt" else 1024
    x = workloads.make_random(kind, M, N, K, seed=11)
    assert_close(kind, to_bits(run(kind, x, M, N, K)), oracle_full(kind, x), f"{kind} {M}x{N}x{K}")


# --- every tile shape, forced ----------------------------------------------------------

SHAPES = [("bf16_nt", 256, 256), ("bf16_nt", 256, 192), ("bf16_nt", 128, 128), ("bf16_nt", 64, 64),
          ("f16_nn", 256, 256), ("f16_nn", 128, 128), ("f16_nn", 64, 64), ("mxfp8_nt", 256, 256)]


@pytest.fixture
def forced_tile():
    def force(tm, tn):
        tg.set_tile(tm, tn)
    yield force
    tg.set_tile(0, 0)


@pytest.mark.parametrize("kind,tm,tn", SHAPES)
def test_tile_shape_tails(kind, tm, tn, forced_tile):
    """Each tile shape over ragged M, N and K: random inputs within the
    tolerance, integer inputs bitwise."""
    forced_tile(tm, tn)
    Ks = [16, 144, 400] if kind == "mxfp8_nt" else [8, 72, 200]
    for K in Ks:
        for M in [1, 129, 300]:
            for N in [8, 200, 264]:
                x = workloads.make_random(kind, M, N, K, seed=M * 5 + N * 11 + K + tn)
                assert_close(kind, to_bits(run(kind, x, M, N, K)), oracle_full(kind, x),
                             f"{kind} {tm}x{tn} {M}x{N}x{K}")
                xi = workloads.make_integer(kind, M, N, K, seed=M + N * 3 + K + tm)
                assert_bitwise(to_bits(run(kind, xi, M, N, K)), oracle_full(kind, xi),
                               f"{kind} {tm}x{tn} int {M}x{N}x{K}")


@pytest.mark.parametrize("kind,tm,tn", SHAPES)
def test_tile_shape_mid_size_full_parity(kind, tm, tn, forced_tile):
    forced_tile(tm, tn)
    M, N, K = 776, 520, 1040 if kind != "mxfp8_nt" else 1024
    x = workloads.make_random(kind, M, N, K, seed=13)
    assert_close(kind, to_bits(run(kind, x, M, N, K)), oracle_full(kind, x), f"{kind} {tm}x{tn}")


def test_tile_shape_missing_for_entry_point_is_rejected(forced_tile):
    forced_tile(128, 128)
    a = torch.zeros(64, 64, dtype=torch.uint8, device="cuda")
    s = torch.zeros(64, 1, dtype=torch.uint8, device="cuda")
    c = torch.zeros(64, 64, dtype=torch.bfloat16, device="cuda")
    rc = tg.lib().gemm_mxfp8_nt(64, 64, 64, a.data_ptr(), a.data_ptr(), s.data_ptr(), s.data_ptr(),
                                c.data_ptr(), None)
    assert rc == tg.EINVAL and "no 128x128 tile" in tg.last_error()


@pytest.mark.parametrize("kind", ["bf16_nt", "f16_nn", "mxfp8_nt"])
def test_K_zero_writes_zeros(kind):
    M, N = 70, 40
    x = {"A": np.zeros((M, 0), np.uint16), "B": np.zeros((N, 0) if kind == "bf16_nt" else (0, N), np.uint16),
         "qA": np.zeros((M, 0), np.uint8), "qB": np.zeros((N, 0), np.uint8),
         "sA": np.zeros((M, 0), np.uint8), "sB": np.zeros((N, 0), np.uint8)}
    dt = torch.float16 if kind == "f16_nn" else torch.bfloat16
    out = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
    got = to_bits(run(kind, x, M, N, 0, out=out))
    assert np.all(got == 0)


def test_output_guard_band_untouched():
    """C inside a larger buffer: nothing outside C's M x N elements changes."""
    M, N, K = 300, 264, 136
    x = workloads.make_random("bf16_nt", M, N, K, seed=2)
    pad = 4096
    buf = torch.full((pad + M * N + pad,), 1.5, dtype=torch.bfloat16, device="cuda")
    out = buf[pad:pad + M * N].view(M, N)
    run("bf16_nt", x, M, N, K, out=out)
    b = buf.cpu()
    assert torch.all(b[:pad] == 1.5) and torch.all(b[pad + M * N:] == 1.5)
    assert_close("bf16_nt", to_bits(out), oracle_full("bf16_nt", x), "guard band")


def test_deterministic_bitwise():
    w = workloads.WORKLOADS["bf16_nt_4000x3000x5000"]
    x = workloads.make_inputs(w)
    a, b = to_dev(x["A"], "bf16"), to_dev(x["B"], "bf16")
    c1 = tg.gemm_bf16_nt(a, b)
    c2 = tg.gemm_bf16_nt(a, b)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


def test_non_default_stream():
    M, N, K = 512, 512, 512
    x = workloads.make_random("bf16_nt", M, N, K, seed=4)
    s = torch.cuda.Stream()
    a, b = to_dev(x["A"], "bf16"), to_dev(x["B"], "bf16")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        c = tg.gemm_bf16_nt(a, b, stream=s)
    s.synchronize()
    assert_close("bf16_nt", to_bits(c), oracle_full("bf16_nt", x), "stream")


def test_misaligned_device_pointer_is_rejected():
    a = torch.zeros(64 * 64 + 8, dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(64, 64, dtype=torch.bfloat16, device="cuda")
    c = torch.zeros(64, 64, dtype=torch.bfloat16, device="cuda")
    rc = tg.lib().gemm_bf16_nt(64, 64, 64, a.data_ptr() + 2, b.data_ptr(), c.data_ptr(), None)
    assert rc == tg.EALIGN and "A is not 16-byte aligned" in tg.last_error()


def _classes(v):
    """Per output: 0 finite, 1 +inf, 2 -inf, 3 NaN."""
    return np.where(np.isnan(v), 3, np.where(v == np.inf, 1, np.where(v == -np.inf, 2, 0)))


@pytest.mark.parametrize("tile", [(0, 0), (256, 256), (128, 128), (64, 64)])
def test_special_values_match_the_oracle(tile, forced_tile):
    """Infinities and NaN planted in A and B (bf16 NT, ragged sizes): every
    output that the oracle makes +inf, -inf or NaN is the same on the GPU,
    and the rest agree within the tolerance.  (IEEE semantics do not depend
    on the summation order: inf + finite = inf, inf - inf = NaN, NaN stays.)"""
    forced_tile(*tile)
    M, N, K = 300, 264, 200
    x = workloads.make_random("bf16_nt", M, N, K, seed=21)
    A, B = x["A"].copy(), x["B"].copy()
    PINF, NINF, NAN = 0x7F80, 0xFF80, 0x7FC0
    A[5, 17] = PINF                 # row 5: +-inf by the sign of B[n, 17]
    A[40, 3], A[40, 150] = PINF, NINF   # row 40: NaN unless B cancels one term
    A[299, 199] = NAN               # the last row, the last (ragged) K column
    B[7, 60] = NINF                 # column 7
    B[263, 0] = NAN                 # the last column
    x["A"], x["B"] = A, B
    got = values("bf16_nt", to_bits(run("bf16_nt", x, M, N, K)))
    ref = values("bf16_nt", oracle_full("bf16_nt", x))
    gc, rc = _classes(got), _classes(ref)
    assert (rc != 0).sum() > M + N, "the planted values should reach whole rows and columns"
    bad = np.argwhere(gc != rc)
    assert bad.size == 0, f"{len(bad)} outputs differ in class, first {bad[0]}: {got[tuple(bad[0])]} vs {ref[tuple(bad[0])]}"
    fin = rc == 0
    ok = np.abs(got[fin] - ref[fin]) <= ATOL + RTOL * np.abs(ref[fin])
    assert ok.all(), f"{int((~ok).sum())} finite outputs outside tolerance"


def test_fp16_overflow_gives_infinity():
    """fp16 NN: sums past 65504 round to +-inf, as the oracle's one rounding does."""
    M, N, K = 64, 72, 136
    A = np.full((M, K), 0x5000, np.uint16)      # 32.0
    A[1::2] = 0xD000                            # -32.0 on odd rows
    B = np.full((K, N), 0x5000, np.uint16)
    B[:, 5] = 0x2C00                            # 0.0625: column 5 stays finite (272)
    x = {"A": A, "B": B}
    got = to_bits(run("f16_nn", x, M, N, K))
    ref = oracle_full("f16_nn", x)
    assert np.array_equal(got, ref)
    assert np.all(got[0::2, 0] == 0x7C00) and np.all(got[1::2, 0] == 0xFC00) and np.all(np.abs(f16_values(got[:, 5])) == 272)


def test_mxfp8_nan_element_and_nan_scale_propagate():
    """A NaN e4m3fn element (0x7F) and a NaN e8m0 scale (0xFF) make their
    rows' and columns' outputs NaN on the GPU exactly where the oracle's do;
    the rest match bit for bit (integer elements, unit scales)."""
    M, N, K = 264, 136, 384
    x = workloads.make_integer("mxfp8_nt", M, N, K, seed=23)
    x["qA"][3, 200] = 0x7F              # row 3
    x["sB"][70, 2] = 0xFF               # column 70 (its third 128-K block)
    got = to_bits(run("mxfp8_nt", x, M, N, K))
    ref = oracle_full("mxfp8_nt", x)
    g, r = bf16_values(got), bf16_values(ref)
    assert np.isnan(r[3]).all() and np.isnan(r[:, 70]).all()
    assert np.array_equal(np.isnan(g), np.isnan(r))
    fin = ~np.isnan(r)
    assert np.array_equal(got[fin], ref[fin])


def test_graph_replays_match_eager():
    # The entry points record only kernel launches (no memset, no
    # allocation), so a caller may capture them into a HIP graph.  Each
    # replay, with eager work and synchronisations between replays, must
    # reproduce the eager outputs bit for bit, and must read the inputs as
    # they are at replay time (the second pass doubles them: scaling by 2 is
    # exact, so every output doubles exactly).
    M, N, K = 520, 264, 1008                   # K ragged against the 64- and 128-element slices
    xb = workloads.make_random("bf16_nt", M, N, K, seed=11)
    a, b = to_dev(xb["A"], "bf16"), to_dev(xb["B"], "bf16")
    g = torch.Generator().manual_seed(12)
    xa32 = torch.randn(M, K, generator=g).cuda()
    xb32 = torch.randn(N, K, generator=g).cuda()
    KB = (K + 127) // 128
    c16 = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    c8 = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    qa = torch.empty(M, K, dtype=torch.uint8, device="cuda")
    qb = torch.empty(N, K, dtype=torch.uint8, device="cuda")
    sa = torch.empty(M, KB, dtype=torch.uint8, device="cuda")
    sb = torch.empty(N, KB, dtype=torch.uint8, device="cuda")

    def work():
        tg.gemm_bf16_nt(a, b, out=c16)
        tg.quantize_mxfp8(xa32, q=qa, scales=sa)
        tg.quantize_mxfp8(xb32, q=qb, scales=sb)
        tg.gemm_mxfp8_nt(qa, qb, sa, sb, out=c8)

    print(f"[gpu] graph capture bf16 NT + quantise + MXFP8 NT M={M} N={N} K={K}", flush=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref16, ref8 = c16.clone(), c8.clone()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work()
    torch.cuda.synchronize()
    for rep in range(4):
        if rep == 2:
            a.mul_(2)
            xa32.mul_(2)
            ref16, ref8 = ref16 * 2, ref8 * 2
        for t in (c16, c8, qa, qb, sa, sb):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(c16.view(torch.int16), ref16.view(torch.int16)), f"bf16 replay {rep}"
        assert torch.equal(c8.view(torch.int16), ref8.view(torch.int16)), f"mxfp8 replay {rep}"


def test_host_threads_keep_their_own_tile_and_error():
    # tgemm_set_tile and the last-error message are per host thread: a
    # thread that forces a tile the NN entry point lacks gets an error,
    # while another thread's calls, with the automatic choice, run and see
    # no message.  Both threads launch on streams of their own.
    import threading
    M, N, K = 320, 264, 520
    x = workloads.make_random("f16_nn", M, N, K, seed=13)
    a, b = to_dev(x["A"], "f16"), to_dev(x["B"], "f16")
    torch.cuda.synchronize()
    out = {}

    def forced():
        try:
            tg.set_tile(256, 192)
            with pytest.raises(tg.TgemmError, match="256x192"):
                tg.gemm_f16_nn(a, b, stream=torch.cuda.Stream())
            out["forced"] = tg.last_error()
        except BaseException as e:  # reported by the main thread
            out["forced_exc"] = e
        finally:
            tg.set_tile(0, 0)

    def auto():
        try:
            s = torch.cuda.Stream()
            cs = [tg.gemm_f16_nn(a, b, stream=s) for _ in range(20)]
            s.synchronize()
            out["auto"] = (cs, tg.last_error())
        except BaseException as e:
            out["auto_exc"] = e

    print(f"[gpu] two host threads, f16_nn M={M} N={N} K={K}", flush=True)
    threads = [threading.Thread(target=forced), threading.Thread(target=auto)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads)
    for k in ("forced_exc", "auto_exc"):
        if k in out:
            raise out[k]
    assert "256x192" in out["forced"]
    cs, msg = out["auto"]
    assert msg == ""
    ref = oracle_full("f16_nn", x)
    for c in cs:
        assert_close("f16_nn", to_bits(c), ref, "thread")
