"""fp16 output rounding, bit for bit in the range where fp16 values are
more than 1 apart.

The fp16 kernels round each fp32 sum to fp16 with round-to-nearest-even,
the rounding of the per-element half casts of the lowered kernel (velog
"tilelang", 1.3 Code Generation & Runtime).  Integer inputs in [-32, 32]
with K = 200 keep every partial sum an integer below 2^24, so the fp32
accumulation is exact whatever the order, and put many sums between 2048 and
65504, where neighbouring fp16 values are 2, 4, 8 or 16 apart: a large share
of them land exactly halfway between two fp16 values.  There
round-to-nearest-even, round-toward-zero and round-half-away-from-zero give
different bits, and the GPU must give the oracle's at every output.  Each
case first checks, on the exact integer sums, that its outputs do tell the
three roundings apart.
"""
import numpy as np
import pytest
import torch

import dense_tiled_gemm_bf16_amd as tg
import oracle
import workloads

pytestmark = pytest.mark.gpu

M, N, K = 300, 264, 200      # ragged against every tile shape
MT = 296                     # M of the transposed-A cases (A stored K x M: M is its contiguous dimension)
LO, HI = -32, 32


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


def f16_int_values(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).double().numpy()


def rounded_f16_bits(s, mode):
    """fp16 bits of the exact integer sums s (|s| < 65504) rounded toward
    zero ("rtz") or half away from zero ("rha"), from the definitions: for
    2^e <= |s| < 2^(e+1) the fp16 spacing is 2^(e-10)."""
    a = np.abs(s).astype(np.float64)
    _, ex = np.frexp(np.maximum(a, 1.0))         # a = f 2^ex, f in [0.5, 1): e = ex - 1
    ulp = np.ldexp(1.0, np.maximum(ex - 11, 0))  # integers below 2048 are exact
    q = np.floor(a / ulp) if mode == "rtz" else np.floor(a / ulp + 0.5)
    v = np.copysign(q * ulp, s.astype(np.float64))
    return v.astype(np.float16).view(np.uint16)


def check_discriminates(opA_bits, opB_bits, ref_bits, what):
    """The exact sums of this case hold fp16 ties: RTZ and RHA differ from
    the oracle's RNE output at a good share of the in-range outputs."""
    s = f16_int_values(opA_bits).astype(np.int64) @ f16_int_values(opB_bits).astype(np.int64)
    a = np.abs(s)
    inr = a < 65504
    ulp = np.ldexp(1.0, np.maximum(np.frexp(np.maximum(a, 1.0))[1] - 11, 0))
    ties = inr & (a >= 2048) & (np.mod(a, ulp) == ulp / 2)
    assert ties.sum() > 0.1 * inr.sum(), f"{what}: too few ties ({int(ties.sum())})"
    for mode in ("rtz", "rha"):
        differ = (rounded_f16_bits(s[inr], mode) != ref_bits[inr]).sum()
        assert differ > 0.05 * inr.sum(), f"{what}: {mode} would match the oracle on all but {differ} outputs"


def to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).cuda()


def to_bits(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def assert_bitwise(got, ref, what):
    diff = got != ref
    if diff.any():
        idx = np.argwhere(diff)[:8]
        raise AssertionError(f"{what}: {int(diff.sum())} of {diff.size} differ; first at "
                             f"{[tuple(int(v) for v in i) for i in idx]}: got {got[diff][:8]} want {ref[diff][:8]}")


@pytest.mark.parametrize("tile", [(256, 256), (128, 128), (64, 64)])
def test_f16_nn_ties_round_to_even(tile, forced_tile):
    forced_tile(*tile)
    x = workloads.make_integer("f16_nn", M, N, K, seed=101 + tile[0], lo=LO, hi=HI)
    ref = oracle.gemm_f16_nn(x["A"], x["B"])
    check_discriminates(x["A"], x["B"], ref, f"NN {tile}")
    print(f"[gpu] f16_nn ties tile={tile} M={M} N={N} K={K}", flush=True)
    c = tg.gemm_f16_nn(to_dev(x["A"]), to_dev(x["B"]))
    torch.cuda.synchronize()
    assert_bitwise(to_bits(c), ref, f"f16 NN {tile[0]}x{tile[1]}")


@pytest.mark.parametrize("trans_b", [0, 1], ids=["TN", "TT"])
@pytest.mark.parametrize("tile", [(0, 0), (128, 128), (64, 64)])
def test_f16_transposed_a_ties_round_to_even(trans_b, tile, forced_tile):
    """A stored K x M (op(A) = A^T); B stored K x N (TN) or N x K (TT)."""
    forced_tile(*tile)
    x = workloads.make_integer("f16_nn", MT, N, K, seed=202 + trans_b + tile[0], lo=LO, hi=HI)
    opA, opB = x["A"], x["B"]                       # M x K, K x N
    ref = oracle.gemm_f16_nn(opA, opB)
    check_discriminates(opA, opB, ref, f"T{'T' if trans_b else 'N'} {tile}")
    a = to_dev(np.ascontiguousarray(opA.T)).t()     # stored K x M
    b = to_dev(np.ascontiguousarray(opB.T)).t() if trans_b else to_dev(opB)
    print(f"[gpu] f16 T{'T' if trans_b else 'N'} ties tile={tile} M={MT} N={N} K={K}", flush=True)
    c = tg.gemm(a, b)
    torch.cuda.synchronize()
    assert_bitwise(to_bits(c), ref, f"f16 T{'T' if trans_b else 'N'} {tile}")
