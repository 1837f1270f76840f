"""Seeded synthetic inputs for the tiled dense GEMM.

This module only *produces inputs*; it holds none of the GEMM's arithmetic.
Both the CPU oracle (``oracle/``) and the GPU library receive the arrays made
here, as raw bit patterns (numpy ``uint16`` for bf16/fp16, ``uint8`` for the
fp8 elements and e8m0 scales), so the two sides see identical bytes.

Recipe (the pages draw ``torch.randn`` matrices, TileLang SM100 README,
"Compilation and Usage"):  a CPU ``torch.Generator`` seeded with ``seed``
draws A and then B as float32 N(0, 1) samples, which are rounded to the
input type by torch's own round-to-nearest-even cast.  For the block-scaled
FP8 workload the float32 samples are quantised per row and per 128 K
elements: the scale is the smallest power of two 2^e with
``absmax <= 448 * 2^e``, stored as the e8m0 byte ``e + 127``, and the
elements are ``x * 2^-e`` cast by torch to OCP ``float8_e4m3fn``.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

FP8_E4M3_MAX = 448.0
SCALE_BLOCK_K = 128
FP4_E2M1_MAX = 6.0
FP4_BLOCK_K = 32                     # OCP MX block: one scale per 32 elements
# Magnitudes of the FP4 E2M1 codes 0..7 (sign in bit 3).
FP4_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _fp6_grid(ebits: int, bias: int) -> np.ndarray:
    """Magnitudes of the 32 non-negative OCP FP6 codes, in code order
    (exponent field 0 subnormal; no infinities or NaN)."""
    mbits = 5 - ebits
    out = []
    for c in range(32):
        e, f = c >> mbits, c & ((1 << mbits) - 1)
        out.append(math.ldexp(f, 1 - bias - mbits) if e == 0 else math.ldexp((1 << mbits) + f, e - bias - mbits))
    return np.array(out)


# OCP FP6 element types: name -> (magnitude grid, largest value).
FP6 = {"e2m3": (_fp6_grid(2, 1), 7.5), "e3m2": (_fp6_grid(3, 3), 28.0)}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str          # "bf16_nt" | "f16_nn" | "mxfp8_nt"
    M: int
    N: int
    K: int
    description: str

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


# The five workloads this library is checked and measured on.
WORKLOADS = {
    w.name: w for w in (
        Workload("bf16_nt_256", "bf16_nt", 256, 256, 256,
                 "bf16 NT GEMM M=N=K=256"),
        Workload("f16_nn_1024", "f16_nn", 1024, 1024, 1024,
                 "fp16 NN GEMM M=N=K=1024"),
        Workload("bf16_nt_4096x4096x8192", "bf16_nt", 4096, 4096, 8192,
                 "bf16 NT GEMM M=4096 N=4096 K=8192"),
        Workload("bf16_nt_4000x3000x5000", "bf16_nt", 4000, 3000, 5000,
                 "bf16 NT GEMM M=4000 N=3000 K=5000 (ragged tails)"),
        # Few output tiles, deep K: the case the K split is for.
        Workload("bf16_nt_512x512x4096", "bf16_nt", 512, 512, 4096,
                 "bf16 NT GEMM M=N=512 K=4096 (few tiles, deep K)"),
        Workload("mxfp8_nt_4096", "mxfp8_nt", 4096, 4096, 4096,
                 "block-scaled fp8 (e4m3 + e8m0 per 128 K) NT GEMM M=N=K=4096"),
        # The step before the block-scaled GEMM: one of its operands, quantised.
        Workload("mxfp4_nt_4096", "mxfp4_nt", 4096, 4096, 4096,
                 "block-scaled fp4 (e2m1 + e8m0 per 32 K) NT GEMM M=N=K=4096"),
        Workload("mxfp6_e2m3_nt_4096", "mxfp6_e2m3_nt", 4096, 4096, 4096,
                 "block-scaled fp6 (e2m3 + e8m0 per 32 K) NT GEMM M=N=K=4096"),
        Workload("quant_mxfp8_4096", "quant_mxfp8", 4096, 0, 4096,
                 "block-scale quantiser fp32 -> e4m3fn + e8m0 per 128 K, M=K=4096"),
    )
}


def generator(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def randn_f32(shape, g: torch.Generator) -> torch.Tensor:
    return torch.randn(*shape, generator=g, dtype=torch.float32)


def to_bits(t: torch.Tensor) -> np.ndarray:
    """Bit patterns of a CPU bf16/fp16 tensor as numpy uint16."""
    assert t.dtype in (torch.bfloat16, torch.float16)
    return t.contiguous().view(torch.int16).numpy().view(np.uint16).copy()


def randn_bits(shape, dtype: torch.dtype, g: torch.Generator) -> np.ndarray:
    return to_bits(randn_f32(shape, g).to(dtype))


def quantize_mxfp8(x: torch.Tensor):
    """Quantise float32 rows to e4m3fn bytes with one e8m0 scale per 128 K.

    Returns (q uint8 (R, K), scales uint8 (R, ceil(K/128))).  The scale of a
    block is the smallest 2^e with absmax <= 448 * 2^e (found from the exact
    binary exponent of absmax, no log2), clamped to e in [-127, 127]; an
    all-zero block gets e = -127 (byte 0).  Elements are x * 2^-e, which is
    exact, cast once to e4m3fn by torch (round to nearest even).
    """
    assert x.dtype == torch.float32 and x.dim() == 2
    R, K = x.shape
    KB = (K + SCALE_BLOCK_K - 1) // SCALE_BLOCK_K
    pad = KB * SCALE_BLOCK_K - K
    xp = torch.nn.functional.pad(x, (0, pad)) if pad else x
    absmax = xp.view(R, KB, SCALE_BLOCK_K).abs().amax(dim=2).double().numpy()
    frac, exp = np.frexp(absmax)                 # absmax = frac * 2^exp, frac in [0.5, 1)
    # absmax / 2^(exp-9) = frac * 512 in [256, 512): <= 448 iff frac <= 0.875.
    e = exp.astype(np.int64) - 9 + (frac > FP8_E4M3_MAX / 512.0)
    e = np.where(absmax == 0.0, -127, e)
    e = np.clip(e, -127, 127)
    scales = (e + 127).astype(np.uint8)
    mult = torch.from_numpy(np.ldexp(1.0, -e)).float()            # 2^-e, exact in fp32
    y = xp.view(R, KB, SCALE_BLOCK_K) * mult[:, :, None]
    q = y.reshape(R, KB * SCALE_BLOCK_K)[:, :K].to(torch.float8_e4m3fn)
    return q.contiguous().view(torch.uint8).numpy().copy(), scales


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """FP4 codes (R, K), K even -> bytes (R, K/2): element 2i in the low nibble."""
    c = codes.astype(np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def quantize_mxfp4(x: torch.Tensor):
    """Quantise float32 rows (R, K), K % 32 == 0, to packed E2M1 with one e8m0
    scale per 32 K elements: the smallest 2^e with absmax <= 6 * 2^e (the
    same rule as the fp8 inputs, with FP4's largest value), then each
    x * 2^-e rounded to the nearest E2M1 value, ties to the even code.
    Returns (q uint8 (R, K/2), scales uint8 (R, K/32))."""
    xr = x.double().numpy()
    R, K = xr.shape
    KB = K // FP4_BLOCK_K
    blocks = xr.reshape(R, KB, FP4_BLOCK_K)
    absmax = np.abs(blocks).max(axis=2)
    frac, exp = np.frexp(absmax)             # absmax = frac * 2^exp, frac in [0.5, 1)
    # absmax / 2^(exp-3) = 8 frac in [4, 8): <= 6 iff frac <= 0.75.
    e = exp.astype(np.int64) - 3 + (frac > FP4_E2M1_MAX / 8.0)
    e = np.clip(np.where(absmax == 0.0, -127, e), -127, 127)
    y = blocks * np.exp2(-e)[:, :, None]                      # exact power-of-two scaling
    a = np.abs(y).reshape(R, K)
    lo = np.clip(np.searchsorted(FP4_GRID, a, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    dlo, dhi = a - FP4_GRID[lo], FP4_GRID[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(pick_hi, hi, lo) | (np.signbit(y.reshape(R, K)) & (a > 0)).astype(np.int64) << 3
    return pack_fp4(code), (e + 127).astype(np.uint8)


def pack_fp6(codes: np.ndarray) -> np.ndarray:
    """FP6 codes (R, K), K % 4 == 0 -> bytes (R, 3K/4): element k at bits
    6k .. 6k + 5 of the row read as a little-endian bit string."""
    c = codes.astype(np.uint32)
    R, K = c.shape
    v = c[:, 0::4] | (c[:, 1::4] << 6) | (c[:, 2::4] << 12) | (c[:, 3::4] << 18)   # 24 bits per 4 elements
    out = np.empty((R, K // 4, 3), np.uint8)
    out[:, :, 0] = v & 255
    out[:, :, 1] = (v >> 8) & 255
    out[:, :, 2] = v >> 16
    return out.reshape(R, K // 4 * 3)


def quantize_mxfp6(x: torch.Tensor, fmt: str):
    """Quantise float32 rows (R, K), K % 32 == 0, to packed FP6 of element
    type fmt ("e2m3" or "e3m2") with one e8m0 scale per 32 K elements: the
    smallest 2^e with absmax <= MAX * 2^e (MAX = 7.5 or 28; the rule of the
    other block-scaled inputs), then each x * 2^-e rounded to the nearest
    FP6 value, ties to the even code.  Returns (q uint8 (R, 3K/4), scales
    uint8 (R, K/32))."""
    grid, vmax = FP6[fmt]
    xr = x.double()                                           # torch: its elementwise ops use every core
    R, K = xr.shape
    KB = K // FP4_BLOCK_K
    blocks = xr.reshape(R, KB, FP4_BLOCK_K)
    absmax = blocks.abs().amax(dim=2)
    frac, exp = torch.frexp(absmax)                           # absmax = frac * 2^exp, frac in [0.5, 1)
    mfrac, mexp = math.frexp(vmax)                            # vmax = mfrac * 2^mexp
    # absmax / 2^(exp - mexp) = 2^mexp frac <= vmax iff frac <= mfrac.
    e = exp.long() - mexp + (frac > mfrac).long()
    e = torch.where(absmax == 0.0, torch.full_like(e, -127), e).clamp(-127, 127)
    y = (blocks * torch.exp2(-e.double())[:, :, None]).reshape(R, K)   # exact power-of-two scaling
    a = y.abs()
    gt = torch.from_numpy(grid)
    lo = (torch.bucketize(a, gt, right=True) - 1).clamp(0, 31)
    hi = (lo + 1).clamp(max=31)
    dlo, dhi = a - gt[lo], gt[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0) & (hi != lo))
    code = torch.where(pick_hi, hi, lo) | ((torch.signbit(y) & (a > 0)).long() << 5)
    e = e.numpy()
    code = code.numpy()
    return pack_fp6(code), (e + 127).astype(np.uint8)


def fp6_format(kind: str) -> str:
    """"mxfp6_e2m3_nt" -> "e2m3"."""
    return kind.split("_")[1]


def make_inputs(w: Workload | str, seed: int = 0):
    """Inputs of a workload as a dict of numpy bit-pattern arrays.

    bf16_nt: A (M,K), B (N,K) uint16.   f16_nn: A (M,K), B (K,N) uint16.
    mxfp8_nt: qA (M,K), qB (N,K) uint8 and sA (M,KB), sB (N,KB) uint8.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    return make_random(w.kind, w.M, w.N, w.K, seed)


def make_random(kind: str, M: int, N: int, K: int, seed: int = 0):
    g = generator(seed)
    if kind == "bf16_nt":
        return {"A": randn_bits((M, K), torch.bfloat16, g),
                "B": randn_bits((N, K), torch.bfloat16, g)}
    if kind == "f16_nn":
        return {"A": randn_bits((M, K), torch.float16, g),
                "B": randn_bits((K, N), torch.float16, g)}
    if kind == "quant_mxfp8":
        return {"X": randn_f32((M, K), g).numpy()}
    if kind == "mxfp4_nt":
        a = randn_f32((M, K), g)
        b = randn_f32((N, K), g)
        qA, sA = quantize_mxfp4(a)
        qB, sB = quantize_mxfp4(b)
        return {"qA": qA, "qB": qB, "sA": sA, "sB": sB}
    if kind == "mxfp8_nt":
        a = randn_f32((M, K), g)
        b = randn_f32((N, K), g)
        qA, sA = quantize_mxfp8(a)
        qB, sB = quantize_mxfp8(b)
        return {"qA": qA, "qB": qB, "sA": sA, "sB": sB}
    if kind in ("mxfp6_e2m3_nt", "mxfp6_e3m2_nt"):
        a = randn_f32((M, K), g)
        b = randn_f32((N, K), g)
        qA, sA = quantize_mxfp6(a, fp6_format(kind))
        qB, sB = quantize_mxfp6(b, fp6_format(kind))
        return {"qA": qA, "qB": qB, "sA": sA, "sB": sB}
    raise ValueError(kind)


def make_integer(kind: str, M: int, N: int, K: int, seed: int = 0, lo: int = -2, hi: int = 2):
    """Integer-valued inputs in [lo, hi] (exact in every input type).

    With |values| <= 2 and K <= 2^21 every partial sum is an integer below
    2^24, so an fp32 accumulator is exact whatever the summation order.
    For mxfp8 every scale is 2^0 (byte 127).
    """
    g = generator(seed)

    def ints(shape):
        return torch.randint(lo, hi + 1, shape, generator=g, dtype=torch.int32).float()

    if kind == "bf16_nt":
        return {"A": to_bits(ints((M, K)).bfloat16()), "B": to_bits(ints((N, K)).bfloat16())}
    if kind == "f16_nn":
        return {"A": to_bits(ints((M, K)).half()), "B": to_bits(ints((K, N)).half())}
    if kind == "mxfp4_nt":
        # Integers in [lo, hi] are E2M1 codes 0 (0), 2 (1), 4 (2) with sign bit 8.
        code = {0: 0, 1: 2, 2: 4, -1: 10, -2: 12}
        lut = np.array([code[v] for v in range(-2, 3)], np.uint8)
        KB = K // FP4_BLOCK_K
        qA = pack_fp4(lut[ints((M, K)).numpy().astype(np.int64) + 2])
        qB = pack_fp4(lut[ints((N, K)).numpy().astype(np.int64) + 2])
        return {"qA": qA, "qB": qB, "sA": np.full((M, KB), 127, np.uint8), "sB": np.full((N, KB), 127, np.uint8)}
    if kind in ("mxfp6_e2m3_nt", "mxfp6_e3m2_nt"):
        # Integers in [lo, hi] are exact in both FP6 types; their codes are
        # found on the type's own grid (sign bit 32).
        grid = FP6[fp6_format(kind)][0]
        lut = np.array([int(np.flatnonzero(grid == abs(v))[0]) | (32 if v < 0 else 0) for v in range(-2, 3)],
                       np.uint8)
        KB = K // FP4_BLOCK_K
        qA = pack_fp6(lut[ints((M, K)).numpy().astype(np.int64) + 2])
        qB = pack_fp6(lut[ints((N, K)).numpy().astype(np.int64) + 2])
        return {"qA": qA, "qB": qB, "sA": np.full((M, KB), 127, np.uint8), "sB": np.full((N, KB), 127, np.uint8)}
    if kind == "mxfp8_nt":
        KB = (K + SCALE_BLOCK_K - 1) // SCALE_BLOCK_K
        qA = ints((M, K)).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
        qB = ints((N, K)).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
        return {"qA": qA, "qB": qB,
                "sA": np.full((M, KB), 127, np.uint8), "sB": np.full((N, KB), 127, np.uint8)}
    raise ValueError(kind)


def sample_positions(M: int, N: int, count: int, seed: int = 1):
    """Output positions for sampled checks: the four corners, the last row and
    column, and ``count`` seeded uniform positions."""
    rng = np.random.default_rng(seed)
    fixed = [(0, 0), (0, N - 1), (M - 1, 0), (M - 1, N - 1)]
    fixed += [(M - 1, int(n)) for n in rng.integers(0, N, 8)]
    fixed += [(int(m), N - 1) for m in rng.integers(0, M, 8)]
    rows = np.concatenate([np.array([p[0] for p in fixed]), rng.integers(0, M, count)])
    cols = np.concatenate([np.array([p[1] for p in fixed]), rng.integers(0, N, count)])
    return rows.astype(np.int64), cols.astype(np.int64)


def gemm_flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def tflops(M: int, N: int, K: int, seconds: float) -> float:
    """2*M*N*K / t in TFLOP/s (the pages' throughput formula)."""
    return 2.0 * M * N * K / seconds / 1e12 if seconds > 0 else math.inf
