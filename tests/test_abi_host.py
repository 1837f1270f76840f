"""The C-ABI library on the host: it loads, exports every entry point that
include/tgemm.h declares, and rejects bad arguments with the documented
status codes and messages before touching any device.

No test here launches a kernel: every call either fails validation or has
nothing to do (M == 0 or N == 0).
"""
import ctypes
import os
import re
import subprocess

import pytest

import dense_tiled_gemm_bf16_amd as tg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tgemm.h")

A16 = 0x10000          # plausible, 16-byte aligned fake device addresses;
B16 = 0x20000000       # validation rejects the call before any use
C16 = 0x40000000


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^TGEMM_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, re.M)


def test_header_declares_the_entry_points():
    assert sorted(declared_functions()) == sorted(
        ["gemm_bf16_nt", "gemm_f16_nn", "gemm_mxfp8_nt", "gemm_mxfp4_nt", "gemm_mxfp6_nt", "gemm_bf16", "gemm_f16", "quantize_mxfp8", "tgemm_init",
         "tgemm_last_error", "tgemm_set_tile", "tgemm_clock_probe", "gemm_bf16_splitk", "gemm_f16_splitk",
         "tgemm_splitk_workspace_bytes", "gemm_bf16_splitk_noalloc"])


def test_library_exports_every_declared_symbol():
    L = tg.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", tg.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(declared_functions())


def test_header_compiles_as_c():
    src = '#include "tgemm.h"\nint main(void){ return TGEMM_OK; }\n'
    res = subprocess.run(["gcc", "-x", "c", "-std=c99", "-fsyntax-only",
                          "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                          "-D__HIP_PLATFORM_AMD__", "-"], input=src, text=True,
                         capture_output=True)
    assert res.returncode == 0, res.stderr


def _bf16(M, N, K, A=A16, B=B16, C=C16):
    return tg.lib().gemm_bf16_nt(M, N, K, A, B, C, None)


def _f16(M, N, K, A=A16, B=B16, C=C16):
    return tg.lib().gemm_f16_nn(M, N, K, A, B, C, None)


def _mx(M, N, K, A=A16, B=B16, SA=0x30000001, SB=0x30800003, C=C16):
    return tg.lib().gemm_mxfp8_nt(M, N, K, A, B, SA, SB, C, None)


def _fp4(M, N, K, A=A16, B=B16, SA=0x30000001, SB=0x30800003, C=C16):
    return tg.lib().gemm_mxfp4_nt(M, N, K, A, B, SA, SB, C, None)


def _fp6(M, N, K, A=A16, B=B16, SA=0x30000001, SB=0x30800003, C=C16, fmt=0):
    return tg.lib().gemm_mxfp6_nt(fmt, M, N, K, A, B, SA, SB, C, None)


ALL = [_bf16, _f16, _mx, _fp4, _fp6]


@pytest.mark.parametrize("call", ALL)
def test_empty_outputs_are_a_no_op(call):
    # M == 0 or N == 0: nothing to compute, success without any device work,
    # even with NULL pointers.
    assert call(0, 16, 16, A=None, B=None, C=None) == tg.OK
    assert call(16, 0, 16, A=None, B=None, C=None) == tg.OK
    assert tg.last_error() == ""


@pytest.mark.parametrize("call", ALL)
def test_negative_sizes(call):
    for dims in [(-1, 16, 16), (16, -8, 16), (16, 16, -16)]:
        assert call(*dims) == tg.EINVAL
        assert "negative size" in tg.last_error()


@pytest.mark.parametrize("call,kmul", [(_bf16, 8), (_f16, 8), (_mx, 16), (_fp4, 32), (_fp6, 64)])
def test_vector_width_rules(call, kmul):
    assert call(16, 16, kmul + kmul // 2) == tg.EALIGN
    assert f"multiple of {kmul}" in tg.last_error()
    assert call(16, 12, 64) == tg.EALIGN
    assert "N=12 must be a multiple of 8" in tg.last_error()


@pytest.mark.parametrize("call", ALL)
def test_null_and_misaligned_pointers(call):
    assert call(16, 16, 64, A=None) == tg.EINVAL and "A is NULL" in tg.last_error()
    assert call(16, 16, 64, B=None) == tg.EINVAL and "B is NULL" in tg.last_error()
    assert call(16, 16, 64, C=None) == tg.EINVAL and "C is NULL" in tg.last_error()
    assert call(16, 16, 64, A=A16 + 8) == tg.EALIGN and "A is not 16-byte aligned" in tg.last_error()
    assert call(16, 16, 64, B=B16 + 2) == tg.EALIGN and "B is not 16-byte aligned" in tg.last_error()
    assert call(16, 16, 64, C=C16 + 4) == tg.EALIGN and "C is not 16-byte aligned" in tg.last_error()


def test_mxfp8_scale_pointers():
    assert _mx(16, 16, 256, SA=None) == tg.EINVAL and "scale_A is NULL" in tg.last_error()
    assert _mx(16, 16, 256, SB=None) == tg.EINVAL and "scale_B is NULL" in tg.last_error()
    # Scale arrays need no alignment: odd addresses pass validation up to the
    # device step, so only a C overlapping them is checked here.
    assert _mx(16, 16, 256, SA=C16 + 100) == tg.EINVAL and "C overlaps scale_A" in tg.last_error()


@pytest.mark.parametrize("call", ALL)
def test_output_may_not_overlap_inputs(call):
    M, N, K = 64, 64, 64
    assert call(M, N, K, C=A16 + 16) == tg.EINVAL and "C overlaps A" in tg.last_error()
    assert call(M, N, K, C=B16 - 1024 + 16 * 4) == tg.EINVAL and "C overlaps B" in tg.last_error()


def test_fp6_format_codes():
    for bad in (-1, 2, 7):
        assert _fp6(16, 16, 64, fmt=bad) == tg.EINVAL and "fmt=" in tg.last_error()


def test_too_big():
    # 256 rows of a K-slice panel must fit 31-bit buffer offsets.
    assert _bf16(16, 16, 1 << 22) == tg.ETOOBIG and "too large" in tg.last_error()
    assert _mx(16, 16, 1 << 23) == tg.ETOOBIG and "too large" in tg.last_error()
    assert _fp4(16, 16, 1 << 24) == tg.ETOOBIG and "too large" in tg.last_error()
    assert _fp6(16, 16, 11 << 20) == tg.ETOOBIG and "too large" in tg.last_error()
    far = 0x7F0000000000     # C far from the (fake, 4 GiB) B
    assert _f16(16, 1 << 16, 1 << 15, C=far) == tg.ETOOBIG and "B too large" in tg.last_error()
    assert _bf16(1 << 31, 16, 16) == tg.ETOOBIG and "below 2^31" in tg.last_error()


def test_k_major_operands_count_whole_slices_of_rows():
    """A K-major operand is read in whole slices of 64 K rows (the rows past K
    read as out of range), so K rounded up to 64, times the row stride, must
    fit 31-bit offsets, not just the K rows themselves."""
    far = 0x7F0000000000
    K, N = 16328, 1 << 16
    assert K * N * 2 < 2**31 - 1 < (K + 63) // 64 * 64 * N * 2
    assert _f16(16, N, K, C=far) == tg.ETOOBIG and "B too large" in tg.last_error()
    for fn in ("gemm_bf16", "gemm_f16"):
        assert _g(1, 0, 16, 16, K, N, 16, 16, C=far, fn=fn) == tg.ETOOBIG and "A too large" in tg.last_error()
        assert _g(0, 0, 16, N, K, K, N, N, C=far, fn=fn) == tg.ETOOBIG and "B too large" in tg.last_error()


def test_error_message_resets_after_success():
    assert _bf16(-1, 1, 1) == tg.EINVAL and tg.last_error() != ""
    assert _bf16(0, 8, 8) == tg.OK and tg.last_error() == ""


def test_python_wrapper_raises_with_code():
    with pytest.raises(tg.TgemmError) as e:
        tg.check(_bf16(-1, 1, 1))
    assert e.value.code == tg.EINVAL


def test_no_device_is_an_error_not_a_crash():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present; the no-device path cannot be exercised")
    assert tg.lib().tgemm_init() == tg.EHIP
    assert "HIP device" in tg.last_error() or "hip" in tg.last_error().lower()


def test_set_tile_validates_shapes():
    L = tg.lib()
    assert L.tgemm_set_tile(100, 100) == tg.EINVAL
    assert "no 100x100 tile" in tg.last_error()
    assert L.tgemm_set_tile(256, 128) == tg.EINVAL
    for tm, tn in [(256, 256), (256, 192), (128, 128), (64, 64), (0, 0)]:
        assert L.tgemm_set_tile(tm, tn) == tg.OK
        assert tg.last_error() == ""


def _q(M, K, X=A16, Q=C16, S=0x30000001):
    return tg.lib().quantize_mxfp8(M, K, X, Q, S, None)


def test_quantize_validation():
    L = tg.lib()
    assert _q(0, 64, X=None, Q=None, S=None) == tg.OK and _q(64, 0, X=None, Q=None, S=None) == tg.OK
    assert _q(-1, 64) == tg.EINVAL and "negative size" in tg.last_error()
    assert _q(16, 24) == tg.EALIGN and "multiple of 16" in tg.last_error()
    assert _q(16, 64, X=None) == tg.EINVAL and "x is NULL" in tg.last_error()
    assert _q(16, 64, Q=None) == tg.EINVAL and "q is NULL" in tg.last_error()
    assert _q(16, 64, S=None) == tg.EINVAL and "scales is NULL" in tg.last_error()
    assert _q(16, 64, X=A16 + 4) == tg.EALIGN and "x is not 16-byte aligned" in tg.last_error()
    assert _q(16, 64, Q=C16 + 8) == tg.EALIGN and "q is not 16-byte aligned" in tg.last_error()
    assert _q(16, 64, Q=A16 + 64) == tg.EINVAL and "q overlaps x" in tg.last_error()
    assert _q(16, 64, S=A16 + 3) == tg.EINVAL and "scales overlaps x" in tg.last_error()
    assert _q(16, 64, S=C16 + 5) == tg.EINVAL and "scales overlaps q" in tg.last_error()
    assert _q(1 << 31, 64) == tg.ETOOBIG


def _g(ta, tb, M, N, K, lda, ldb, ldc, A=A16, B=B16, C=C16, fn="gemm_bf16"):
    return getattr(tg.lib(), fn)(ta, tb, M, N, K, A, lda, B, ldb, C, ldc, None)


@pytest.mark.parametrize("fn", ["gemm_bf16", "gemm_f16"])
def test_general_entry_validation(fn):
    assert _g(0, 0, 0, 16, 16, 16, 16, 16, A=None, B=None, C=None, fn=fn) == tg.OK
    assert _g(2, 0, 16, 16, 16, 16, 16, 16, fn=fn) == tg.EINVAL and "0 or 1" in tg.last_error()
    assert _g(0, 0, -1, 16, 16, 16, 16, 16, fn=fn) == tg.EINVAL and "negative size" in tg.last_error()
    # Strides below the stored row length: A M x K (lda >= K), A K x M (lda >= M), ...
    assert _g(0, 0, 32, 16, 64, 48, 16, 16, fn=fn) == tg.EINVAL and "lda=48" in tg.last_error()
    assert _g(1, 0, 32, 16, 64, 24, 16, 16, fn=fn) == tg.EINVAL and "lda=24" in tg.last_error()
    assert _g(0, 0, 32, 16, 64, 64, 8, 16, fn=fn) == tg.EINVAL and "ldb=8" in tg.last_error()
    assert _g(0, 1, 32, 16, 64, 64, 32, 16, fn=fn) == tg.EINVAL and "ldb=32" in tg.last_error()
    assert _g(0, 0, 32, 16, 64, 64, 16, 8, fn=fn) == tg.EINVAL and "ldc=8" in tg.last_error()
    # Vector width: the contiguous dimension of each stored operand, N, and the strides.
    assert _g(0, 0, 32, 16, 60, 64, 16, 16, fn=fn) == tg.EALIGN and "contiguous dimension of A" in tg.last_error()
    assert _g(1, 0, 30, 16, 64, 32, 16, 16, fn=fn) == tg.EALIGN and "M=30" in tg.last_error()
    assert _g(0, 1, 32, 16, 60, 64, 64, 16, fn=fn) == tg.EALIGN
    assert _g(0, 0, 32, 12, 64, 64, 16, 16, fn=fn) == tg.EALIGN
    assert _g(0, 0, 32, 16, 64, 68, 16, 16, fn=fn) == tg.EALIGN and "multiples of 8" in tg.last_error()
    # Pointers and overlap.
    assert _g(0, 0, 32, 16, 64, 64, 16, 16, A=A16 + 2, fn=fn) == tg.EALIGN and "A is not" in tg.last_error()
    assert _g(0, 0, 32, 16, 64, 64, 16, 16, C=None, fn=fn) == tg.EINVAL and "C is NULL" in tg.last_error()
    assert _g(0, 0, 32, 16, 64, 64, 16, 16, C=A16 + 64, fn=fn) == tg.EINVAL and "C overlaps A" in tg.last_error()
    # 31-bit offsets: an M-contiguous A addressed as a whole.
    far = 0x7F0000000000
    assert _g(1, 0, 1 << 16, 16, 1 << 15, 1 << 16, 16, 16, C=far, fn=fn) == tg.ETOOBIG


def test_wrapper_rejects_fp6_rows_that_are_not_whole_groups():
    # 49 bytes per row is no whole number of 3-byte groups of four elements;
    # the wrapper must refuse it before any pitch is derived from it.
    import torch
    a = torch.zeros((4, 49), dtype=torch.uint8)
    with pytest.raises(ValueError, match="3 bytes per 4 elements"):
        tg.gemm_mxfp6_nt(a, a, a, a)


def test_wrapper_requires_one_device():
    import torch
    a = torch.zeros(2, device="cpu")
    b = torch.zeros(2, device="meta")
    assert tg._same_device(a=a, x=a) == torch.device("cpu")
    with pytest.raises(ValueError, match="b is on meta"):
        tg._same_device(a=a, b=b)


def test_clock_probe_validation():
    L = tg.lib()
    khz = ctypes.c_int(0)
    assert L.tgemm_clock_probe(None, ctypes.byref(khz), None) == tg.EINVAL
    assert "out is NULL" in tg.last_error()
    assert L.tgemm_clock_probe(A16 + 8, ctypes.byref(khz), None) == tg.EALIGN
    assert "aligned" in tg.last_error()


def test_splitk_validation():
    L = tg.lib()
    M, N, K = 64, 64, 256
    ws = 0x60000000
    need = L.tgemm_splitk_workspace_bytes(M, N, 2)
    assert need == 2 * M * N * 4
    assert L.tgemm_splitk_workspace_bytes(M, N, 0) == 4 * M * N * 4
    assert L.tgemm_splitk_workspace_bytes(M, N, 1) == 0
    assert L.tgemm_splitk_workspace_bytes(M, N, 17) == 0
    assert L.tgemm_splitk_workspace_bytes(0, N, 2) == 0
    call = lambda splits, w, nb: L.gemm_bf16_splitk(0, 1, M, N, K, A16, K, B16, K, C16, N, splits, w, nb, None)
    assert call(17, ws, need) == tg.EINVAL and "splits" in tg.last_error()
    assert call(-1, ws, need) == tg.EINVAL
    assert call(2, ws, need - 1) == tg.EINVAL and "workspace bytes" in tg.last_error()
    assert call(2, None, need) == tg.EINVAL and "NULL" in tg.last_error()
    assert call(2, ws + 8, need) == tg.EALIGN
    assert call(2, A16, need) == tg.EINVAL and "overlaps A" in tg.last_error()
    assert call(2, C16 - 16, need) == tg.EINVAL and "overlaps C" in tg.last_error()
    assert L.gemm_f16_splitk(0, 0, M, N, K, A16, K, B16, N, C16, N, 3, ws, need, None) == tg.EINVAL


def test_noalloc_splitk_rejects_what_the_scratch_cannot_hold():
    L = tg.lib()
    M, N, K = 1024, 1024, 4096      # 3 planes of 4 MiB > 8 MiB
    rc = L.gemm_bf16_splitk_noalloc(0, 1, M, N, K, A16, K, B16, K, C16, N, 3, None)
    assert rc == tg.ETOOBIG and "scratch" in tg.last_error()
    assert L.gemm_bf16_splitk_noalloc(0, 1, M, N, K, A16, K, B16, K, C16, N, 17, None) in (tg.EINVAL, tg.ETOOBIG)
    assert L.gemm_bf16_splitk_noalloc(0, 1, 0, N, K, A16, K, B16, K, C16, N, 2, None) == tg.OK
