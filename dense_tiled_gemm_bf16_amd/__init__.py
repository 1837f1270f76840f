"""Python binding of libtgemm.so, the tiled dense GEMM library for MI355X.

Argument marshalling only: every step of the GEMM runs in the library's
gfx950 kernels.  The functions here check tensor dtypes, shapes and
contiguity, allocate the output when none is given, and call the C entry
point of the same name on the device the tensors live on, on that device's
current HIP stream unless a stream is given.  There is no fallback:
if libtgemm.so is missing the import of the library fails loudly.

The C ABI itself is declared in include/tgemm.h; ``lib()`` returns the
ctypes handle with those signatures for callers that hold raw pointers.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libtgemm.so")

OK, EINVAL, EALIGN, ETOOBIG, EHIP = 0, -1, -2, -3, -4

_lib = None


class TgemmError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


def lib() -> ctypes.CDLL:
    """The loaded libtgemm.so with argument types set (raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m dense_tiled_gemm_bf16_amd.build` "
            "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    i64, p = ctypes.c_int64, ctypes.c_void_p
    L.gemm_bf16_nt.argtypes = [i64, i64, i64, p, p, p, p]
    L.gemm_f16_nn.argtypes = [i64, i64, i64, p, p, p, p]
    L.gemm_mxfp8_nt.argtypes = [i64, i64, i64, p, p, p, p, p, p]
    L.gemm_mxfp4_nt.argtypes = [i64, i64, i64, p, p, p, p, p, p]
    L.gemm_mxfp4_nt.restype = ctypes.c_int
    L.gemm_mxfp6_nt.argtypes = [ctypes.c_int, i64, i64, i64, p, p, p, p, p, p]
    L.gemm_mxfp6_nt.restype = ctypes.c_int
    for f in (L.gemm_bf16_nt, L.gemm_f16_nn, L.gemm_mxfp8_nt):
        f.restype = ctypes.c_int
    L.tgemm_init.argtypes = []
    L.tgemm_init.restype = ctypes.c_int
    L.tgemm_last_error.argtypes = []
    L.tgemm_last_error.restype = ctypes.c_char_p
    L.tgemm_set_tile.argtypes = [ctypes.c_int, ctypes.c_int]
    L.tgemm_set_tile.restype = ctypes.c_int
    L.quantize_mxfp8.argtypes = [i64, i64, p, p, p, p]
    for f in (L.gemm_bf16, L.gemm_f16):
        f.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, p, i64, p, i64, p, i64, p]
        f.restype = ctypes.c_int
    L.quantize_mxfp8.restype = ctypes.c_int
    for f in (L.gemm_bf16_splitk, L.gemm_f16_splitk):
        f.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, p, i64, p, i64, p, i64, ctypes.c_int, p,
                      ctypes.c_uint64, p]
        f.restype = ctypes.c_int
    L.gemm_bf16_splitk_noalloc.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, p, i64, p, i64, p, i64,
                                           ctypes.c_int, p]
    L.gemm_bf16_splitk_noalloc.restype = ctypes.c_int
    L.tgemm_splitk_workspace_bytes.argtypes = [i64, i64, ctypes.c_int]
    L.tgemm_splitk_workspace_bytes.restype = ctypes.c_uint64
    L.tgemm_clock_probe.argtypes = [p, ctypes.POINTER(ctypes.c_int), p]
    L.tgemm_clock_probe.restype = ctypes.c_int
    _lib = L
    return L


def last_error() -> str:
    return lib().tgemm_last_error().decode()


def check(rc: int) -> None:
    if rc != OK:
        raise TgemmError(rc, last_error())


def init() -> None:
    check(lib().tgemm_init())


def set_tile(tile_m: int = 0, tile_n: int = 0) -> None:
    """Force the output tile of this thread's later calls; (0, 0) restores
    the library's own choice (tgemm_set_tile)."""
    check(lib().tgemm_set_tile(tile_m, tile_n))


def _torch():
    import torch
    return torch


def _stream_ptr(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    elif stream.device != device:
        raise ValueError(f"stream is on {stream.device}, the tensors on {device}")
    return ctypes.c_void_p(stream.cuda_stream)


def _same_device(**named):
    """The one device all the named tensors live on (raises otherwise)."""
    devs = {n: t.device for n, t in named.items()}
    first = next(iter(devs.values()))
    for n, d in devs.items():
        if d != first:
            raise ValueError(f"{n} is on {d}, not on {first} with the other operands")
    return first


def _call(fn, device, stream, *args):
    """Call a C entry point with the tensors' device current (the library
    sets up and launches on the current device) and check its status."""
    torch = _torch()
    with torch.cuda.device(device):
        check(fn(*args, _stream_ptr(stream, device)))


def _want(t, name, dtype, shape):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major, packed)")


def _out(out, shape, dtype, like):
    torch = _torch()
    if out is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    _want(out, "out", dtype, shape)
    return out


def gemm_bf16_nt(a, b, out=None, stream=None):
    """C = a @ b.T for bf16 a (M,K), b (N,K) -> bf16 (M,N), fp32 accumulation."""
    torch = _torch()
    M, K = a.shape
    N = b.shape[0]
    _want(a, "a", torch.bfloat16, (M, K))
    _want(b, "b", torch.bfloat16, (N, K))
    c = _out(out, (M, N), torch.bfloat16, a)
    dev = _same_device(a=a, b=b, out=c)
    _call(lib().gemm_bf16_nt, dev, stream, M, N, K, a.data_ptr(), b.data_ptr(), c.data_ptr())
    return c


def gemm_f16_nn(a, b, out=None, stream=None):
    """C = a @ b for fp16 a (M,K), b (K,N) -> fp16 (M,N), fp32 accumulation."""
    torch = _torch()
    M, K = a.shape
    N = b.shape[1]
    _want(a, "a", torch.float16, (M, K))
    _want(b, "b", torch.float16, (K, N))
    c = _out(out, (M, N), torch.float16, a)
    dev = _same_device(a=a, b=b, out=c)
    _call(lib().gemm_f16_nn, dev, stream, M, N, K, a.data_ptr(), b.data_ptr(), c.data_ptr())
    return c


def gemm_mxfp8_nt(a, b, scale_a, scale_b, out=None, stream=None):
    """Block-scaled FP8 NT GEMM -> bf16 (M,N).

    a (M,K), b (N,K): e4m3fn elements (torch.float8_e4m3fn or uint8 bytes);
    scale_a (M,ceil(K/128)), scale_b (N,ceil(K/128)): e8m0 bytes (uint8).
    """
    torch = _torch()
    M, K = a.shape
    N = b.shape[0]
    KB = (K + 127) // 128
    if a.dtype == torch.float8_e4m3fn:
        a = a.view(torch.uint8)
    if b.dtype == torch.float8_e4m3fn:
        b = b.view(torch.uint8)
    _want(a, "a", torch.uint8, (M, K))
    _want(b, "b", torch.uint8, (N, K))
    _want(scale_a, "scale_a", torch.uint8, (M, KB))
    _want(scale_b, "scale_b", torch.uint8, (N, KB))
    c = _out(out, (M, N), torch.bfloat16, a)
    dev = _same_device(a=a, b=b, scale_a=scale_a, scale_b=scale_b, out=c)
    _call(lib().gemm_mxfp8_nt, dev, stream, M, N, K, a.data_ptr(), b.data_ptr(), scale_a.data_ptr(),
          scale_b.data_ptr(), c.data_ptr())
    return c


def quantize_mxfp8(x, q=None, scales=None, stream=None):
    """float32 (M,K) -> (q uint8 (M,K) e4m3fn bytes, scales uint8 (M,ceil(K/128))
    e8m0 bytes), the operands of gemm_mxfp8_nt (quantize_mxfp8 in the C ABI)."""
    torch = _torch()
    M, K = x.shape
    KB = (K + 127) // 128
    _want(x, "x", torch.float32, (M, K))
    q = _out(q, (M, K), torch.uint8, x)
    scales = _out(scales, (M, KB), torch.uint8, x)
    dev = _same_device(x=x, q=q, scales=scales)
    _call(lib().quantize_mxfp8, dev, stream, M, K, x.data_ptr(), q.data_ptr(), scales.data_ptr())
    return q, scales


def _layout(t, name):
    """(transposed, leading dimension) of a 2-D tensor stored row-major
    (stride (ld, 1)) or as the transpose of a row-major array (stride (1, ld))."""
    r, c = t.shape
    s0, s1 = t.stride()
    if s1 == 1 and (s0 >= c or r == 1):
        return 0, max(s0, c)
    if s0 == 1 and (s1 >= r or c == 1):
        return 1, max(s1, r)
    raise ValueError(f"{name} must be row-major or a transposed row-major view (strides {t.stride()})")


def gemm(a, b, out=None, stream=None):
    """C = a @ b for 2-D bfloat16 or float16 CUDA tensors (gemm_bf16 / gemm_f16).

    a (M,K) and b (K,N) may each be row-major with any row stride or the
    transpose of such an array (e.g. ``x.t()``); out (M,N) row-major with
    any row stride, allocated when None.  Output dtype = input dtype.
    """
    torch = _torch()
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[0]:
        raise ValueError(f"shapes {tuple(a.shape)} and {tuple(b.shape)} do not multiply")
    if a.dtype != b.dtype or a.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("a and b must both be bfloat16 or both float16")
    if a.device.type != "cuda" or b.device.type != "cuda":
        raise ValueError("a and b must be on a GPU")
    M, K = a.shape
    N = b.shape[1]
    ta, lda = _layout(a, "a")
    # b is (K, N): row-major means B stored K x N (trans_b = 0); a transposed
    # view means B stored N x K (trans_b = 1).
    tb, ldb = _layout(b, "b")
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    if out.dtype != a.dtype or tuple(out.shape) != (M, N) or (out.stride(1) != 1 and N > 1):
        raise ValueError("out must be a row-major (M, N) tensor of the input dtype")
    ldc = max(out.stride(0), N)
    dev = _same_device(a=a, b=b, out=out)
    fn = lib().gemm_bf16 if a.dtype == torch.bfloat16 else lib().gemm_f16
    _call(fn, dev, stream, ta, tb, M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb, out.data_ptr(), ldc)
    return out


def gemm_splitk(a, b, splits=0, out=None, workspace=None, stream=None):
    """C = a @ b as gemm(), with K split over several workgroups per output
    tile (gemm_bf16_splitk / gemm_f16_splitk).  splits: 0 lets the library
    choose, 1 disables, 2-16 forces.  workspace: a 16-byte aligned CUDA
    tensor of at least tgemm_splitk_workspace_bytes(M, N, splits) bytes;
    allocated (uint8) when None."""
    torch = _torch()
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[0]:
        raise ValueError(f"shapes {tuple(a.shape)} and {tuple(b.shape)} do not multiply")
    if a.dtype != b.dtype or a.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("a and b must both be bfloat16 or both float16")
    if a.device.type != "cuda" or b.device.type != "cuda":
        raise ValueError("a and b must be on a GPU")
    M, K = a.shape
    N = b.shape[1]
    ta, lda = _layout(a, "a")
    tb, ldb = _layout(b, "b")
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    if out.dtype != a.dtype or tuple(out.shape) != (M, N) or (out.stride(1) != 1 and N > 1):
        raise ValueError("out must be a row-major (M, N) tensor of the input dtype")
    ldc = max(out.stride(0), N)
    need = lib().tgemm_splitk_workspace_bytes(M, N, splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=a.device)
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous CUDA tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    dev = _same_device(a=a, b=b, out=out, workspace=workspace)
    fn = lib().gemm_bf16_splitk if a.dtype == torch.bfloat16 else lib().gemm_f16_splitk
    _call(fn, dev, stream, ta, tb, M, N, K, a.data_ptr(), lda, b.data_ptr(), ldb, out.data_ptr(), ldc, splits,
          workspace.data_ptr(), ws_bytes)
    return out


def gemm_mxfp4_nt(a, b, scale_a, scale_b, out=None, stream=None):
    """Block-scaled FP4 NT GEMM -> bf16 (M,N).

    a (M,K/2), b (N,K/2): packed E2M1 bytes (uint8; element 2i in the low
    nibble of byte i); scale_a (M,K/32), scale_b (N,K/32): e8m0 bytes.
    """
    torch = _torch()
    M, KH = a.shape
    N = b.shape[0]
    K = 2 * KH
    _want(a, "a", torch.uint8, (M, KH))
    _want(b, "b", torch.uint8, (N, KH))
    _want(scale_a, "scale_a", torch.uint8, (M, K // 32))
    _want(scale_b, "scale_b", torch.uint8, (N, K // 32))
    c = _out(out, (M, N), torch.bfloat16, a)
    dev = _same_device(a=a, b=b, scale_a=scale_a, scale_b=scale_b, out=c)
    _call(lib().gemm_mxfp4_nt, dev, stream, M, N, K, a.data_ptr(), b.data_ptr(), scale_a.data_ptr(),
          scale_b.data_ptr(), c.data_ptr())
    return c


FP6_FORMATS = {"e2m3": 0, "e3m2": 1}   # TGEMM_FP6_E2M3, TGEMM_FP6_E3M2


def gemm_mxfp6_nt(a, b, scale_a, scale_b, fmt="e2m3", out=None, stream=None):
    """Block-scaled FP6 NT GEMM -> bf16 (M,N).

    a (M,3K/4), b (N,3K/4): FP6 elements of type fmt ("e2m3" or "e3m2")
    packed densely (element k at bits 6k .. 6k+5 of the row, little-endian),
    uint8; scale_a (M,K/32), scale_b (N,K/32): e8m0 bytes.  K % 64 == 0.
    """
    torch = _torch()
    M, RB = a.shape
    N = b.shape[0]
    if RB % 3 != 0:
        raise ValueError(f"a has {RB} bytes per row; packed FP6 rows hold 3 bytes per 4 elements")
    K = RB // 3 * 4
    if fmt not in FP6_FORMATS:
        raise ValueError(f"fmt must be one of {sorted(FP6_FORMATS)}")
    _want(a, "a", torch.uint8, (M, RB))
    _want(b, "b", torch.uint8, (N, RB))
    _want(scale_a, "scale_a", torch.uint8, (M, K // 32))
    _want(scale_b, "scale_b", torch.uint8, (N, K // 32))
    c = _out(out, (M, N), torch.bfloat16, a)
    dev = _same_device(a=a, b=b, scale_a=scale_a, scale_b=scale_b, out=c)
    _call(lib().gemm_mxfp6_nt, dev, stream, FP6_FORMATS[fmt], M, N, K, a.data_ptr(), b.data_ptr(),
          scale_a.data_ptr(), scale_b.data_ptr(), c.data_ptr())
    return c
