"""MI355X (gfx950) fp16 GEMM: C = fp16(A @ B^T) with fp32 accumulation, and the
second contract D = A @ B (B [K,N], fp32 out).

Thin ctypes binding over ``libgemm_f16.so`` (C ABI declared in
``include/gemm_f16.h``).  This module only marshals arguments: shapes,
device pointers and the HIP stream go straight to the library, and every
step of the GEMM runs in its HIP kernels.  PyTorch supplies device memory
and streams.  There is no fallback: if the library is missing the calls
raise.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgemm_f16.so")

OK = 0
EINVAL = -1
ENULL = -2
EALIGN = -3
EDEVICE = -4
EHIP = -5
EOVERLAP = -6

TILE_AUTO = 0
TILE_256x256 = 1
TILE_128x128 = 2
TILE_64x64 = 3
TILE_256x256_W8 = 4
TILE_256x128 = 5
TILE_128x256 = 6
TILE_128x128_M16 = 7
TILE_64x128 = 8
TILE_128x64 = 9
TILES = {TILE_256x256: (256, 256), TILE_128x128: (128, 128), TILE_64x64: (64, 64),
         TILE_256x256_W8: (256, 256), TILE_256x128: (256, 128), TILE_128x256: (128, 256),
         TILE_128x128_M16: (128, 128), TILE_64x128: (64, 128), TILE_128x64: (128, 64)}
# kernel variants (block_k, LDS stages, loader waves) for gemm_f16_nt_ex
VARIANT_DEFAULT = 0
VARIANTS = {1: (64, 2, 0), 2: (64, 3, 0), 3: (32, 2, 0), 4: (32, 3, 0), 5: (32, 4, 0),
            6: (64, 2, 4), 7: (64, 3, 4)}
# tiles on v_mfma_f32_16x16x32_f16: the C = A B^T contract only
M16_TILES = (TILE_128x128_M16,)

# Every symbol include/gemm_f16.h declares.
EXPORTS = (
    "gemm_f16_nt",
    "gemm_f16_nt_ex",
    "gemm_f16_nn_f32",
    "gemm_f16_nn_f32_ex",
    "gemm_f16_status_string",
    "gemm_f16_tile_coord",
    "gemm_f16_select_tile",
    "gemm_f16_select_xcd",
)


class Options(ctypes.Structure):
    _fields_ = [("tile", ctypes.c_int32), ("swizzle", ctypes.c_int32),
                ("xcd", ctypes.c_int32), ("variant", ctypes.c_int32)]


class GemmError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"gemm_f16 error {status}: {status_string(status)}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with dense_fp16_gemm_f16_amd.build.build() "
            "(there is no fallback path)")
    L = ctypes.CDLL(LIB_PATH)
    i64, p, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32
    L.gemm_f16_nt.argtypes = [i64, i64, i64, p, p, p, p]
    L.gemm_f16_nt.restype = ctypes.c_int
    L.gemm_f16_nt_ex.argtypes = [i64, i64, i64, p, p, p, p, ctypes.POINTER(Options)]
    L.gemm_f16_nt_ex.restype = ctypes.c_int
    L.gemm_f16_nn_f32.argtypes = [i64, i64, i64, p, p, p, p]
    L.gemm_f16_nn_f32.restype = ctypes.c_int
    L.gemm_f16_nn_f32_ex.argtypes = [i64, i64, i64, p, p, p, p, ctypes.POINTER(Options)]
    L.gemm_f16_nn_f32_ex.restype = ctypes.c_int
    L.gemm_f16_status_string.argtypes = [ctypes.c_int]
    L.gemm_f16_status_string.restype = ctypes.c_char_p
    L.gemm_f16_tile_coord.argtypes = [i64, i64, i64, i32, i32,
                                      ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.gemm_f16_tile_coord.restype = ctypes.c_int
    L.gemm_f16_select_tile.argtypes = [i64, i64, i64]
    L.gemm_f16_select_tile.restype = ctypes.c_int
    L.gemm_f16_select_xcd.argtypes = [i64, i64, i32, i32]
    L.gemm_f16_select_xcd.restype = ctypes.c_int
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().gemm_f16_status_string(int(status)).decode()


def gemm_f16_nt_raw(m: int, n: int, k: int, a_ptr: int, b_ptr: int, c_ptr: int,
                    stream: int = 0, tile: int = TILE_AUTO, swizzle: int = 0, xcd: int = -1,
                    variant: int = VARIANT_DEFAULT) -> int:
    """Direct call of gemm_f16_nt_ex with integer device pointers; returns the status."""
    opt = Options(tile, swizzle, xcd, variant)
    return lib().gemm_f16_nt_ex(m, n, k, a_ptr or None, b_ptr or None, c_ptr or None,
                                stream or None, ctypes.byref(opt))


def gemm_f16_nn_f32_raw(m: int, n: int, k: int, a_ptr: int, b_ptr: int, d_ptr: int,
                        stream: int = 0, tile: int = TILE_AUTO, swizzle: int = 0, xcd: int = -1) -> int:
    """Direct call of gemm_f16_nn_f32_ex (D fp32 = A B, B [K,N]); returns the status."""
    opt = Options(tile, swizzle, xcd, 0)
    return lib().gemm_f16_nn_f32_ex(m, n, k, a_ptr or None, b_ptr or None, d_ptr or None,
                                    stream or None, ctypes.byref(opt))


def gemm_f16_nt(a, b, out=None, *, stream=None, tile: int = TILE_AUTO, swizzle: int = 0,
                xcd: int = -1):
    """C = fp16(A @ B^T) for CUDA/HIP float16 tensors A [M,K] and B [N,K].

    Runs asynchronously on ``stream`` (default: torch's current stream).
    ``out`` (float16 [M,N], contiguous, same device) is overwritten if given.
    """
    import torch

    if a.dtype != torch.float16 or b.dtype != torch.float16:
        raise TypeError("a and b must be float16")
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[1]:
        raise ValueError("expected a [M,K] and b [N,K]")
    if not (a.is_cuda and b.is_cuda) or a.device != b.device:
        raise ValueError("a and b must be on the same GPU")
    if not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("a and b must be contiguous (row-major)")
    m, k = a.shape
    n = b.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.float16, device=a.device)
    elif (out.dtype != torch.float16 or tuple(out.shape) != (m, n) or not out.is_contiguous()
          or out.device != a.device):
        raise ValueError("out must be a contiguous float16 [M,N] tensor on a's device")
    if stream is None:
        stream = torch.cuda.current_stream(a.device)
    with torch.cuda.device(a.device):
        rc = gemm_f16_nt_raw(m, n, k, a.data_ptr(), b.data_ptr(), out.data_ptr(),
                             stream.cuda_stream, tile, swizzle, xcd)
    if rc != OK:
        raise GemmError(rc)
    return out


def gemm_f16_nn_f32(a, b, out=None, *, stream=None, tile: int = TILE_AUTO, swizzle: int = 0,
                    xcd: int = -1):
    """D = A @ B in fp32 for CUDA/HIP float16 tensors A [M,K] and B [K,N]."""
    import torch

    if a.dtype != torch.float16 or b.dtype != torch.float16:
        raise TypeError("a and b must be float16")
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[0]:
        raise ValueError("expected a [M,K] and b [K,N]")
    if not (a.is_cuda and b.is_cuda) or a.device != b.device:
        raise ValueError("a and b must be on the same GPU")
    if not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("a and b must be contiguous (row-major)")
    m, k = a.shape
    n = b.shape[1]
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=a.device)
    elif (out.dtype != torch.float32 or tuple(out.shape) != (m, n) or not out.is_contiguous()
          or out.device != a.device):
        raise ValueError("out must be a contiguous float32 [M,N] tensor on a's device")
    if stream is None:
        stream = torch.cuda.current_stream(a.device)
    with torch.cuda.device(a.device):
        rc = gemm_f16_nn_f32_raw(m, n, k, a.data_ptr(), b.data_ptr(), out.data_ptr(),
                                 stream.cuda_stream, tile, swizzle, xcd)
    if rc != OK:
        raise GemmError(rc)
    return out


def tile_coord(pid: int, num_m: int, num_n: int, swizzle: int, xcd: int) -> tuple[int, int]:
    mb, nb = ctypes.c_int64(), ctypes.c_int64()
    rc = lib().gemm_f16_tile_coord(pid, num_m, num_n, swizzle, xcd, ctypes.byref(mb), ctypes.byref(nb))
    if rc != OK:
        raise GemmError(rc)
    return mb.value, nb.value


def select_tile(m: int, n: int, k: int) -> int:
    rc = lib().gemm_f16_select_tile(m, n, k)
    if rc < 0:
        raise GemmError(rc)
    return rc


def select_xcd(num_m: int, num_n: int, swizzle: int = 4, cus: int = 256) -> int:
    rc = lib().gemm_f16_select_xcd(num_m, num_n, swizzle, cus)
    if rc < 0:
        raise GemmError(rc)
    return rc
