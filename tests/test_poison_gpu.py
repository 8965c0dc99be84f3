"""The debug build whose kernels fill their LDS with fp16 NaN before the first
load (libgemm_f16_poison.so, -DGEMM_F16_POISON_LDS): an MFMA operand read from
LDS that no load has written would turn outputs into NaN.  Every kernel path
runs through it on {-8..8}/8 operands, where every partial sum is exact in
fp32, so C must equal the oracle bit for bit (and D its exact fp64 sum):
the direct-to-LDS kernels of every block tile with and without a K tail
(lanes past K must land zeros over the poison), the one-workgroup-per-CU
kernels, the register-staged loaders, the kernel variants and the second
contract."""
import ctypes
import os

import numpy as np
import pytest

import dense_fp16_gemm_f16_amd as g
import oracle
from dense_fp16_gemm_f16_amd import build

pytestmark = pytest.mark.gpu

GUARD = 64


def _lib():
    if not os.path.exists(build.POISON_LIB):
        pytest.skip("libgemm_f16_poison.so is not built (python -m dense_fp16_gemm_f16_amd.build --poison)")
    lib = ctypes.CDLL(build.POISON_LIB)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    for name in ("gemm_f16_nt_ex", "gemm_f16_nn_f32_ex"):
        f = getattr(lib, name)
        f.argtypes = [i64, i64, i64, vp, vp, vp, vp, ctypes.POINTER(g.Options)]
        f.restype = ctypes.c_int
    return lib


def _eighths(rng, shape):
    return (rng.integers(-8, 9, size=shape) / 8).astype(np.float16)


def _run(a_np, b_np, nn=False, a_offset=0, tile=g.TILE_AUTO, variant=0):
    import torch

    lib = _lib()
    m, k = a_np.shape
    n = b_np.shape[1] if nn else b_np.shape[0]
    dev = torch.device("cuda")
    a_buf = torch.zeros(a_offset + m * k + 8, dtype=torch.float16, device=dev)
    a_buf[a_offset:a_offset + m * k] = torch.from_numpy(a_np.reshape(-1)).to(dev)
    b = torch.from_numpy(np.ascontiguousarray(b_np)).to(dev)
    out_dtype = torch.float32 if nn else torch.float16
    c_buf = torch.full((GUARD + m * n + GUARD,), 7.0, dtype=out_dtype, device=dev)
    opt = g.Options(tile, 0, -1, variant)
    f = lib.gemm_f16_nn_f32_ex if nn else lib.gemm_f16_nt_ex
    rc = f(m, n, k, a_buf.data_ptr() + 2 * a_offset, b.data_ptr(), c_buf.data_ptr() + c_buf.element_size() * GUARD,
           None, ctypes.byref(opt))
    assert rc == g.OK, g.status_string(rc)
    torch.cuda.synchronize()
    host = c_buf.cpu().numpy()
    assert np.all(host[:GUARD] == 7.0) and np.all(host[GUARD + m * n:] == 7.0), "write outside C"
    return host[GUARD:GUARD + m * n].reshape(m, n)


def _check_nt(a, b, what, **kw):
    print("case:", what, flush=True)
    got = _run(a, b, **kw)
    ref = oracle.gemm_f16_nt(a, b)
    bad = np.argwhere(got.view(np.uint16) != ref.view(np.uint16))
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {tuple(bad[0])}: {got[tuple(bad[0])]} vs {ref[tuple(bad[0])]}"


@pytest.mark.parametrize("tile", sorted(g.TILES))
@pytest.mark.parametrize("k", [640, 1000])
def test_direct_paths_every_tile(tile, k):
    rng = np.random.default_rng(tile * 1000 + k)
    _check_nt(_eighths(rng, (300, k)), _eighths(rng, (520, k)), f"direct tile {tile} k {k}", tile=tile)


@pytest.mark.parametrize("tile,m,n,k", [(g.TILE_256x256, 4608, 4096, 256), (g.TILE_128x128, 2100, 2112, 1024),
                                        (g.TILE_256x128, 4100, 4104, 640), (g.TILE_64x64, 1100, 1064, 256),
                                        (g.TILE_64x128, 1100, 2104, 256),
                                        # a partial last K-tile, and an odd count
                                        # (a K-tile of zeros added)
                                        (g.TILE_256x256, 4608, 4096, 456), (g.TILE_128x128, 2100, 2112, 136),
                                        (g.TILE_64x64, 1100, 1064, 200), (g.TILE_256x128, 4100, 4104, 960)])
def test_one_workgroup_per_cu(tile, m, n, k):
    rng = np.random.default_rng(m + n + k)
    _check_nt(_eighths(rng, (m, k)), _eighths(rng, (n, k)), f"per-CU tile {tile} {m}x{n}x{k}", tile=tile)


@pytest.mark.parametrize("k,a_offset,tile", [(1001, 0, g.TILE_128x128), (1002, 0, g.TILE_256x128),
                                             (1004, 0, g.TILE_AUTO), (640, 1, g.TILE_128x256)])
def test_register_staged_loaders(k, a_offset, tile):
    rng = np.random.default_rng(k + a_offset)
    _check_nt(_eighths(rng, (300, k)), _eighths(rng, (520, k)), f"staged k {k} a+{a_offset} tile {tile}",
              tile=tile, a_offset=a_offset)


@pytest.mark.parametrize("variant", sorted(g.VARIANTS))
def test_variants(variant):
    bk = g.VARIANTS[variant][0]
    rng = np.random.default_rng(variant)
    _check_nt(_eighths(rng, (513, 5 * bk)), _eighths(rng, (260, 5 * bk)), f"variant {variant}",
              tile=g.TILE_128x128, variant=variant)


@pytest.mark.parametrize("m,n,k,tile", [(300, 520, 640, g.TILE_AUTO), (300, 520, 1000, g.TILE_128x128),
                                        (4608, 4096, 256, g.TILE_256x256), (300, 524, 1001, g.TILE_AUTO),
                                        (4608, 4096, 456, g.TILE_256x256), (2100, 2112, 136, g.TILE_128x128)])
def test_second_contract(m, n, k, tile):
    rng = np.random.default_rng(m * n + k)
    a, b = _eighths(rng, (m, k)), _eighths(rng, (k, n))
    print("case: nn", m, n, k, tile, flush=True)
    got = _run(a, b, nn=True, tile=tile)
    d64, _ = oracle.gemm_f16_nn_f64(a, b)
    bad = np.argwhere(got.astype(np.float64) != d64)
    assert bad.size == 0, f"nn {m}x{n}x{k}: {len(bad)} mismatches, first at {tuple(bad[0])}"
