"""Parity of the HIP GEMM against the CPU oracle, through the C ABI.

Bars (written here, from the method's arithmetic):
* {-8..8}/8 inputs and the closed forms: bit-exact.  Every partial sum of
  those inputs is a multiple of 1/64 far below 2^24, so fp32 accumulation is
  exact in any order and the one fp16 rounding (to nearest, ties to even)
  has a unique result; this is stricter than the 1e-3 relative gate of
  "wgmma_gemm.cu" (day 78), which is checked as well.
* N(0,1), N(0,0.5), uniform[-1,1] inputs: |C - C_oracle| <= 2 ulp_fp16(|C_oracle|)
  + 1e-2 sqrt(K) 2^-11 per element.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import dense_fp16_gemm_f16_amd as g  # noqa: E402
import oracle  # noqa: E402
from dense_fp16_gemm_f16_amd import inputs  # noqa: E402
from tests import pins  # noqa: E402

pytestmark = pytest.mark.gpu

GUARD = 64  # fp16 elements of sentinel on each side of C
SENTINEL = 0x7E5A  # a NaN pattern the kernel never produces


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    g.lib()
    yield
    torch.cuda.synchronize()


def _announce(*what):
    print("case:", *what, flush=True)


def run_gemm(a_np, b_np, a_offset=0, b_offset=0, **opts):
    """C from the HIP path; A/B may be placed `offset` elements past an aligned
    base to exercise the unaligned loader.  The elements around A and B are
    NaN, so a kernel that let one of them into a product would show it.  C
    sits between guard bands."""
    m, k = a_np.shape
    n = b_np.shape[0]
    dev = torch.device("cuda")
    a_buf = torch.full((a_offset + m * k + 8,), float("nan"), dtype=torch.float16, device=dev)
    b_buf = torch.full((b_offset + n * k + 8,), float("nan"), dtype=torch.float16, device=dev)
    if m * k:
        a_buf[a_offset:a_offset + m * k] = torch.from_numpy(a_np.reshape(-1)).to(dev)
    if n * k:
        b_buf[b_offset:b_offset + n * k] = torch.from_numpy(b_np.reshape(-1)).to(dev)
    c_buf = torch.full((GUARD + m * n + GUARD,), SENTINEL, dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream()
    rc = g.gemm_f16_nt_raw(m, n, k, a_buf.data_ptr() + 2 * a_offset, b_buf.data_ptr() + 2 * b_offset,
                           c_buf.data_ptr() + 2 * GUARD, stream.cuda_stream, **opts)
    assert rc == g.OK, g.status_string(rc)
    torch.cuda.synchronize()
    host = c_buf.cpu().numpy().view(np.uint16)
    assert np.all(host[:GUARD] == SENTINEL) and np.all(host[GUARD + m * n:] == SENTINEL), \
        "write outside C"
    return host[GUARD:GUARD + m * n].reshape(m, n).view(np.float16)


def assert_bits_equal(got, ref, what):
    gb, rb = got.view(np.uint16), ref.view(np.uint16)
    bad = np.argwhere(gb != rb)
    assert bad.size == 0, (f"{what}: {len(bad)} mismatches, first at {tuple(bad[0])}: "
                           f"gpu {got[tuple(bad[0])]} oracle {ref[tuple(bad[0])]}")


def assert_ulp(got, ref, k, what):
    ok, worst, idx = pins.check_ulp(got, ref, k)
    assert ok, f"{what}: worst |err|/tol = {worst:.3f} at {idx}: gpu {got[idx]} oracle {ref[idx]}"


TILES = sorted(g.TILES)


def normal_f16(rng, shape):
    """N(0,1) rounded to fp16, with magnitudes below 2^-10 pushed to 2^-10 so
    the bit-exact layout checks do not depend on fp16 subnormal handling."""
    x = rng.standard_normal(shape)
    x = np.where(np.abs(x) < 2.0**-10, np.copysign(2.0**-10, x), x)
    return x.astype(np.float16)


@pytest.mark.parametrize("tile", TILES)
def test_one_hot_rows_place_fragments(tile):
    """A[m, p(m)] = 1, else 0  =>  C[m, n] = B[n, p(m)] exactly: pins the MFMA
    operand and result layouts and the LDS swizzle for every tile shape."""
    _announce("one_hot", tile)
    rng = np.random.default_rng(20 + tile)
    m, n, k = 300, 270, 192
    p = rng.integers(0, k, size=m)
    a = np.zeros((m, k), dtype=np.float16)
    a[np.arange(m), p] = 1.0
    b = normal_f16(rng, (n, k))
    got = run_gemm(a, b, tile=tile)
    assert_bits_equal(got, b[:, p].T.copy(), "one-hot")


@pytest.mark.parametrize("tile", TILES)
def test_identity_and_all_ones(tile):
    _announce("identity/all-ones", tile)
    rng = np.random.default_rng(30 + tile)
    k = 256
    b = normal_f16(rng, (200, k))
    got = run_gemm(np.eye(k, dtype=np.float16), b, tile=tile)
    assert_bits_equal(got, b.T.copy(), "A = I")
    a = normal_f16(rng, (77, k))
    assert_bits_equal(run_gemm(a, np.eye(k, dtype=np.float16), tile=tile), a, "B = I")
    ones = run_gemm(np.ones((70, 1000), np.float16), np.ones((90, 1000), np.float16), tile=tile)
    assert np.all(ones == np.float16(1000))


@pytest.mark.parametrize("name", ["gemm_256_eighths", "gemm_5000x3000x1000_eighths"])
def test_eighths_workloads_bit_exact(name):
    _announce(name)
    a, b = inputs.workload_inputs(name)
    got = run_gemm(a, b)
    ref = oracle.gemm_f16_nt(a, b)
    assert_bits_equal(got, ref, name)
    assert_bits_equal(got, pins.eighths_exact_bits(a, b).view(np.float16), name + " (exact)")
    ok, worst, idx = pins.check_rel(got, ref, 1e-3)
    assert ok, f"rel {worst} at {idx}"


def test_4096_normal_full_oracle():
    _announce("gemm_4096_normal")
    a, b = inputs.workload_inputs("gemm_4096_normal")
    got = run_gemm(a, b)
    assert_ulp(got, oracle.gemm_f16_nt(a, b), 4096, "gemm_4096_normal")


@pytest.mark.parametrize("name", ["gemm_8192_uniform", "gemm_16384x4096x2048_normal05",
                                  "gemm_1024x8192x8192_uniform"])
def test_large_workloads_whole_c(name):
    """Full-size runs in the default launch configuration, every element of C
    against the oracle (about 15 s of oracle time for 8192^3 on 16 cores)."""
    _announce(name)
    w = inputs.WORKLOADS[name]
    a, b = inputs.workload_inputs(name)
    got = run_gemm(a, b)
    assert np.all(np.isfinite(got.astype(np.float32)))
    assert_ulp(got, oracle.gemm_f16_nt(a, b), w.k, name)


# Rows that are not 16-byte aligned at full size, on random operands: the
# register-staged loaders with 16-byte loads at 4-byte aligned offsets (K
# even) and shifted by 2 bytes (odd K, or A at an odd element offset).  Rows
# of C sampled across every 256-row block, checked element by element.
@pytest.mark.parametrize("m,n,k,a_off", [(4096, 4096, 4095, 0), (4096, 4096, 4094, 0), (4096, 4096, 4096, 1)])
def test_unaligned_rows_at_full_size(m, n, k, a_off):
    _announce("unaligned rows, full size", m, n, k, a_off)
    rng = np.random.default_rng(m + n + k + a_off)
    a = rng.uniform(-1, 1, size=(m, k)).astype(np.float16)
    b = rng.uniform(-1, 1, size=(n, k)).astype(np.float16)
    got = run_gemm(a, b, a_offset=a_off)
    rows = np.arange(m // 256) * 256 + rng.integers(0, 256, size=m // 256)
    ref = oracle.gemm_f16_nt_rows(a, b, rows)
    assert_ulp(got[rows], ref, k, f"{m}x{n}x{k} A offset {a_off} sampled rows")


# K % 64 != 0 and an odd K-tile count at full size, on random operands: the
# one-workgroup-per-CU kernels with a partial last K-tile (1000: 16 K-tiles,
# the last 40 k; 960: 15) and a K-tile of zeros added (960).  Rows of C
# sampled across every 256-row block, checked element by element.
@pytest.mark.parametrize("m,n,k", [(8192, 8192, 1000), (8192, 8192, 960), (16384, 4096, 2000)])
def test_partial_k_tiles_at_full_size(m, n, k):
    _announce("partial K, full size", m, n, k)
    rng = np.random.default_rng(m + n + k)
    a = rng.uniform(-1, 1, size=(m, k)).astype(np.float16)
    b = rng.uniform(-1, 1, size=(n, k)).astype(np.float16)
    got = run_gemm(a, b)
    rows = np.arange(m // 256) * 256 + rng.integers(0, 256, size=m // 256)
    ref = oracle.gemm_f16_nt_rows(a, b, rows)
    assert_ulp(got[rows], ref, k, f"{m}x{n}x{k} sampled rows")


RAGGED = [
    (1, 1, 1), (1, 1, 8), (7, 5, 3), (31, 33, 17), (33, 31, 64), (64, 64, 64), (65, 63, 72),
    (129, 200, 136), (255, 257, 1000), (257, 255, 520), (300, 70, 7), (513, 130, 65),
]


@pytest.mark.parametrize("m,n,k", RAGGED)
@pytest.mark.parametrize("tile", TILES)
def test_ragged_shapes(m, n, k, tile):
    _announce("ragged", m, n, k, tile)
    rng = np.random.default_rng(m * 7 + n * 13 + k)
    a = rng.standard_normal((m, k)).astype(np.float16)
    b = rng.standard_normal((n, k)).astype(np.float16)
    assert_ulp(run_gemm(a, b, tile=tile), oracle.gemm_f16_nt(a, b), k, f"{m}x{n}x{k}")


# K and operand offsets (in elements) chosen so each row alignment of the
# register-staged loader runs: 4-byte aligned rows (K even, operands 4-byte
# aligned), whose 16-byte loads start at 4-byte aligned offsets, and 2-byte
# aligned rows (odd K: every other row; an operand at an odd element offset:
# every row), whose loads are shifted by 2 bytes.  Chunks straddle K in the
# last K-tile, and below one K-tile.
GRANULARITY = [
    (100, 0, 0), (132, 0, 0), (2500, 0, 0), (4, 0, 0),  # K % 8 == 4
    (98, 0, 0), (130, 0, 0), (6, 0, 0), (1026, 0, 0),   # K % 8 == 2 or 6
    (96, 4, 0), (96, 0, 4),                             # K % 8 == 0, an operand 8-byte aligned
    (96, 2, 0), (64, 0, 6),                             # ... an operand 4-byte aligned
    (99, 0, 0), (1, 0, 0), (7, 0, 0), (63, 0, 0),       # odd K
    (65, 0, 0), (129, 0, 0), (1001, 0, 0),
    (96, 1, 0), (64, 0, 3), (98, 1, 1),                 # even K, an operand at an odd offset
    (99, 1, 0), (101, 0, 5), (127, 3, 7),               # odd K and odd offsets
]


@pytest.mark.parametrize("k,a_off,b_off", GRANULARITY)
@pytest.mark.parametrize("tile", TILES)
def test_load_widths_bit_exact(k, a_off, b_off, tile):
    _announce("load widths", k, a_off, b_off, tile)
    rng = np.random.default_rng(k * 31 + a_off * 7 + b_off)
    m, n = 150, 140
    a = (rng.integers(-8, 9, size=(m, k)) / 8).astype(np.float16)
    b = (rng.integers(-8, 9, size=(n, k)) / 8).astype(np.float16)
    got = run_gemm(a, b, a_offset=a_off, b_offset=b_off, tile=tile)
    assert_bits_equal(got, oracle.gemm_f16_nt(a, b), f"K={k} offsets {a_off},{b_off} tile {tile}")


# K % 8 == 0 with 16-byte aligned rows: the loads go straight into LDS.  1,
# 2, 3, 5 and 15 full K-tiles (odd counts end on the first stage), partial
# last K-tiles (K % 64 = 8, 40, 56: chunks past K read as zeros), K below one
# K-tile, rows and columns past M and N inside the last block tile.
DIRECT = [(1, 1, 64), (257, 129, 64), (64, 64, 128), (300, 270, 192), (33, 300, 320), (130, 515, 960),
          (1, 1, 8), (70, 90, 40), (300, 270, 200), (257, 129, 1000), (65, 63, 504), (129, 257, 72)]


@pytest.mark.parametrize("m,n,k", DIRECT)
@pytest.mark.parametrize("tile", TILES)
def test_direct_to_lds_path_bit_exact(m, n, k, tile):
    _announce("direct", m, n, k, tile)
    rng = np.random.default_rng(m + 3 * n + 5 * k + tile)
    a = (rng.integers(-8, 9, size=(m, k)) / 8).astype(np.float16)
    b = (rng.integers(-8, 9, size=(n, k)) / 8).astype(np.float16)
    assert_bits_equal(run_gemm(a, b, tile=tile), oracle.gemm_f16_nt(a, b), f"{m}x{n}x{k}")


# More block tiles than CUs, K a multiple of the K-tile with
# an even count of at least 4, 16-byte aligned C with N % 8 == 0: one
# workgroup per CU walks several tiles and the K-tile stream runs across the
# tile changes; on every block tile but 64x64 each tile's C leaves under the
# next tile's first MFMAs, in 16-byte stores straight from the accumulators.  Ragged last tiles in M and
# N; 1 to 5 tiles per workgroup; 4 to 10 K-tiles.  These problems fit in the
# Infinity Cache, so C's stores are device-scope; the store policies of larger
# problems are covered by test_store_policies_past_the_infinity_cache.
PERSISTENT = [(g.TILE_64x64, 1100, 1064, 256), (g.TILE_64x64, 2100, 2104, 256),
              (g.TILE_128x128, 2100, 2088, 384), (g.TILE_256x256, 4200, 4152, 512),
              (g.TILE_256x128, 4200, 2088, 256), (g.TILE_128x256, 2100, 4152, 256),
              (g.TILE_256x256, 4200, 4096, 512), (g.TILE_128x128, 2100, 2112, 256),
              (g.TILE_256x256, 8200, 2056, 384), (g.TILE_256x128, 4100, 4104, 640),
              (g.TILE_64x128, 1100, 2104, 256), (g.TILE_128x64, 2100, 1064, 384),
              # K % 64 != 0: every tile's last K-tile is partial (8, 8, 40 and
              # 56 of its 64 k), its chunks past K read as zeros
              (g.TILE_128x128, 2100, 2088, 200), (g.TILE_256x256, 4200, 4152, 456),
              (g.TILE_256x128, 4200, 2088, 1000), (g.TILE_128x256, 2100, 4152, 248),
              # an odd K-tile count (15 whole, 3 with a partial last one): the
              # kernel adds a K-tile of zeros
              (g.TILE_256x128, 4200, 2088, 960), (g.TILE_128x128, 2100, 2088, 136),
              # the same on the persistent kernel's tiles
              (g.TILE_64x64, 1100, 1064, 200), (g.TILE_64x128, 1100, 2104, 136),
              (g.TILE_128x64, 2100, 1064, 960)]


@pytest.mark.parametrize("tile,m,n,k", PERSISTENT)
def test_persistent_path_bit_exact(tile, m, n, k):
    _announce("persistent", tile, m, n, k)
    rng = np.random.default_rng(m + n + k + tile)
    a = (rng.integers(-8, 9, size=(m, k)) / 8).astype(np.float16)
    b = (rng.integers(-8, 9, size=(n, k)) / 8).astype(np.float16)
    assert_bits_equal(run_gemm(a, b, tile=tile), oracle.gemm_f16_nt(a, b), f"{m}x{n}x{k}")


# The C store policies that apply only past the 256 MiB Infinity Cache (A,
# B and C together larger): non-temporal stores on rows of whole 128-byte
# lines, the default policy on rows that end inside a line, on the one-tile,
# stream and one-workgroup-per-CU (64x64) kernels.  One-hot rows of A
# (A[m, p(m)] = 1) make C[m, n] = B[n, p(m)] exactly (+0 where that is -0),
# so the check is a gather at any size.
PAST_THE_CACHE = [
    (4096, 4096, 16384, g.TILE_AUTO, "one tile per workgroup, whole-line rows"),
    (4096, 4088, 16384, g.TILE_AUTO, "one tile per workgroup, rows ending inside a line"),
    (16384, 8200, 2048, g.TILE_AUTO, "stream kernel, rows ending inside a line"),
    (16384, 8192, 2048, g.TILE_64x64, "one workgroup per CU on 64x64, whole-line rows"),
    (16384, 8200, 2048, g.TILE_64x64, "one workgroup per CU on 64x64, rows ending inside a line"),
]


@pytest.mark.parametrize("m,n,k,tile,what", PAST_THE_CACHE)
def test_store_policies_past_the_infinity_cache(m, n, k, tile, what):
    _announce("store policy", what, m, n, k, tile)
    assert (m * k + n * k) * 2 + m * n * 2 > 256 << 20
    rng = np.random.default_rng(m + n + k)
    p = (np.arange(m, dtype=np.int64) * 7 + 3) % k
    a = np.zeros((m, k), np.float16)
    a[np.arange(m), p] = 1
    b = rng.standard_normal((n, k)).astype(np.float16)
    got = run_gemm(a, b, tile=tile)
    # C is a sum that starts at +0: where B holds -0, +0 + (-0) = +0
    ref = (b[:, p].T.astype(np.float32) + np.float32(0)).astype(np.float16)
    assert_bits_equal(got, np.ascontiguousarray(ref), what)


# The largest K the library takes (K < 2^22): a 64x64 output, so the oracle
# stays cheap, on the direct path (K % 64 == 0, the automatic 64x64 tile and
# the 256x256 tile, whose operand ranges are then 256 rows x K x 2 bytes, just
# below 2^31) and on the element loader (K odd).  Entries from {-1, 0, 1}:
# every partial sum is an integer of magnitude below 2^22 < 2^24, exact in
# fp32 in any order, so the one fp16 rounding is unique and the bar is
# bit-exact.
MAX_K = [((1 << 22) - 64, g.TILE_AUTO), ((1 << 22) - 64, g.TILE_256x256), ((1 << 22) - 1, g.TILE_AUTO)]


@pytest.mark.parametrize("k,tile", MAX_K)
def test_largest_k_bit_exact(k, tile):
    _announce("max-k", k, tile)
    rng = np.random.default_rng(k + tile)
    a = rng.integers(-1, 2, size=(64, k), dtype=np.int8).astype(np.float16)
    b = rng.integers(-1, 2, size=(64, k), dtype=np.int8).astype(np.float16)
    assert_bits_equal(run_gemm(a, b, tile=tile), oracle.gemm_f16_nt(a, b), f"64x64x{k}")


# C rows of nearly 2^22 columns: with N = 2^22 - 8 a 256-row block of C still
# spans less than 2^31 bytes and the one-workgroup-per-CU kernel takes the
# shape (32768 tiles); with N = 2^22 it does not, and the one-tile-per-workgroup
# kernel does.  A has one 1 per row, at column p(m), so C[m][n] = B[n][p(m)]
# exactly (one non-zero product, exact in fp32, and an fp16 value needs no
# rounding): the check runs on the GPU over all of C, with guard bands.
@pytest.mark.parametrize("n", [(1 << 22) - 8, 1 << 22])
def test_widest_rows_one_hot(n):
    _announce("wide-n", n)
    m, k = 512, 256
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(n)
    b = torch.randn((n, k), generator=gen, device=dev).to(torch.float16)
    tiny = b.abs() < 2.0**-10  # keep clear of fp16 subnormals, as normal_f16 does
    b = torch.where(tiny, torch.copysign(torch.full_like(b, 2.0**-10), b), b)
    p = (torch.arange(m, device=dev) * 37 + 11) % k
    a = torch.zeros((m, k), dtype=torch.float16, device=dev)
    a[torch.arange(m, device=dev), p] = 1.0
    c_buf = torch.full((GUARD + m * n + GUARD,), SENTINEL, dtype=torch.int16, device=dev)
    rc = g.gemm_f16_nt_raw(m, n, k, a.data_ptr(), b.data_ptr(), c_buf.data_ptr() + 2 * GUARD,
                           torch.cuda.current_stream().cuda_stream)
    assert rc == g.OK, g.status_string(rc)
    torch.cuda.synchronize()
    assert bool((c_buf[:GUARD] == SENTINEL).all()) and bool((c_buf[GUARD + m * n:] == SENTINEL).all()), \
        "write outside C"
    c = c_buf[GUARD:GUARD + m * n].view(m, n)
    expect = b[:, p].t().contiguous().view(torch.int16)
    bad = int((c != expect).sum())
    assert bad == 0, f"{m}x{n}x{k} one-hot: {bad} mismatches"


# The epilogue's cast at the top of the fp16 range: a sum of 65520 or more
# rounds to infinity (65520 is the midpoint between the largest finite value,
# 65504, and 2^16, and ties go to the even neighbour, 2^16), 65519 rounds
# down to 65504.  Every sum here is an integer below 2^24, exact in fp32 in
# any order, so the rounded result is unique and the bar is bit-exact.
@pytest.mark.parametrize("tile", TILES)
def test_epilogue_overflow_bit_exact(tile):
    _announce("overflow", tile)
    rng = np.random.default_rng(65520 + tile)
    m, n, k = 70, 90, 40
    a = np.zeros((m, k), np.float64)
    b = np.zeros((n, k), np.float64)
    a[:, 0], a[:, 1] = 256.0, 1.0
    b[:, 0] = 255.875  # 256 * 255.875 = 65504, the largest finite fp16
    b[:, 1] = rng.integers(-20, 21, size=n)  # 65504 + t for t in [-20, 20]
    sign = np.where(rng.random(m) < 0.5, -1.0, 1.0)
    a[:, 0] *= sign
    a[:, 1] *= sign
    a[:, 2] = rng.integers(0, 3, size=m)  # plus 0, 64 or 128 more on some rows
    b[:, 2] = 64.0
    a, b = a.astype(np.float16), b.astype(np.float16)
    ref = oracle.gemm_f16_nt(a, b)
    assert np.isinf(ref.astype(np.float32)).any() and (np.abs(ref.astype(np.float32)) == 65504).any()
    assert_bits_equal(run_gemm(a, b, tile=tile), ref, f"overflow tile {tile}")


# Non-finite operands: +-inf times a non-zero value gives +-inf, inf times 0
# and inf - inf give NaN, and NaN propagates.  NaN payloads and signs are not
# fixed by the arithmetic, so NaN is compared as a class; every other
# element bit for bit.
@pytest.mark.parametrize("tile", TILES)
def test_non_finite_operands(tile):
    _announce("non-finite", tile)
    rng = np.random.default_rng(7 + tile)
    m, n, k = 66, 72, 24
    a = (rng.integers(-8, 9, size=(m, k)) / 8).astype(np.float16)
    b = (rng.integers(-8, 9, size=(n, k)) / 8).astype(np.float16)
    b[:, 0] = np.where(rng.random(n) < 0.2, 0.0, b[:, 0])
    a[0, 0] = np.inf
    a[1, 0] = -np.inf
    a[2, 0], a[2, 1] = np.inf, -np.inf
    a[3, 5] = np.nan
    b[4, 7] = np.inf
    ref = oracle.gemm_f16_nt(a, b)
    got = run_gemm(a, b, tile=tile)
    rn, gn = np.isnan(ref.astype(np.float32)), np.isnan(got.astype(np.float32))
    assert rn.any() and np.isinf(ref.astype(np.float32)).any()
    bad = np.argwhere(rn != gn)
    assert bad.size == 0, f"NaN pattern differs at {tuple(bad[0])}: gpu {got[tuple(bad[0])]} oracle {ref[tuple(bad[0])]}"
    keep = ~rn
    assert np.array_equal(got.view(np.uint16)[keep], ref.view(np.uint16)[keep]), "finite/inf elements differ"


def test_concurrent_host_threads():
    """Eight host threads call the C ABI at once (ctypes releases the GIL for
    the call), each on its own stream, from a fresh start of nothing: every
    result must match the oracle bit for bit."""
    import threading

    _announce("threads")
    rng = np.random.default_rng(31)
    m, n, k = 300, 270, 200
    a = (rng.integers(-8, 9, size=(m, k)) / 8).astype(np.float16)
    b = (rng.integers(-8, 9, size=(n, k)) / 8).astype(np.float16)
    ref = oracle.gemm_f16_nt(a, b)
    dev = torch.device("cuda")
    a_d, b_d = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    outs = [torch.empty((m, n), dtype=torch.float16, device=dev) for _ in range(8)]
    streams = [torch.cuda.Stream() for _ in range(8)]  # default priority
    codes = [None] * 8
    torch.cuda.synchronize()

    def work(i):
        rc = g.OK
        for _ in range(5):
            rc = rc or g.gemm_f16_nt_raw(m, n, k, a_d.data_ptr(), b_d.data_ptr(), outs[i].data_ptr(),
                                         streams[i].cuda_stream, tile=1 + i % 7)
        codes[i] = rc

    threads = [threading.Thread(target=work, args=(i,)) for i in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert codes == [g.OK] * 8, codes
    for i, o in enumerate(outs):
        assert_bits_equal(o.cpu().numpy(), ref, f"thread {i}")


def test_hip_graph_capture_and_replay():
    """The library allocates nothing and sets no memory, so its launches can
    be captured in a HIP graph: one capture of a GEMM per block tile, K = 0
    included, replayed several times with eager work and synchronisations in
    between; every replay must match the oracle bit for bit."""
    _announce("graph")
    rng = np.random.default_rng(41)
    m, n, k = 300, 270, 200
    a = (rng.integers(-8, 9, size=(m, k)) / 8).astype(np.float16)
    b = (rng.integers(-8, 9, size=(n, k)) / 8).astype(np.float16)
    ref = oracle.gemm_f16_nt(a, b)
    dev = torch.device("cuda")
    a_d, b_d = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
    outs = [torch.empty((m, n), dtype=torch.float16, device=dev) for _ in TILES]
    zero_out = torch.empty((m, n), dtype=torch.float16, device=dev)
    # warm the library's per-device caches outside the capture
    g.gemm_f16_nt(a_d, b_d, out=outs[0])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            cap = torch.cuda.current_stream()
            for t, o in zip(TILES, outs):
                rc = g.gemm_f16_nt_raw(m, n, k, a_d.data_ptr(), b_d.data_ptr(), o.data_ptr(), cap.cuda_stream,
                                       tile=t)
                assert rc == g.OK, g.status_string(rc)
            rc = g.gemm_f16_nt_raw(m, n, 0, a_d.data_ptr(), b_d.data_ptr(), zero_out.data_ptr(), cap.cuda_stream)
            assert rc == g.OK, g.status_string(rc)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.view(torch.int16).fill_(SENTINEL)  # eager work between replays
        zero_out.view(torch.int16).fill_(SENTINEL)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, o in zip(TILES, outs):
            assert_bits_equal(o.cpu().numpy(), ref, f"replay {rep} tile {t}")
        assert bool((zero_out.view(torch.int16) == 0).all()), f"replay {rep}: K = 0 output not zero"
        # eager calls between replays
        g.gemm_f16_nt(a_d, b_d, out=outs[0])
        torch.cuda.synchronize()


@pytest.mark.parametrize("a_off,b_off", [(1, 0), (0, 3), (5, 7)])
def test_unaligned_operands_take_the_register_staged_loader(a_off, b_off):
    _announce("unaligned", a_off, b_off)
    rng = np.random.default_rng(a_off * 10 + b_off)
    m, n, k = 150, 140, 96
    a = (rng.integers(-8, 9, size=(m, k)) / 8).astype(np.float16)
    b = (rng.integers(-8, 9, size=(n, k)) / 8).astype(np.float16)
    got = run_gemm(a, b, a_offset=a_off, b_offset=b_off)
    assert_bits_equal(got, oracle.gemm_f16_nt(a, b), "unaligned")


def test_k_zero_writes_zeros_and_empty_is_a_no_op():
    _announce("degenerate")
    got = run_gemm(np.zeros((37, 0), np.float16), np.zeros((45, 0), np.float16))
    assert np.all(got.view(np.uint16) == 0)
    assert run_gemm(np.zeros((0, 16), np.float16), np.ones((9, 16), np.float16)).shape == (0, 9)
    assert run_gemm(np.ones((9, 16), np.float16), np.zeros((0, 16), np.float16)).shape == (9, 0)


@pytest.mark.parametrize("tile", TILES)
def test_a_sum_of_zeros_is_positive_zero(tile):
    """Every product -0 (one-hot A against -0, and zeros against negative
    numbers): C is +0, since the fp32 sum starts at +0 and +0 + (-0) = +0."""
    _announce("signed zero", tile)
    m, n, k = 70, 40, 128
    a = np.zeros((m, k), np.float16)
    a[:, 0] = 1
    b = -np.abs(np.random.default_rng(7).standard_normal((n, k))).astype(np.float16)
    b[:, 0] = -0.0
    got = run_gemm(a, b, tile=tile)
    assert np.all(got.view(np.uint16) == 0), "C must be +0"
    assert_bits_equal(got, oracle.gemm_f16_nt(a, b), "signed zero")


# more tiles than CUs: one workgroup per CU walks tiles; an odd K-tile count
# (3, 15) has a K-tile of zeros added, and K % 64 != 0 a partial last one
@pytest.mark.parametrize("tile,m,n,k", [(g.TILE_128x128, 2100, 2088, 136), (g.TILE_256x256, 4200, 4152, 960),
                                        (g.TILE_256x128, 4200, 2088, 1000)])
def test_a_sum_of_zeros_is_positive_zero_on_the_stream_kernel(tile, m, n, k):
    """The same sum of -0 products over several tiles per CU: C stays +0."""
    _announce("signed zero, stream", tile, m, n, k)
    a = np.zeros((m, k), np.float16)
    a[:, 0] = 1
    b = -np.abs(np.random.default_rng(k).standard_normal((n, k))).astype(np.float16)
    b[:, 0] = -0.0
    got = run_gemm(a, b, tile=tile)
    assert np.all(got.view(np.uint16) == 0), "C must be +0"


def test_schedule_options_do_not_change_bits():
    """Rasterization only reorders tiles; each output's sum order is fixed."""
    _announce("determinism")
    rng = np.random.default_rng(99)
    a = rng.standard_normal((2048, 640)).astype(np.float16)
    b = rng.standard_normal((1536, 640)).astype(np.float16)
    base = run_gemm(a, b, tile=g.TILE_256x256)
    for sw, xcd in [(1, 0), (1, 1), (3, 1), (8, 0), (64, 1)]:
        assert_bits_equal(run_gemm(a, b, tile=g.TILE_256x256, swizzle=sw, xcd=xcd), base, f"{sw},{xcd}")
    assert_bits_equal(run_gemm(a, b, tile=g.TILE_256x256), base, "repeat")


def test_default_rasterization_on_a_grid_of_one_tile_per_cu():
    """4096^2 on 256x256 tiles is a 16x16 grid: on a 256-CU device the
    default keeps the dispatch order there (no XCD gets more operand panels).
    Exact operands: bit-exact against the oracle, and the same bits with
    either explicit setting."""
    _announce("default rasterization, 16x16 grid")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert g.select_xcd(16, 16, 4, cus) == (0 if cus == 256 else 1)
    rng = np.random.default_rng(256)
    a = (rng.integers(-8, 9, size=(4096, 256)) / 8).astype(np.float16)
    b = (rng.integers(-8, 9, size=(4096, 256)) / 8).astype(np.float16)
    base = run_gemm(a, b, tile=g.TILE_256x256)
    assert_bits_equal(base, oracle.gemm_f16_nt(a, b), "default vs oracle")
    for xcd in (0, 1):
        assert_bits_equal(run_gemm(a, b, tile=g.TILE_256x256, xcd=xcd), base, f"xcd {xcd}")


def test_torch_wrapper_on_a_side_stream():
    _announce("stream")
    rng = np.random.default_rng(5)
    a = rng.standard_normal((384, 320)).astype(np.float16)
    b = rng.standard_normal((448, 320)).astype(np.float16)
    ta = torch.from_numpy(a).cuda()
    tb = torch.from_numpy(b).cuda()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        c = g.gemm_f16_nt(ta, tb)
    s.synchronize()
    assert_ulp(c.cpu().numpy(), oracle.gemm_f16_nt(a, b), 320, "side stream")


def test_overlap_and_null_are_refused_on_device():
    _announce("errors")
    x = torch.zeros(64 * 64, dtype=torch.float16, device="cuda")
    assert g.gemm_f16_nt_raw(64, 64, 64, x.data_ptr(), x.data_ptr(), x.data_ptr()) == g.EOVERLAP
    assert g.gemm_f16_nt_raw(64, 64, 64, 0, x.data_ptr(), x.data_ptr()) == g.ENULL


# The tuning variants (options.variant): block_k 32 / 64, 2 to 4 LDS stages,
# and 4 loader waves beside the 4 MFMA waves, on every tile they fit.  One
# tile per workgroup; the K-tile count is padded with all-zero K-tiles to a
# whole unrolled block (K = one K-tile up to well past it, ragged M and N).
VARIANT_TILES = {g.TILE_256x256: (1, 3, 4, 5), g.TILE_256x128: (1, 2, 3, 4, 5, 6),
                 g.TILE_128x256: (1, 2, 3, 4, 5, 6), g.TILE_128x128: (1, 2, 3, 4, 5, 6, 7)}
VARIANT_CASES = [(tile, v) for tile, vs in VARIANT_TILES.items() for v in vs]


@pytest.mark.parametrize("tile,variant", VARIANT_CASES)
def test_variants_bit_exact(tile, variant):
    bk = g.VARIANTS[variant][0]
    rng = np.random.default_rng(tile * 10 + variant)
    for m, n, k in [(300, 520, bk), (513, 260, 5 * bk), (700, 900, 13 * bk)]:
        _announce("variant", tile, variant, m, n, k)
        a = (rng.integers(-8, 9, size=(m, k)) / 8).astype(np.float16)
        b = (rng.integers(-8, 9, size=(n, k)) / 8).astype(np.float16)
        assert_bits_equal(run_gemm(a, b, tile=tile, variant=variant), oracle.gemm_f16_nt(a, b),
                          f"variant {variant} tile {tile} {m}x{n}x{k}")


# Race check.  Every 4-wave tile's direct-to-LDS kernels, the
# one-workgroup-per-CU kernels and every kernel variant run
# v_mfma_f32_16x16x32_f16 over K in 32-wide k steps in increasing order, so
# each output's fp32 sum is formed in the same order whatever the kernel,
# tile, ring depth or loader arrangement: on random operands their C must
# agree bit for bit.  A race (a stale or early LDS read, a stage reused too
# soon) shows up as a difference.  Shapes: one tile per workgroup (and the
# K tail), the stream kernel (more 256x256 tiles than CUs) and the
# persistent one (64x64, 64x128, 128x64 tiles).
M16_DIRECT_TILES = [g.TILE_256x256, g.TILE_256x128, g.TILE_128x256, g.TILE_128x128, g.TILE_128x128_M16,
                    g.TILE_64x64, g.TILE_64x128, g.TILE_128x64]


@pytest.mark.parametrize("m,n,k", [(1000, 1100, 640), (1000, 1100, 1000), (4608, 4096, 256), (2100, 2112, 1024)])
def test_same_bits_across_kernels(m, n, k):
    _announce("same bits", m, n, k)
    rng = np.random.default_rng(m * 7 + n * 3 + k)
    a = rng.standard_normal((m, k)).astype(np.float16)
    b = rng.standard_normal((n, k)).astype(np.float16)
    base = run_gemm(a, b, tile=g.TILE_256x256)
    assert_ulp(base, oracle.gemm_f16_nt(a, b), k, f"{m}x{n}x{k} 256x256")
    for tile in M16_DIRECT_TILES:
        assert_bits_equal(run_gemm(a, b, tile=tile), base, f"{m}x{n}x{k} tile {tile}")
    for tile, variants in VARIANT_TILES.items():
        for v in variants:
            if k % g.VARIANTS[v][0] == 0:
                assert_bits_equal(run_gemm(a, b, tile=tile, variant=v), base, f"{m}x{n}x{k} tile {tile} variant {v}")


@pytest.mark.parametrize("variant", [1, 4, 6])
def test_variants_random_operands(variant):
    """uniform[-1,1] operands, 1024x1024x2048 on the 128x128 tile: ulp bar."""
    _announce("variant random", variant)
    rng = np.random.default_rng(variant)
    a = rng.uniform(-1, 1, (1024, 2048)).astype(np.float16)
    b = rng.uniform(-1, 1, (1024, 2048)).astype(np.float16)
    assert_ulp(run_gemm(a, b, tile=g.TILE_128x128, variant=variant), oracle.gemm_f16_nt(a, b), 2048,
               f"variant {variant}")
