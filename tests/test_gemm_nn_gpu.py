"""Parity of the second contract, D fp32 = A * B with B [K,N] (the day-78
listing "wgmma_gemm.cu"), against its CPU reference, through the C ABI.

Bars (written here, from the arithmetic):
* {-8..8}/8 inputs, identity, one-hot: bit-exact.  Every partial sum is a
  multiple of 1/64 below 2^24, so any fp32 summation order gives the exact
  sum, which fp32 D holds exactly.  The listing's own gate, |gpu - ref| /
  max(|ref|, 1) <= 1e-3, is checked as well.
* random inputs: |D - D_ref| <= 2 * gamma_K * sum_k |A[m,k] B[k,n]| with
  gamma_K = K u / (1 - K u), u = 2^-24: the classical bound on the error of
  any order of K fp32 additions (doubled to cover an MFMA that rounds its
  partial sums less carefully than round-to-nearest), with the sum of
  |products| from the oracle.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import dense_fp16_gemm_f16_amd as g  # noqa: E402
import oracle  # noqa: E402
from dense_fp16_gemm_f16_amd import inputs  # noqa: E402
from tests import pins  # noqa: E402

pytestmark = pytest.mark.gpu

GUARD = 32  # fp32 elements of sentinel on each side of D
SENTINEL = np.float32(-12345.5)
NN_TILES = [t for t in sorted(g.TILES) if t not in g.M16_TILES]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    g.lib()
    yield
    torch.cuda.synchronize()


def _announce(*what):
    print("case:", *what, flush=True)


def run_nn(a_np, b_np, a_offset=0, b_offset=0, **opts):
    m, k = a_np.shape
    kb, n = b_np.shape
    assert kb == k
    dev = torch.device("cuda")
    # NaN around A and B: an element outside them in a product would show
    a_buf = torch.full((a_offset + m * k + 8,), float("nan"), dtype=torch.float16, device=dev)
    b_buf = torch.full((b_offset + k * n + 8,), float("nan"), dtype=torch.float16, device=dev)
    if m * k:
        a_buf[a_offset:a_offset + m * k] = torch.from_numpy(a_np.reshape(-1)).to(dev)
    if k * n:
        b_buf[b_offset:b_offset + k * n] = torch.from_numpy(b_np.reshape(-1)).to(dev)
    d_buf = torch.full((GUARD + m * n + GUARD,), float(SENTINEL), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    rc = g.gemm_f16_nn_f32_raw(m, n, k, a_buf.data_ptr() + 2 * a_offset, b_buf.data_ptr() + 2 * b_offset,
                               d_buf.data_ptr() + 4 * GUARD, stream.cuda_stream, **opts)
    assert rc == g.OK, g.status_string(rc)
    torch.cuda.synchronize()
    host = d_buf.cpu().numpy()
    assert np.all(host[:GUARD] == SENTINEL) and np.all(host[GUARD + m * n:] == SENTINEL), "write outside D"
    return host[GUARD:GUARD + m * n].reshape(m, n)


def assert_exact(got, ref64, what):
    bad = np.argwhere(got.astype(np.float64) != ref64)
    assert bad.size == 0, (f"{what}: {len(bad)} mismatches, first at {tuple(bad[0])}: "
                           f"gpu {got[tuple(bad[0])]} ref {ref64[tuple(bad[0])]}")


def assert_fp32_bound(got, ref64, dabs, k, what):
    u = 2.0 ** -24
    gamma = k * u / (1 - k * u)
    err = np.abs(got.astype(np.float64) - ref64)
    tol = 2.0 * gamma * dabs + 1e-30
    ratio = err / tol
    idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    assert np.all(err <= tol), f"{what}: worst err/bound {ratio[idx]:.3f} at {idx}"
    ok, worst, widx = pins.check_rel(got, ref64, 1e-3)
    assert ok, f"{what}: day-78 gate rel {worst} at {widx}"


@pytest.mark.parametrize("name", ["gemm_nn_256_eighths", "gemm_nn_5000x3000x1000_eighths"])
def test_day78_workloads_exact(name):
    _announce(name)
    a, b = inputs.workload_inputs(name)
    got = run_nn(a, b)
    d64, _ = oracle.gemm_f16_nn_f64(a, b)
    assert_exact(got, d64, name)
    ok, worst, idx = pins.check_rel(got, d64, 1e-3)
    assert ok, f"rel {worst} at {idx}"


@pytest.mark.parametrize("tile", NN_TILES)
def test_identity_and_one_hot(tile):
    """A = I => D = B; one-hot rows of A select rows of B: pins the transposed
    B fragment reads and the fp32 result layout for every tile."""
    _announce("nn identity/one-hot", tile)
    rng = np.random.default_rng(60 + tile)
    k, n = 192, 264
    b = rng.standard_normal((k, n)).astype(np.float16)
    assert_exact(run_nn(np.eye(k, dtype=np.float16), b, tile=tile), b.astype(np.float64), "A = I")
    m = 300
    p = rng.integers(0, k, size=m)
    a = np.zeros((m, k), dtype=np.float16)
    a[np.arange(m), p] = 1.0
    assert_exact(run_nn(a, b, tile=tile), b[p].astype(np.float64), "one-hot")


RAGGED = [(1, 8, 8), (7, 16, 3), (31, 40, 17), (65, 72, 64), (129, 200, 136), (255, 264, 1000),
          (300, 72, 7), (513, 136, 65)]


@pytest.mark.parametrize("m,n,k", RAGGED)
@pytest.mark.parametrize("tile", NN_TILES)
def test_ragged_shapes(m, n, k, tile):
    _announce("nn ragged", m, n, k, tile)
    rng = np.random.default_rng(m * 3 + n * 5 + k)
    a = rng.standard_normal((m, k)).astype(np.float16)
    b = rng.standard_normal((k, n)).astype(np.float16)
    d64, dabs = oracle.gemm_f16_nn_f64(a, b)
    assert_fp32_bound(run_nn(a, b, tile=tile), d64, dabs, k, f"{m}x{n}x{k}")


# K and N multiples of 8 on the 16x16x32 tiles: B [K,N] goes straight into
# LDS by k-rows and is read back transposed.  Odd and even K-tile counts, a
# last K-tile of 8..56 k, N ragged by 8 past a tile, a single 8-wide column
# chunk, several tiles in both directions.
NN_DIRECT = [(1, 8, 8), (64, 128, 64), (300, 264, 200), (129, 520, 72), (513, 1032, 520), (257, 392, 1000),
             (70, 136, 8), (1000, 776, 1088)]
NN_DIRECT_TILES = [t for t in NN_TILES if t not in (g.TILE_256x256_W8, g.TILE_64x64, g.TILE_128x64)]


@pytest.mark.parametrize("m,n,k", NN_DIRECT)
@pytest.mark.parametrize("tile", NN_DIRECT_TILES)
def test_direct_to_lds_b_path_bit_exact(m, n, k, tile):
    _announce("nn direct", m, n, k, tile)
    rng = np.random.default_rng(m * 7 + n * 11 + k + tile)
    a = (rng.integers(-8, 9, size=(m, k)) / 8).astype(np.float16)
    b = (rng.integers(-8, 9, size=(k, n)) / 8).astype(np.float16)
    d64, _ = oracle.gemm_f16_nn_f64(a, b)
    assert_exact(run_nn(a, b, tile=tile), d64, f"{m}x{n}x{k}")


# More tiles than CUs, K a multiple of 64 with an even K-tile count >= 4:
# one workgroup per CU walking tiles, the next tile's K-tiles 0 and 1 loaded
# under the current one's last two, D staged in eighths of a wave's piece.
# Ragged M and N (by 8..64 past a tile) on every 16x16x32 tile; N % 32 == 0
# (fp32 rows of whole 128-byte lines) takes the non-temporal stores.
NN_PERSISTENT = [(g.TILE_128x128, 2100, 2088, 384), (g.TILE_256x256, 4200, 4152, 512),
                 (g.TILE_256x128, 4200, 2088, 256), (g.TILE_128x256, 2100, 4152, 256),
                 (g.TILE_256x256, 4200, 4128, 256), (g.TILE_128x256, 2100, 4160, 256),
                 (g.TILE_64x128, 1100, 2104, 256),
                 # K % 64 != 0 (a partial last K-tile) and odd K-tile counts
                 # (a K-tile of zeros added)
                 (g.TILE_128x128, 2100, 2088, 200), (g.TILE_256x128, 4200, 2088, 1000),
                 (g.TILE_128x256, 2100, 4152, 248), (g.TILE_256x128, 4200, 2088, 960),
                 (g.TILE_64x128, 1100, 2104, 136)]


@pytest.mark.parametrize("tile,m,n,k", NN_PERSISTENT)
def test_persistent_path_bit_exact(tile, m, n, k):
    _announce("nn persistent", tile, m, n, k)
    rng = np.random.default_rng(m + n + k + tile)
    a = (rng.integers(-8, 9, size=(m, k)) / 8).astype(np.float16)
    b = (rng.integers(-8, 9, size=(k, n)) / 8).astype(np.float16)
    d64, _ = oracle.gemm_f16_nn_f64(a, b)
    assert_exact(run_nn(a, b, tile=tile), d64, f"{m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(70, 13, 40), (33, 100, 24), (64, 21, 19), (150, 140, 99), (130, 70, 129),
                                   (300, 40, 1001)])
def test_n_or_k_not_multiple_of_8_takes_the_register_staged_loaders(m, n, k):
    _announce("nn scalar", m, n, k)
    rng = np.random.default_rng(n * k)
    a = (rng.integers(-8, 9, size=(m, k)) / 8).astype(np.float16)
    b = (rng.integers(-8, 9, size=(k, n)) / 8).astype(np.float16)
    d64, _ = oracle.gemm_f16_nn_f64(a, b)
    assert_exact(run_nn(a, b), d64, "scalar path")
    assert_exact(run_nn(a, b, a_offset=1, b_offset=3), d64, "unaligned")


def test_k_zero_and_empty():
    _announce("nn degenerate")
    got = run_nn(np.zeros((9, 0), np.float16), np.zeros((0, 12), np.float16))
    assert np.all(got == 0) and not np.any(np.signbit(got))
    assert run_nn(np.zeros((0, 8), np.float16), np.ones((8, 16), np.float16)).shape == (0, 16)


# Rows of B (and D) near the column limits of the second contract's kernels:
# a 256-row block of fp32 D spans less than 2^31 bytes below N = 2^21 (the
# one-workgroup-per-CU kernel takes 2^21 - 8, the one-tile-per-workgroup
# kernel 2^21), and a K-tile's 64 k-rows of B do below N = 2^24 (the
# direct-to-LDS loader takes 2^24 - 8, the register-staged one 2^24).  A has
# one 1 per row, at column p(m), so D[m][n] = B[p(m)][n] exactly; the check
# runs on the GPU over all of D, with guard bands.
WIDE_NN = [(512, (1 << 21) - 8, 256), (512, 1 << 21, 256), (64, (1 << 24) - 8, 64), (64, 1 << 24, 64)]


@pytest.mark.parametrize("m,n,k", WIDE_NN)
def test_widest_rows_one_hot(m, n, k):
    _announce("nn wide-n", m, n, k)
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(n + k)
    b = torch.randn((k, n), generator=gen, device=dev).to(torch.float16)
    tiny = b.abs() < 2.0**-10  # keep clear of fp16 subnormals
    b = torch.where(tiny, torch.copysign(torch.full_like(b, 2.0**-10), b), b)
    p = (torch.arange(m, device=dev) * 37 + 11) % k
    a = torch.zeros((m, k), dtype=torch.float16, device=dev)
    a[torch.arange(m, device=dev), p] = 1.0
    d_buf = torch.full((GUARD + m * n + GUARD,), float(SENTINEL), dtype=torch.float32, device=dev)
    rc = g.gemm_f16_nn_f32_raw(m, n, k, a.data_ptr(), b.data_ptr(), d_buf.data_ptr() + 4 * GUARD,
                               torch.cuda.current_stream().cuda_stream)
    assert rc == g.OK, g.status_string(rc)
    torch.cuda.synchronize()
    assert bool((d_buf[:GUARD] == float(SENTINEL)).all()) and \
        bool((d_buf[GUARD + m * n:] == float(SENTINEL)).all()), "write outside D"
    d = d_buf[GUARD:GUARD + m * n].view(m, n)
    bad = int((d.view(torch.int32) != b[p, :].float().view(torch.int32)).sum())
    assert bad == 0, f"{m}x{n}x{k} one-hot: {bad} mismatches"


# Non-finite operands: +-inf times a non-zero value gives +-inf, inf times 0
# and inf - inf give NaN, and NaN propagates.  NaN is compared as a class;
# every other element exactly ({-8..8}/8 elsewhere: exact sums).
@pytest.mark.parametrize("tile", NN_TILES)
def test_non_finite_operands(tile):
    _announce("nn non-finite", tile)
    rng = np.random.default_rng(11 + tile)
    m, n, k = 66, 72, 24
    a = (rng.integers(-8, 9, size=(m, k)) / 8).astype(np.float16)
    b = (rng.integers(-8, 9, size=(k, n)) / 8).astype(np.float16)
    b[0, :] = np.where(rng.random(n) < 0.2, 0.0, b[0, :])
    a[0, 0] = np.inf
    a[1, 0] = -np.inf
    a[2, 0], a[2, 1] = np.inf, -np.inf
    a[3, 5] = np.nan
    b[7, 4] = np.inf
    with np.errstate(invalid="ignore"):
        d64, _ = oracle.gemm_f16_nn_f64(a, b)
    got = run_nn(a, b, tile=tile)
    rn, gn = np.isnan(d64), np.isnan(got)
    assert rn.any() and np.isinf(d64).any()
    bad = np.argwhere(rn != gn)
    assert bad.size == 0, f"NaN pattern differs at {tuple(bad[0])}: gpu {got[tuple(bad[0])]} ref {d64[tuple(bad[0])]}"
    assert np.array_equal(got[~rn].astype(np.float64), d64[~rn]), "finite/inf elements differ"


def test_8192_uniform_sampled_rows():
    """The measurement workload of this contract, default launch; the oracle
    computes one row per 256-row block tile."""
    _announce("gemm_nn_8192_uniform")
    w = inputs.WORKLOADS["gemm_nn_8192_uniform"]
    a, b = inputs.workload_inputs(w.name)
    got = run_nn(a, b)
    rows = sorted({0, w.m - 1} | {t * 256 + (t * 53 + 7) % 256 for t in range(w.m // 256)})
    d64, dabs = oracle.gemm_f16_nn_f64(a, b, rows=rows)
    assert_fp32_bound(got[rows], d64, dabs, w.k, w.name)


def test_schedule_options_do_not_change_bits():
    _announce("nn determinism")
    rng = np.random.default_rng(77)
    a = rng.standard_normal((1024, 384)).astype(np.float16)
    b = rng.standard_normal((384, 1280)).astype(np.float16)
    base = run_nn(a, b, tile=g.TILE_256x256)
    for sw, xcd in [(1, 0), (3, 1), (8, 0)]:
        assert np.array_equal(run_nn(a, b, tile=g.TILE_256x256, swizzle=sw, xcd=xcd).view(np.uint32),
                              base.view(np.uint32))


def test_torch_wrapper():
    _announce("nn torch wrapper")
    rng = np.random.default_rng(4)
    a = rng.standard_normal((200, 96)).astype(np.float16)
    b = rng.standard_normal((96, 136)).astype(np.float16)
    d = g.gemm_f16_nn_f32(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda())
    torch.cuda.synchronize()
    d64, dabs = oracle.gemm_f16_nn_f64(a, b)
    assert_fp32_bound(d.cpu().numpy(), d64, dabs, 96, "wrapper")
