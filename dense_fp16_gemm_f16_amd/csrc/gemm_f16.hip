// libgemm_f16 host side: the C ABI of include/gemm_f16.h -- argument
// checks, the device gate, the block-tile choice and the launch.  The
// kernels live in kernels.h and are compiled per block tile (tile_*.hip).
#include <atomic>
#include <cstdlib>
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <algorithm>
#include <bitset>

#include "gemm_f16.h"
#include "kernels.h"

namespace gemm_f16 {

// Fill the output with +0 (K == 0: the zero accumulator is what gets stored).
template <class T>
__global__ __launch_bounds__(256) void fill_zero_kernel(T *c, int64_t count) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
        c[i] = (T)0.0f;
}

struct TileShape {
    int bm, bn;
};

static TileShape tile_shape(int tile) {
    switch (tile) {
        case GEMM_F16_TILE_256x256: return {256, 256};
        case GEMM_F16_TILE_256x256_W8: return {256, 256};
        case GEMM_F16_TILE_256x128: return {256, 128};
        case GEMM_F16_TILE_128x256: return {128, 256};
        case GEMM_F16_TILE_128x128: return {128, 128};
        case GEMM_F16_TILE_128x128_M16: return {128, 128};
        case GEMM_F16_TILE_64x128: return {64, 128};
        case GEMM_F16_TILE_128x64: return {128, 64};
        default: return {64, 64};
    }
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Automatic block tile: the candidate with the smallest modelled time
//     t = c + a * rounds * k_tiles + b * tiles / cus,
// rounds = ceil(tiles / cus) rounds of one workgroup per CU, k_tiles =
// ceil(K / 64): a fixed cost per launch (c), the K loop of each round (a per
// K-tile) and a cost per tile that the one-workgroup-per-CU kernels spread
// over the CUs (b: prologue, epilogue and C stores).  The coefficients (us)
// are a least-squares fit, in relative error, to two sweeps of every block
// tile over 42 shapes (M, N from 512 to 16384, K 256 / 1024 / 4096) on
// MI355X, taking the geometric mean of the two (python -m
// dense_fp16_gemm_f16_amd.tune --fit).  Only the ranking matters.  cus:
// compute units of the device (256 if unknown).  With K % 8 != 0 the 256x256
// tile would run as 128x256 (see gemm_impl), so it is not a candidate.
//
// The model cannot tell 256x128 from 128x256 by the matrix's orientation;
// measured, the long side of the tile along the shorter matrix dimension
// was the faster (8192x1024x1024: 128x256 19.8 us, 256x128 21.7;
// 1024x8192x1024: 256x128 19.9, 128x256 21.5), so that one is taken unless
// it needs more rounds of tiles.  With that, the model's tile was within 3%
// of the fastest on 38 of the 42 shapes and within 8.2% on all of them.
static int auto_tile(int64_t m, int64_t n, int64_t k, int cus) {
    if (cus <= 0) cus = 256;
    struct Cand {
        int id, bm, bn;
        double c, a, b;
    };
    static const Cand cands[] = {
        {GEMM_F16_TILE_256x256, 256, 256, 8.280, 1.115, 6.212},
        {GEMM_F16_TILE_256x128, 256, 128, 5.825, 0.663, 3.036},
        {GEMM_F16_TILE_128x256, 128, 256, 5.856, 0.661, 2.886},
        {GEMM_F16_TILE_128x128, 128, 128, 4.492, 0.436, 1.517},
        {GEMM_F16_TILE_128x64, 128, 64, 3.479, 0.385, 0.845},
        {GEMM_F16_TILE_64x128, 64, 128, 3.545, 0.391, 0.780},
        {GEMM_F16_TILE_64x64, 64, 64, 3.254, 0.308, 0.315},
    };
    const int64_t k_tiles = cdiv(k, 64);
    int best = GEMM_F16_TILE_64x64;
    double best_t = 1e300;
    for (const Cand &c : cands) {
        if (c.id == GEMM_F16_TILE_256x256 && k % 8 != 0) continue;
        const int64_t tiles = cdiv(m, c.bm) * cdiv(n, c.bn);
        const int64_t rounds = cdiv(tiles, cus);
        const double t = c.c + c.a * (double)rounds * (double)k_tiles + c.b * (double)tiles / cus;
        if (t < best_t * 0.999) {
            best_t = t;
            best = c.id;
        }
    }
    if ((best == GEMM_F16_TILE_256x128 || best == GEMM_F16_TILE_128x256) && m != n) {
        // rounds of tiles on 128 x 256 (wide) or 256 x 128
        auto rounds = [&](bool wide) { return cdiv(cdiv(m, wide ? 128 : 256) * cdiv(n, wide ? 256 : 128), cus); };
        const bool wide = m > n;
        if (rounds(wide) <= rounds(best == GEMM_F16_TILE_128x256))
            best = wide ? GEMM_F16_TILE_128x256 : GEMM_F16_TILE_256x128;
    }
    return best;
}

// Operand panels that the busiest XCD reads in a grid of one round: the
// distinct tile rows (panels of A) plus tile columns (panels of B) among
// the tiles it runs, dispatch index p running on XCD p % 8.  At most 1024
// tiles.
static int busiest_xcd_panels(uint32_t num_m, uint32_t num_n, uint32_t swizzle, bool remap) {
    const uint32_t grid = num_m * num_n;
    int most = 0;
    for (uint32_t x = 0; x < (uint32_t)kNumXcd; ++x) {
        std::bitset<1024> rows, cols;
        for (uint32_t pid = x; pid < grid; pid += kNumXcd) {
            const TileCoord t = tile_coord<uint32_t>(pid, num_m, num_n, swizzle, remap);
            rows.set((size_t)t.m_block);
            cols.set((size_t)t.n_block);
        }
        most = std::max(most, (int)(rows.count() + cols.count()));
    }
    return most;
}

// Rasterization when the options leave it open (xcd == -1): the XCD remap,
// except on a grid that fills the CUs exactly once.  There the hardware's
// dispatch order is kept when it leaves no XCD more operand panels than
// the remap does: on MI355X it ran 1-6% faster on 16x16 grids of 256 tiles
// (4096^2 x K, 2048^3 on 128x128) and level on 8x32, while grids where it
// gives more panels (32x8, 4x64) ran level to 17% slower.  Returns 1
// (remap) or 0 (dispatch order).
static int default_xcd(int64_t num_m, int64_t num_n, int32_t swizzle, int cus) {
    const int64_t tiles = num_m * num_n;
    if (cus <= 0 || swizzle < 1 || tiles != cus || tiles > 1024) return 1;
    // the panel count walks the grid: one remembered shape per host thread
    thread_local int64_t key_m = -1, key_n = -1;
    thread_local int32_t key_s = -1;
    thread_local int value = 1;
    if (key_m != num_m || key_n != num_n || key_s != swizzle) {
        const uint32_t nm = (uint32_t)num_m, nn = (uint32_t)num_n, sw = (uint32_t)swizzle;
        value = busiest_xcd_panels(nm, nn, sw, false) <= busiest_xcd_panels(nm, nn, sw, true) ? 0 : 1;
        key_m = num_m, key_n = num_n, key_s = swizzle;
    }
    return value;
}

// Cache policy of C's 16-byte stores (CStore in kernels.h).  While A, B
// and C together fit in the 256 MiB Infinity Cache, device-scope stores let
// it take C's store bursts: interleaved on MI355X, 1-5% faster on such
// shapes (4096^3 98.2 vs 100.6 us, 3072^3 54.4 vs 55.8, 4096x16384x2048
// 195.2 vs 205.3, 8192^2x1024 108.9 vs 113.6).  Past that they evict A and
// B (16384x8192x1024, 304 MiB: 9% slower; 16384^2x2048: 9.5%), so larger
// problems keep streaming stores on rows of whole 128-byte lines and the
// default elsewhere.  The second contract (fp32 D) takes the same rule
// (device scope: 2048^3 23.8 vs 25.7 us, 4096^3 111.2 vs 116.3), except that
// its one-tile kernels store past the cache with the default policy.
static int32_t c_store_policy(bool nn, int64_t m, int64_t n, int64_t k, const void *c) {
    constexpr int64_t kInfinityCacheBytes = int64_t(256) << 20;
    const int64_t out_bytes = nn ? 4 : 2;
    const bool lines = (n * out_bytes) % 128 == 0 && ((uintptr_t)c % 128) == 0;
    if ((m * k + n * k) * 2 + m * n * out_bytes <= kInfinityCacheBytes) return kStoreDevice;
    return lines ? kStoreStream : kStoreDefault;
}

// A kernel variant (options.variant 1..7): block_k and stages of each, and
// the tiles whose LDS holds its ring (S x (BM + BN) x 2 block_k bytes <= 160
// KB) and, with loader waves, whose MFMA waves fit in 256 registers (2
// stages: up to 128x64 per MFMA wave, not 256x256; 3 stages: 128x128
// only).  The same conditions decide, at compile time, which variants exist
// (ring_fits in kernels.h).
static bool variant_ok(bool nn, int tile, int variant, int64_t k, const void *a, const void *b) {
    static const int bk[] = {0, 64, 64, 32, 32, 32, 64, 64};
    static const int st[] = {0, 2, 3, 2, 3, 4, 2, 3};
    if (nn || variant < 1 || variant > GEMM_F16_VARIANT_LAST) return false;
    if (k <= 0 || k % bk[variant] != 0 || (((uintptr_t)a | (uintptr_t)b) % 16) != 0) return false;
    int bm, bn;
    switch (tile) {
        case GEMM_F16_TILE_256x256: bm = 256, bn = 256; break;
        case GEMM_F16_TILE_256x128: bm = 256, bn = 128; break;
        case GEMM_F16_TILE_128x256: bm = 128, bn = 256; break;
        case GEMM_F16_TILE_128x128: bm = 128, bn = 128; break;
        default: return false;
    }
    const bool prod = variant >= GEMM_F16_VARIANT_PRODUCER_S2;
    if (prod && bm * bn > (variant == GEMM_F16_VARIANT_PRODUCER_S2 ? 256 * 128 : 128 * 128)) return false;
    return st[variant] * (bm + bn) * 2 * bk[variant] <= 160 * 1024;
}

static int check_sizes(int64_t m, int64_t n, int64_t k) {
    if (m < 0 || n < 0 || k < 0) return GEMM_F16_EINVAL;
    // The kernels index rows and columns of C in 32-bit ints, and the last
    // block tile reaches up to 255 past m and n: below 2^30 that cannot wrap.
    if (m >= (int64_t(1) << 30) || n >= (int64_t(1) << 30)) return GEMM_F16_EINVAL;
    if (k >= (int64_t(1) << 22)) return GEMM_F16_EINVAL;
    // m, n < 2^30, so the product cannot overflow; the bound keeps every
    // byte extent (m*n*4, m*k*2, n*k*2) far below 2^63 and the address range
    // checks free of wrap-around
    if (m * n >= (int64_t(1) << 47)) return GEMM_F16_EINVAL;
    return GEMM_F16_OK;
}

static bool ranges_overlap(const void *p, int64_t pb, const void *q, int64_t qb) {
    const uintptr_t a0 = (uintptr_t)p, a1 = a0 + (uintptr_t)pb;
    const uintptr_t b0 = (uintptr_t)q, b1 = b0 + (uintptr_t)qb;
    return pb > 0 && qb > 0 && a0 < b1 && b0 < a1;
}

// Per-device caches below: host threads may call the library at the same
// time, so the entries are atomics; a first call on a device in two threads
// at once computes the same value twice and stores it twice.

// Compute units of the current device (0 if unknown), cached per device.
static int device_cus() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// "gfx950", optionally followed by ":" and target features.
static bool is_gfx950(const char *arch) {
    return arch[0] == 'g' && arch[1] == 'f' && arch[2] == 'x' && arch[3] == '9' && arch[4] == '5' &&
           arch[5] == '0' && (arch[6] == '\0' || arch[6] == ':');
}

// Test hook: when the environment variable GEMM_F16_TEST_ARCH is set as the
// library loads, its value stands in for every device's architecture name
// in the gate below (no device is queried), so the refusal path can be
// exercised on any host.
static const char *const kTestArch = std::getenv("GEMM_F16_TEST_ARCH");

// gfx950 check, cached per device.
static int check_device() {
    if (kTestArch) return is_gfx950(kTestArch) ? GEMM_F16_OK : GEMM_F16_EDEVICE;
    static std::atomic<int> cached[64];  // 0 = unknown, 1 = gfx950, -1 = other
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GEMM_F16_EHIP;
    if (dev < 0 || dev >= 64) return GEMM_F16_EDEVICE;
    int state = cached[dev].load(std::memory_order_relaxed);
    if (state == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GEMM_F16_EHIP;
        state = is_gfx950(prop.gcnArchName) ? 1 : -1;
        cached[dev].store(state, std::memory_order_relaxed);
    }
    return state == 1 ? GEMM_F16_OK : GEMM_F16_EDEVICE;
}

// Both contracts: NN == false is C fp16 = A B^T (B [N,K]); NN == true is
// D fp32 = A B (B [K,N]).
static int gemm_impl(bool nn, int64_t m, int64_t n, int64_t k, const void *a, const void *b, void *c,
                     void *stream, const gemm_f16_options *opt) {
    int rc = check_sizes(m, n, k);
    if (rc != GEMM_F16_OK) return rc;
    if (nn && n >= (int64_t(1) << 25)) return GEMM_F16_EINVAL;
    gemm_f16_options o = {0, 0, -1, 0};
    if (opt) o = *opt;
    if (o.tile < 0 || o.tile > GEMM_F16_TILE_LAST || o.swizzle < 0 || o.xcd < -1 || o.xcd > 1)
        return GEMM_F16_EINVAL;
    if (o.variant != GEMM_F16_VARIANT_DEFAULT && !variant_ok(nn, o.tile, o.variant, k, a, b)) return GEMM_F16_EINVAL;
    if (nn && o.tile == GEMM_F16_TILE_128x128_M16) return GEMM_F16_EINVAL;
    if (m == 0 || n == 0) return GEMM_F16_OK;
    if (!c || (k > 0 && (!a || !b))) return GEMM_F16_ENULL;
    const int out_bytes = nn ? 4 : 2;
    if (((uintptr_t)c & (out_bytes - 1)) || ((uintptr_t)a & 1) || ((uintptr_t)b & 1)) return GEMM_F16_EALIGN;
    if (k > 0 && (ranges_overlap(c, m * n * out_bytes, a, m * k * 2) ||
                  ranges_overlap(c, m * n * out_bytes, b, n * k * 2)))
        return GEMM_F16_EOVERLAP;
    rc = check_device();
    if (rc != GEMM_F16_OK) return rc;
    hipStream_t s = (hipStream_t)stream;

    if (k == 0) {
        const int64_t count = m * n;
        const dim3 grid((unsigned)std::min<int64_t>(cdiv(count, 256), 4096)), block(256);
        hipError_t e;
        if (nn) {
            float *d = (float *)c;
            void *args[] = {&d, const_cast<int64_t *>(&count)};
            e = hipLaunchKernel(reinterpret_cast<const void *>(fill_zero_kernel<float>), grid, block, args, 0, s);
        } else {
            _Float16 *h = (_Float16 *)c;
            void *args[] = {&h, const_cast<int64_t *>(&count)};
            e = hipLaunchKernel(reinterpret_cast<const void *>(fill_zero_kernel<_Float16>), grid, block, args, 0, s);
        }
        return e == hipSuccess ? GEMM_F16_OK : GEMM_F16_EHIP;
    }

    // The operands' row alignment: 16-byte aligned rows of A, and of B in
    // its layout, take the direct-to-LDS loads; for C = A B^T, rows aligned
    // to 4 bytes take 16-byte loads at 4-byte aligned offsets; otherwise
    // (2-byte aligned rows) 16-byte loads shifted into place.
    const uintptr_t ab = (uintptr_t)a | (uintptr_t)b;
    int g = 1;
    if ((k % 8) == 0 && (!nn || (n % 8) == 0) && (ab % 16) == 0)
        g = 8;
    else if (!nn && (k % 2) == 0 && (ab % 4) == 0)
        g = 2;

    const int cus = device_cus();
    int tile = o.tile ? o.tile : auto_tile(m, n, k, cus);
    // The 256x256 tiles' register-staged kernels would spill their staging
    // registers with loads narrower than 16 bytes: those operands run on
    // the 128x256 tile.
    if (g < 8 && (tile == GEMM_F16_TILE_256x256 || tile == GEMM_F16_TILE_256x256_W8)) tile = GEMM_F16_TILE_128x256;
    const TileShape ts = tile_shape(tile);
    Params p;
    p.a = (const _Float16 *)a;
    p.b = (const _Float16 *)b;
    p.c = c;
    p.m = (int32_t)m;
    p.n = (int32_t)n;
    p.k = (int32_t)k;
    p.num_m = (int32_t)cdiv(m, ts.bm);
    p.num_n = (int32_t)cdiv(n, ts.bn);
    p.k_tiles = (int32_t)cdiv(k, 64);
    p.swizzle = o.swizzle ? o.swizzle : 4;
    p.xcd = o.xcd < 0 ? default_xcd(p.num_m, p.num_n, p.swizzle, cus) : o.xcd;
    p.c_store = c_store_policy(nn, m, n, k, c);
    if ((int64_t)p.num_m * p.num_n >= (int64_t(1) << 31)) return GEMM_F16_EINVAL;

    hipError_t e;
    if (o.variant != GEMM_F16_VARIANT_DEFAULT) {
        switch (tile) {
            case GEMM_F16_TILE_256x256: e = launch_ring_256x256(o.variant, p, s); break;
            case GEMM_F16_TILE_256x128: e = launch_ring_256x128(o.variant, p, s); break;
            case GEMM_F16_TILE_128x256: e = launch_ring_128x256(o.variant, p, s); break;
            default: e = launch_ring_128x128(o.variant, p, s); break;
        }
        return e == hipSuccess ? GEMM_F16_OK : GEMM_F16_EHIP;
    }
    switch (tile) {
        case GEMM_F16_TILE_256x256: e = launch_256x256(nn, p, g, cus, s); break;
        case GEMM_F16_TILE_256x256_W8: e = launch_256x256_w8(nn, p, g, cus, s); break;
        case GEMM_F16_TILE_256x128: e = launch_256x128(nn, p, g, cus, s); break;
        case GEMM_F16_TILE_128x256: e = launch_128x256(nn, p, g, cus, s); break;
        case GEMM_F16_TILE_128x128: e = launch_128x128(nn, p, g, cus, s); break;
        case GEMM_F16_TILE_128x128_M16: e = launch_128x128_m16(p, g, cus, s); break;
        case GEMM_F16_TILE_64x128: e = launch_64x128(nn, p, g, cus, s); break;
        case GEMM_F16_TILE_128x64: e = launch_128x64(nn, p, g, cus, s); break;
        default: e = launch_64x64(nn, p, g, cus, s); break;
    }
    return e == hipSuccess ? GEMM_F16_OK : GEMM_F16_EHIP;
}

}  // namespace gemm_f16

using namespace gemm_f16;

extern "C" {

int gemm_f16_select_tile(int64_t m, int64_t n, int64_t k) {
    const int rc = check_sizes(m, n, k);
    if (rc != GEMM_F16_OK) return rc;
    return auto_tile(m, n, k, device_cus());
}

int gemm_f16_select_xcd(int64_t num_m, int64_t num_n, int32_t swizzle, int32_t cus) {
    if (num_m < 1 || num_n < 1 || num_m > INT64_MAX / num_n || num_m * num_n >= (int64_t(1) << 31) ||
        swizzle < 1 || cus < 0)
        return GEMM_F16_EINVAL;
    return default_xcd(num_m, num_n, swizzle, cus);
}

int gemm_f16_tile_coord(int64_t pid, int64_t num_m, int64_t num_n, int32_t swizzle, int32_t xcd,
                        int64_t *m_block, int64_t *n_block) {
    // the grid's size first, so that num_m * num_n cannot overflow
    if (num_m < 1 || num_n < 1 || num_m > INT64_MAX / num_n || swizzle < 1 || pid < 0 || pid >= num_m * num_n)
        return GEMM_F16_EINVAL;
    if (!m_block || !n_block) return GEMM_F16_ENULL;
    // grids the kernels run (below 2^31 tiles) take their 32-bit arithmetic
    const TileCoord t = num_m * num_n < (int64_t(1) << 31)
                            ? tile_coord<uint32_t>((uint32_t)pid, (uint32_t)num_m, (uint32_t)num_n,
                                                   (uint32_t)swizzle, xcd != 0)
                            : tile_coord<int64_t>(pid, num_m, num_n, swizzle, xcd != 0);
    *m_block = t.m_block;
    *n_block = t.n_block;
    return GEMM_F16_OK;
}

int gemm_f16_nt_ex(int64_t m, int64_t n, int64_t k, const void *a, const void *b, void *c,
                   void *stream, const gemm_f16_options *opt) {
    return gemm_impl(false, m, n, k, a, b, c, stream, opt);
}

int gemm_f16_nt(int64_t m, int64_t n, int64_t k, const void *a, const void *b, void *c,
                void *stream) {
    return gemm_impl(false, m, n, k, a, b, c, stream, nullptr);
}

int gemm_f16_nn_f32_ex(int64_t m, int64_t n, int64_t k, const void *a, const void *b, void *d,
                       void *stream, const gemm_f16_options *opt) {
    return gemm_impl(true, m, n, k, a, b, d, stream, opt);
}

int gemm_f16_nn_f32(int64_t m, int64_t n, int64_t k, const void *a, const void *b, void *d,
                    void *stream) {
    return gemm_impl(true, m, n, k, a, b, d, stream, nullptr);
}

const char *gemm_f16_status_string(int status) {
    switch (status) {
        case GEMM_F16_OK: return "ok";
        case GEMM_F16_EINVAL: return "invalid argument (size out of range or bad option)";
        case GEMM_F16_ENULL: return "null pointer with a non-empty extent";
        case GEMM_F16_EALIGN: return "pointer not aligned to its element size";
        case GEMM_F16_EDEVICE: return "current device is not gfx950 (MI355X)";
        case GEMM_F16_EHIP: return "HIP runtime error or kernel launch failure";
        case GEMM_F16_EOVERLAP: return "the output overlaps a or b";
        default: return "unknown status";
    }
}

}  // extern "C"
