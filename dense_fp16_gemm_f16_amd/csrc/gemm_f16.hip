// libgemm_f16: C = fp16(A * B^T), fp16 inputs, fp32 accumulation, for gfx950.
//
// The operation is the one the Tilus tutorial "1. WGMMA: Hopper's
// Asynchronous Tensor Core" builds in "The Full Kernel": A is [M,K], B is
// [N,K], the fp32 accumulator starts at zero, the block tile walks K in
// block_k steps, and the accumulator is cast to fp16 and stored at the
// block's (m, n) offset.  The mechanism here is CDNA4's, not Hopper's:
//
//  * scheduler  one workgroup per output block tile over a 1D grid,
//               XCD-aware and swizzle-rasterized (tile_sched.h);
//  * loader     buffer_load_dwordx4 of 16-byte K-chunks (one 128-byte row
//               segment per 8 lanes), staged in VGPRs one K-tile ahead and
//               written to a 2-stage LDS ring; hardware range checks of the
//               buffer descriptor return zero for rows past M/N, and a
//               per-chunk mask returns zero for k >= K;
//  * LDS        each row of a tile is 8 chunks of 16 bytes, stored at chunk
//               position (c ^ swz(row)), so the ds_read_b128 fragment reads
//               of the MFMA loop and the ds_write_b128 stores are free of
//               bank conflicts;
//  * compute    4 waves in a 2 x 2 arrangement, each owning a
//               (BM/2) x (BN/2) piece of C as independent 32x32 fp32
//               accumulators, fed by v_mfma_f32_32x32x16_f16;
//  * epilogue   fp32 -> fp16 round-to-nearest-even, stores masked to
//               [M, N].
//
// The sum of each output runs over K-tiles in increasing order, and inside
// a K-tile over 16-wide k steps in increasing order, whatever the grid
// order: results do not depend on the rasterization options.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "gemm_f16.h"
#include "tile_sched.h"

namespace gemm_f16 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int int4v __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 waves of 64
constexpr int kWave = 64;
constexpr uint32_t kOutOfRange = 0x80000000u;  // buffer offset past any num_records: reads 0

struct Params {
    const _Float16 *a;
    const _Float16 *b;
    _Float16 *c;
    int32_t m, n, k;
    int32_t num_m, num_n;  // block tiles along M and N
    int32_t k_tiles;       // ceil(k / BK)
    int32_t swizzle;
    int32_t xcd;
    int32_t vec_c;         // C rows allow 8-byte stores (N % 4 == 0, c 8-byte aligned)
};

// Position of 16-byte chunk `c` of tile row `row` inside that row (8 chunks
// per 128-byte row).  A 64-lane ds_read_b128 of a 32x32x16 MFMA fragment
// reads 32 consecutive rows at one chunk; XORing with row ^ (row >> 3)
// spreads any 8 consecutive rows over all 8 chunk slots and any 16
// consecutive rows over distinct (row parity, slot) pairs, so neither
// 8-lane nor 16-lane groups of the read hit a bank twice.
__device__ __forceinline__ int swz8(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    // word3 0x00020000: raw (untyped) 32-bit data format, as gfx9-family
    // buffer descriptors expect.
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// LDS barrier that waits only for this wave's LDS traffic (lgkmcnt), not for
// the global loads still in flight for the next K-tile.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One operand's K-tile: ROWS x 64 fp16, 8 chunks per row, 32 rows per
// pass of the 256 threads; thread t owns chunk t % 8 of rows t / 8 + 32 i.
template <int ROWS, bool VEC>
struct TileLoader {
    static constexpr int kPasses = ROWS / 32;
    int4v regs[kPasses];

    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rsrc, int k_elems, int k0, int tid) {
        const int chunk = tid & 7;
        const int row0 = tid >> 3;
        const int kc = k0 + chunk * 8;
        if constexpr (VEC) {
            // K % 8 == 0 here, so a chunk is either wholly inside K or wholly
            // out.  Bit 31 is set when kc >= K (kc - K >= 0), which moves the
            // offset past num_records; computed without a branch.
            const uint32_t oor = (~(uint32_t)(kc - k_elems)) & kOutOfRange;
#pragma unroll
            for (int i = 0; i < kPasses; ++i) {
                const int row = row0 + 32 * i;
                const uint32_t off = ((uint32_t)(row * k_elems + kc) * 2u) | oor;
                regs[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
            }
        } else {
#pragma unroll
            for (int i = 0; i < kPasses; ++i) {
                const int row = row0 + 32 * i;
                union {
                    short s[8];
                    int4v v;
                } u;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t off =
                        (kc + e < k_elems) ? (uint32_t)(row * k_elems + kc + e) * 2u : kOutOfRange;
                    u.s[e] = __builtin_amdgcn_raw_buffer_load_b16(rsrc, off, 0, 0);
                }
                regs[i] = u.v;
            }
        }
    }

    __device__ __forceinline__ void store(int4v *lds_tile, int tid) const {
        const int chunk = tid & 7;
        const int row0 = tid >> 3;
#pragma unroll
        for (int i = 0; i < kPasses; ++i) {
            const int row = row0 + 32 * i;
            lds_tile[row * 8 + (chunk ^ swz8(row))] = regs[i];
        }
    }
};

template <int BM, int BN, bool VEC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_f16_nt_kernel(const Params p) {
    constexpr int BK = 64;
    constexpr int TM = BM / 2;  // wave tile (2 x 2 waves)
    constexpr int TN = BN / 2;
    constexpr int FM = TM / 32;  // 32x32 MFMA blocks per wave
    constexpr int FN = TN / 32;
    constexpr int kStageChunks = (BM + BN) * (BK / 8);
    __shared__ int4v smem[2 * kStageChunks];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave >> 1;
    const int wn = wave & 1;

    const TileCoord tc = tile_coord(blockIdx.x, p.num_m, p.num_n, p.swizzle, p.xcd != 0);
    const int m0 = (int)tc.m_block * BM;
    const int n0 = (int)tc.n_block * BN;

    // Per-tile buffer descriptors: rows past M (N) lie beyond num_records.
    const int rows_a = min(BM, p.m - m0);
    const int rows_b = min(BN, p.n - n0);
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(p.a + (int64_t)m0 * p.k, (uint32_t)rows_a * (uint32_t)p.k * 2u);
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(p.b + (int64_t)n0 * p.k, (uint32_t)rows_b * (uint32_t)p.k * 2u);

    TileLoader<BM, VEC> la;
    TileLoader<BN, VEC> lb;

    floatx16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = floatx16{};

    const int kt_count = p.k_tiles;
    if (kt_count > 0) {
        la.load(ra, p.k, 0, tid);
        lb.load(rb, p.k, 0, tid);
        la.store(smem, tid);
        lb.store(smem + BM * 8, tid);
        if (kt_count > 1) {
            la.load(ra, p.k, BK, tid);
            lb.load(rb, p.k, BK, tid);
        }
        lds_barrier();
    }

    // Fragment rows this lane reads: lanes 0-31 and 32-63 take the two
    // 8-wide k halves of each 16-wide k step.
    const int frag_row = lane & 31;
    const int frag_half = lane >> 5;

    for (int kt = 0; kt < kt_count; ++kt) {
        const int4v *sa = smem + (kt & 1) * kStageChunks;
        const int4v *sb = sa + BM * 8;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int chunk = ks * 2 + frag_half;
            half8 af[FM];
            half8 bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * TM + i * 32 + frag_row;
                af[i] = __builtin_bit_cast(half8, sa[row * 8 + (chunk ^ swz8(row))]);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int row = wn * TN + j * 32 + frag_row;
                bf[j] = __builtin_bit_cast(half8, sb[row * 8 + (chunk ^ swz8(row))]);
            }
            // B rows feed the MFMA's A operand and A rows its B operand, so
            // the 32x32 result block is C^T: each lane then holds 4
            // consecutive n of one m row, which stores as 8 bytes.
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[j], af[i], acc[j][i], 0, 0, 0);
        }
        if (kt + 1 < kt_count) {
            int4v *nxt = smem + ((kt + 1) & 1) * kStageChunks;
            la.store(nxt, tid);
            lb.store(nxt + BM * 8, tid);
            if (kt + 2 < kt_count) {
                la.load(ra, p.k, (kt + 2) * BK, tid);
                lb.load(rb, p.k, (kt + 2) * BK, tid);
            }
        }
        lds_barrier();
    }

    // Epilogue.  32x32 MFMA result layout: lane l, register r holds row
    // 8*(r/4) + 4*(l/32) + r%4, column l%32 of the block; with the swapped
    // operands the row is n and the column is m.
    const int quad = (lane >> 5) * 4;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * TM + i * 32 + frag_row;
        if (m >= p.m) continue;
        _Float16 *crow = p.c + (int64_t)m * p.n;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * TN + j * 32 + 8 * g + quad;
                half4 h;
                h[0] = (_Float16)acc[j][i][4 * g + 0];
                h[1] = (_Float16)acc[j][i][4 * g + 1];
                h[2] = (_Float16)acc[j][i][4 * g + 2];
                h[3] = (_Float16)acc[j][i][4 * g + 3];
                if (p.vec_c && n + 3 < p.n) {
                    *reinterpret_cast<half4 *>(crow + n) = h;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < p.n) crow[n + e] = h[e];
                }
            }
        }
    }
}

// Fill C with +0 (K == 0: the zero accumulator is what gets stored).
__global__ __launch_bounds__(256) void fill_zero_kernel(_Float16 *c, int64_t count) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
        c[i] = (_Float16)0.0f;
}

// ---- host side --------------------------------------------------------------

struct TileShape {
    int bm, bn;
};

static TileShape tile_shape(int tile) {
    switch (tile) {
        case GEMM_F16_TILE_256x256: return {256, 256};
        case GEMM_F16_TILE_128x128: return {128, 128};
        default: return {64, 64};
    }
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Largest tile that still gives at least one workgroup per CU (256 CUs);
// otherwise the tile with the most workgroups.
static int auto_tile(int64_t m, int64_t n) {
    if (cdiv(m, 256) * cdiv(n, 256) >= 256) return GEMM_F16_TILE_256x256;
    if (cdiv(m, 128) * cdiv(n, 128) >= 128) return GEMM_F16_TILE_128x128;
    return GEMM_F16_TILE_64x64;
}

static int check_sizes(int64_t m, int64_t n, int64_t k) {
    if (m < 0 || n < 0 || k < 0) return GEMM_F16_EINVAL;
    if (m >= (int64_t(1) << 31) || n >= (int64_t(1) << 31)) return GEMM_F16_EINVAL;
    if (k >= (int64_t(1) << 22)) return GEMM_F16_EINVAL;
    return GEMM_F16_OK;
}

static bool ranges_overlap(const void *p, int64_t pb, const void *q, int64_t qb) {
    const uintptr_t a0 = (uintptr_t)p, a1 = a0 + (uintptr_t)pb;
    const uintptr_t b0 = (uintptr_t)q, b1 = b0 + (uintptr_t)qb;
    return pb > 0 && qb > 0 && a0 < b1 && b0 < a1;
}

// gfx950 check, cached per device.
static int check_device() {
    static int cached[64];  // 0 = unknown, 1 = gfx950, -1 = other
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return GEMM_F16_EHIP;
    if (dev < 0 || dev >= 64) return GEMM_F16_EDEVICE;
    if (cached[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return GEMM_F16_EHIP;
        const char *arch = prop.gcnArchName;
        const bool ok = arch[0] == 'g' && arch[1] == 'f' && arch[2] == 'x' && arch[3] == '9' &&
                        arch[4] == '5' && arch[5] == '0' && (arch[6] == '\0' || arch[6] == ':');
        cached[dev] = ok ? 1 : -1;
    }
    return cached[dev] == 1 ? GEMM_F16_OK : GEMM_F16_EDEVICE;
}

template <int BM, int BN>
static void launch(const Params &p, bool vec, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)p.num_m * p.num_n));
    if (vec)
        hipLaunchKernelGGL((gemm_f16_nt_kernel<BM, BN, true>), grid, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((gemm_f16_nt_kernel<BM, BN, false>), grid, dim3(kThreads), 0, stream, p);
}

}  // namespace gemm_f16

using namespace gemm_f16;

extern "C" {

int gemm_f16_select_tile(int64_t m, int64_t n, int64_t k) {
    const int rc = check_sizes(m, n, k);
    if (rc != GEMM_F16_OK) return rc;
    return auto_tile(m, n);
}

int gemm_f16_tile_coord(int64_t pid, int64_t num_m, int64_t num_n, int32_t swizzle, int32_t xcd,
                        int64_t *m_block, int64_t *n_block) {
    if (num_m < 1 || num_n < 1 || swizzle < 1 || pid < 0 || pid >= num_m * num_n)
        return GEMM_F16_EINVAL;
    if (!m_block || !n_block) return GEMM_F16_ENULL;
    const TileCoord t = tile_coord(pid, num_m, num_n, swizzle, xcd != 0);
    *m_block = t.m_block;
    *n_block = t.n_block;
    return GEMM_F16_OK;
}

int gemm_f16_nt_ex(int64_t m, int64_t n, int64_t k, const void *a, const void *b, void *c,
                   void *stream, const gemm_f16_options *opt) {
    int rc = check_sizes(m, n, k);
    if (rc != GEMM_F16_OK) return rc;
    gemm_f16_options o = {0, 0, -1, 0};
    if (opt) o = *opt;
    if (o.tile < 0 || o.tile > GEMM_F16_TILE_64x64 || o.swizzle < 0 || o.xcd < -1 || o.xcd > 1)
        return GEMM_F16_EINVAL;
    if (m == 0 || n == 0) return GEMM_F16_OK;
    if (!c || (k > 0 && (!a || !b))) return GEMM_F16_ENULL;
    if (((uintptr_t)c & 1) || ((uintptr_t)a & 1) || ((uintptr_t)b & 1)) return GEMM_F16_EALIGN;
    if (k > 0 && (ranges_overlap(c, m * n * 2, a, m * k * 2) || ranges_overlap(c, m * n * 2, b, n * k * 2)))
        return GEMM_F16_EOVERLAP;
    rc = check_device();
    if (rc != GEMM_F16_OK) return rc;
    hipStream_t s = (hipStream_t)stream;

    if (k == 0) {
        const int64_t count = m * n;
        const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(count, 256), 4096);
        hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, s, (_Float16 *)c, count);
        return hipGetLastError() == hipSuccess ? GEMM_F16_OK : GEMM_F16_EHIP;
    }

    const int tile = o.tile ? o.tile : auto_tile(m, n);
    const TileShape ts = tile_shape(tile);
    Params p;
    p.a = (const _Float16 *)a;
    p.b = (const _Float16 *)b;
    p.c = (_Float16 *)c;
    p.m = (int32_t)m;
    p.n = (int32_t)n;
    p.k = (int32_t)k;
    p.num_m = (int32_t)cdiv(m, ts.bm);
    p.num_n = (int32_t)cdiv(n, ts.bn);
    p.k_tiles = (int32_t)cdiv(k, 64);
    p.swizzle = o.swizzle ? o.swizzle : 4;
    p.xcd = o.xcd < 0 ? 1 : o.xcd;
    p.vec_c = ((n % 4) == 0 && ((uintptr_t)c % 8) == 0) ? 1 : 0;
    const bool vec = (k % 8) == 0 && ((uintptr_t)a % 16) == 0 && ((uintptr_t)b % 16) == 0;
    if ((int64_t)p.num_m * p.num_n >= (int64_t(1) << 31)) return GEMM_F16_EINVAL;

    switch (tile) {
        case GEMM_F16_TILE_256x256: launch<256, 256>(p, vec, s); break;
        case GEMM_F16_TILE_128x128: launch<128, 128>(p, vec, s); break;
        default: launch<64, 64>(p, vec, s); break;
    }
    return hipGetLastError() == hipSuccess ? GEMM_F16_OK : GEMM_F16_EHIP;
}

int gemm_f16_nt(int64_t m, int64_t n, int64_t k, const void *a, const void *b, void *c,
                void *stream) {
    return gemm_f16_nt_ex(m, n, k, a, b, c, stream, nullptr);
}

const char *gemm_f16_status_string(int status) {
    switch (status) {
        case GEMM_F16_OK: return "ok";
        case GEMM_F16_EINVAL: return "invalid argument (size out of range or bad option)";
        case GEMM_F16_ENULL: return "null pointer with a non-empty extent";
        case GEMM_F16_EALIGN: return "pointer not 2-byte aligned";
        case GEMM_F16_EDEVICE: return "current device is not gfx950 (MI355X)";
        case GEMM_F16_EHIP: return "HIP runtime error or kernel launch failure";
        case GEMM_F16_EOVERLAP: return "c overlaps a or b";
        default: return "unknown status";
    }
}

}  // extern "C"
