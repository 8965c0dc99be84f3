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
//               written to a 2-stage LDS ring.  Buffer descriptors bound
//               each operand tile, so rows past M / N read as zero;
//  * LDS        a stage holds each operand as four 16-wide k planes of
//               32-byte rows; within a row the two 16-byte halves swap by
//               a bit of the row index and planes are padded, so both the
//               MFMA fragment reads and the loader's writes are free of
//               bank conflicts, and every LDS address is one per-lane base
//               register plus an immediate offset;
//  * compute    WM x WN waves (4 or 8), each owning a (BM/WM) x (BN/WN) piece of C
//               as independent 32x32 fp32 accumulators fed by
//               v_mfma_f32_32x32x16_f16; fragment reads run one 16-wide k
//               step ahead of the MFMAs that use them;
//  * epilogue   fp32 -> fp16 round-to-nearest-even, stores masked to
//               [M, N].
//
// The sum of each output runs over K-tiles in increasing order, and inside
// a K-tile over 16-wide k steps in increasing order, whatever the grid
// order: results do not depend on the rasterization options.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <type_traits>

#include "gemm_f16.h"
#include "tile_sched.h"

namespace gemm_f16 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Accumulator block and MFMA for each result-block edge.
template <int MB> struct Mfma;
template <> struct Mfma<32> {
    using Acc = floatx16;
    static __device__ __forceinline__ Acc run(half8 a, half8 b, Acc c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<16> {
    using Acc = floatx4;
    static __device__ __forceinline__ Acc run(half8 a, half8 b, Acc c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};
typedef int int4v __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr uint32_t kOutOfRange = 0x80000000u;  // buffer offset past any num_records: reads 0

#ifndef GEMM_PLANE_PAD
#define GEMM_PLANE_PAD 32
#endif

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

// Block-tile configuration: BM x BN output tile, K walked 64 at a time in
// four 16-wide k steps, WM x WN waves each owning a (BM/WM) x (BN/WN) piece
// of C made of 32x32 MFMA blocks.
template <int BM_, int BN_, int WM_, int WN_, int MB_ = 32>
struct Cfg {
    // MB: edge of the MFMA result block.  32: v_mfma_f32_32x32x16_f16 (k 16
    // per instruction, 16 fp32 results per lane); 16: v_mfma_f32_16x16x32_f16
    // (k 32 per instruction, 4 results per lane).
    static constexpr int MB = MB_, MK = MB_ == 32 ? 16 : 32;
    static constexpr int BM = BM_, BN = BN_, BK = 64, KS = BK / MK;
    static constexpr int kPlanes = BK / 16;  // 16-wide k planes per stage
    static constexpr int WM = WM_, WN = WN_;
    static constexpr int kWaves = WM * WN;
    static constexpr int kThreads = kWaves * kWave;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / MB, FN = TN / MB;
    static constexpr int kRowsPerPass = kThreads / 8;  // 8 chunks of 16 B per 64-wide row
    static constexpr int kMinWavesPerEU = kWaves <= 4 ? 1 : kWaves / 4;
    // LDS: per operand and stage, kPlanes planes of ROWS x 32 B (+ padding).
    static constexpr int kPlaneA = BM * 32 + GEMM_PLANE_PAD;
    static constexpr int kPlaneB = BN * 32 + GEMM_PLANE_PAD;
    static constexpr int kStageA = kPlanes * kPlaneA;
    static constexpr int kStageB = kPlanes * kPlaneB;
    static constexpr int kLdsB = 2 * kStageA;  // B's two stages follow A's
    static constexpr int kLdsBytes = 2 * kStageA + 2 * kStageB;
    static_assert(MB == 32 || MB == 16, "MFMA block edge");
    static_assert(TM % MB == 0 && TN % MB == 0, "wave tile must be whole MFMA blocks");
    static_assert(kRowsPerPass % 32 == 0, "passes must keep row bits 2-4 per lane");
    static_assert(BM % kRowsPerPass == 0 && BN % kRowsPerPass == 0, "loader passes");
    static_assert(kStageA + (kPlanes - 1) * kPlaneA + TM * 32 < 65536 &&
                      kStageB + (kPlanes - 1) * kPlaneB + TN * 32 < 65536,
                  "LDS immediates must fit the 16-bit offset field");
    static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
};

// Which 16-byte half of a 32-byte plane row holds k-half h of row `row`:
// h ^ bit2(row) ^ bit3(row).  A fragment read touches 32 consecutive rows
// at one half; with this swap its ds_read_b128 is free of bank conflicts.
// The loader's 8-lane groups write one row's four planes; a 32-byte plane
// padding staggers those planes across banks so its ds_write_b128 is free
// of conflicts too (64 bytes, or none, costs 8-24 conflict cycles per
// write on gfx950, measured with SQ_LDS_BANK_CONFLICT).
__device__ __forceinline__ int half_swap(int row) { return ((row >> 2) ^ (row >> 3)) & 1; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    // word3 0x00020000: raw (untyped) 32-bit data format, as gfx9-family
    // buffer descriptors expect.
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// LDS barrier that waits only for this wave's LDS traffic (lgkmcnt), not for
// the global loads still in flight for later K-tiles.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One operand's K-tile: ROWS x 64 fp16 = ROWS x 8 chunks of 16 bytes.  Each
// pass of the workgroup covers RPP rows; thread t owns chunk t % 8 of rows
// t / 8 + RPP * i, so every 8 consecutive lanes read one 128-byte row
// segment.
template <int ROWS, int RPP, bool VEC>
struct TileLoader {
    static constexpr int kPasses = ROWS / RPP;
    int4v regs[kPasses];
    uint32_t voff[kPasses];  // VEC: byte offset of this lane's chunk from the K-tile start
    int chunk, row0;

    __device__ __forceinline__ void init(int tid, int k_elems) {
        chunk = tid & 7;
        row0 = tid >> 3;
#pragma unroll
        for (int i = 0; i < kPasses; ++i) voff[i] = (uint32_t)((row0 + RPP * i) * k_elems + chunk * 8) * 2u;
    }

    // VEC: 0, or kOutOfRange when this lane's chunk of the K-tile starting
    // at k0 lies past K (K % 8 == 0 on this path, so a chunk is wholly
    // inside or wholly past K).  Computed once per K-tile.
    __device__ __forceinline__ uint32_t k_mask(int k_elems, int k0) const {
        return (k0 + chunk * 8 >= k_elems) ? kOutOfRange : 0u;
    }

    // VEC: rsrc_tile starts at this K-tile's first column and `mask` (from
    // k_mask) pushes chunks past K out of range, so they read as zero.
    // Scalar: every element is bounds-checked against K and the tile rows.
    __device__ __forceinline__ void load(int i, __amdgpu_buffer_rsrc_t rsrc_tile, uint32_t mask,
                                         __amdgpu_buffer_rsrc_t rsrc0, int k_elems, int k0) {
        if constexpr (VEC) {
            regs[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_tile, voff[i] | mask, 0, 0);
        } else {
            const int row = row0 + RPP * i;
            const int kc = k0 + chunk * 8;
            union {
                short s[8];
                int4v v;
            } u;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t off =
                    (kc + e < k_elems) ? (uint32_t)(row * k_elems + kc + e) * 2u : kOutOfRange;
                u.s[e] = __builtin_amdgcn_raw_buffer_load_b16(rsrc0, off, 0, 0);
            }
            regs[i] = u.v;
        }
    }

    // LDS byte offset of this lane's chunk in pass 0 (plane = chunk / 2).
    template <int PLANE>
    __device__ __forceinline__ int lds_lane_offset() const {
        return (chunk >> 1) * PLANE + row0 * 32 + (((chunk & 1) ^ half_swap(row0)) * 16);
    }
};

template <class C, bool VEC>
__global__ __launch_bounds__(C::kThreads)
__attribute__((amdgpu_waves_per_eu(C::kMinWavesPerEU, C::kMinWavesPerEU)))
void gemm_f16_nt_kernel(const Params p) {
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK, KS = C::KS;
    constexpr int TM = C::TM, TN = C::TN, FM = C::FM, FN = C::FN;
    constexpr int RPP = C::kRowsPerPass;
    using LoaderA = TileLoader<BM, RPP, VEC>;
    using LoaderB = TileLoader<BN, RPP, VEC>;
    constexpr int PA = LoaderA::kPasses, PB = LoaderB::kPasses;
    __shared__ __attribute__((aligned(1024))) char smem[C::kLdsBytes];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave / C::WN;
    const int wn = wave % C::WN;

    const TileCoord tc = tile_coord(blockIdx.x, p.num_m, p.num_n, p.swizzle, p.xcd != 0);
    const int m0 = (int)tc.m_block * BM;
    const int n0 = (int)tc.n_block * BN;

    // Per-tile buffer descriptors: rows past M (N) lie beyond num_records.
    const int rows_a = min(BM, p.m - m0);
    const int rows_b = min(BN, p.n - n0);
    const _Float16 *a_tile = p.a + (int64_t)m0 * p.k;
    const _Float16 *b_tile = p.b + (int64_t)n0 * p.k;
    const uint32_t bytes_a = (uint32_t)rows_a * (uint32_t)p.k * 2u;
    const uint32_t bytes_b = (uint32_t)rows_b * (uint32_t)p.k * 2u;
    const __amdgpu_buffer_rsrc_t ra0 = make_rsrc(a_tile, bytes_a);
    const __amdgpu_buffer_rsrc_t rb0 = make_rsrc(b_tile, bytes_b);
    // Descriptor of K-tile t: starts t*BK columns in and its range shrinks
    // to match; a K-tile at or past K (fetched by the last iterations, never
    // used) gets an empty range, so nothing is read.
    auto rsrc_at = [&](const _Float16 *tile, uint32_t bytes, int t) {
        const uint32_t skip = (uint32_t)t * (BK * 2);
        return make_rsrc(tile + (t < p.k_tiles ? t * BK : 0), (t < p.k_tiles && bytes > skip) ? bytes - skip : 0u);
    };

    LoaderA la;
    LoaderB lb;
    la.init(tid, p.k);
    lb.init(tid, p.k);
    const int wa_lane = la.template lds_lane_offset<C::kPlaneA>();
    const int wb_lane = C::kLdsB + lb.template lds_lane_offset<C::kPlaneB>();

    using M = Mfma<C::MB>;
    typename M::Acc acc[FN][FM];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i) acc[j][i] = typename M::Acc{};

    // Fragment reads.  32x32x16: lane l reads row (wave tile row) + l % 32
    // at k half l / 32 of the step's 16-wide plane.  16x16x32: lane l reads
    // row + l % 16, k eighth l / 16 of the step's 32-wide k range, i.e.
    // plane 2 ks + l / 32, half (l / 16) % 2.  Either way the per-lane part
    // is one register and fragment / step offsets are immediates.
    constexpr int MB = C::MB;
    const int frow = lane % MB;
    const int fhalf = MB == 32 ? (lane >> 5) : ((lane >> 4) & 1);
    const int fplane = MB == 32 ? 0 : (lane >> 5);
    const int ra_lane = fplane * C::kPlaneA + (wm * TM + frow) * 32 + ((fhalf ^ half_swap(frow)) * 16);
    const int rb_lane = C::kLdsB + fplane * C::kPlaneB + (wn * TN + frow) * 32 + ((fhalf ^ half_swap(frow)) * 16);
    constexpr int kPlanesPerStep = C::MK / 16;
    half8 af[2][FM];
    half8 bf[2][FN];
    auto read_frags = [&](int buf, int stage, int ks) {
        // in the order the MFMAs consume them: B0, A0..A(FM-1), B1..
        bf[buf][0] = *reinterpret_cast<const half8 *>(smem + rb_lane + stage * C::kStageB +
                                                      ks * kPlanesPerStep * C::kPlaneB);
#pragma unroll
        for (int i = 0; i < FM; ++i)
            af[buf][i] = *reinterpret_cast<const half8 *>(smem + ra_lane + stage * C::kStageA +
                                                          ks * kPlanesPerStep * C::kPlaneA + i * MB * 32);
#pragma unroll
        for (int j = 1; j < FN; ++j)
            bf[buf][j] = *reinterpret_cast<const half8 *>(smem + rb_lane + stage * C::kStageB +
                                                          ks * kPlanesPerStep * C::kPlaneB + j * MB * 32);
    };
    auto store_a = [&](int i, int stage) {
        *reinterpret_cast<int4v *>(smem + wa_lane + stage * C::kStageA + i * RPP * 32) = la.regs[i];
    };
    auto store_b = [&](int i, int stage) {
        *reinterpret_cast<int4v *>(smem + wb_lane + stage * C::kStageB + i * RPP * 32) = lb.regs[i];
    };

    const int kt_count = p.k_tiles;
    if (kt_count == 0) return;  // never launched with K == 0

    // Prologue: K-tile 0 into stage 0, K-tile 1 (zeros if K has one K-tile)
    // into the staging registers.
    {
        const __amdgpu_buffer_rsrc_t a_t = rsrc_at(a_tile, bytes_a, 0), b_t = rsrc_at(b_tile, bytes_b, 0);
        const uint32_t ma = la.k_mask(p.k, 0), mb = lb.k_mask(p.k, 0);
#pragma unroll
        for (int i = 0; i < PA; ++i) la.load(i, a_t, ma, ra0, p.k, 0);
#pragma unroll
        for (int i = 0; i < PB; ++i) lb.load(i, b_t, mb, rb0, p.k, 0);
#pragma unroll
        for (int i = 0; i < PA; ++i) store_a(i, 0);
#pragma unroll
        for (int i = 0; i < PB; ++i) store_b(i, 0);
    }
    {
        const __amdgpu_buffer_rsrc_t a_t = rsrc_at(a_tile, bytes_a, 1), b_t = rsrc_at(b_tile, bytes_b, 1);
        const uint32_t ma = la.k_mask(p.k, BK), mb = lb.k_mask(p.k, BK);
#pragma unroll
        for (int i = 0; i < PA; ++i) la.load(i, a_t, ma, ra0, p.k, BK);
#pragma unroll
        for (int i = 0; i < PB; ++i) lb.load(i, b_t, mb, rb0, p.k, BK);
    }
    lds_barrier();
    read_frags(0, 0, 0);

    // One K-tile of work, as KS k steps (MK wide) on stage STAGE, which also
    // moves the staged K-tile kt+1 into the other stage and refills the
    // staging registers with K-tile kt+2.  Past the last K-tile those moves
    // carry zeros that are never read, so every iteration is the same
    // branch-free block, whose issue order is pinned:
    //   step ks < KS-1: MFMAs of step ks interleaved with the fragment reads
    //                   for step ks+1 and a slice of the LDS writes and
    //                   global loads;
    //   step KS-1:      wait for this wave's LDS traffic, workgroup barrier,
    //                   then MFMAs of step KS-1 interleaved with the
    //                   fragment reads for step 0 of K-tile kt+1.
    constexpr int kSlices = KS - 1;
    auto k_iter = [&](auto stage_tag, int kt) {
        constexpr int STAGE = decltype(stage_tag)::value;
        constexpr int NXT = STAGE ^ 1;
        const int k_load = (kt + 2) * BK;
        const __amdgpu_buffer_rsrc_t a_t = rsrc_at(a_tile, bytes_a, kt + 2);
        const __amdgpu_buffer_rsrc_t b_t = rsrc_at(b_tile, bytes_b, kt + 2);
        const uint32_t ma = la.k_mask(p.k, k_load), mb = lb.k_mask(p.k, k_load);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int cur = ks & 1;
            constexpr int NM = FM * FN;
            if (ks + 1 < KS) {
                read_frags(cur ^ 1, STAGE, ks + 1);
            } else {
                // The other stage is complete for everyone, and everyone has
                // read its last fragments of this stage.
                lds_barrier();
                read_frags(cur ^ 1, NXT, 0);
            }
            if (ks < kSlices) {
#pragma unroll
                for (int i = ks * PA / kSlices; i < (ks + 1) * PA / kSlices; ++i) {
                    store_a(i, NXT);
                    la.load(i, a_t, ma, ra0, p.k, k_load);
                }
#pragma unroll
                for (int i = ks * PB / kSlices; i < (ks + 1) * PB / kSlices; ++i) {
                    store_b(i, NXT);
                    lb.load(i, b_t, mb, rb0, p.k, k_load);
                }
            }
            // B rows feed the MFMA's A operand and A rows its B operand, so
            // each 32x32 result block is C^T: a lane then holds 4
            // consecutive n of one m row, which stores as 8 bytes.
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int i = 0; i < FM; ++i) acc[j][i] = M::run(bf[cur][j], af[cur][i], acc[j][i]);
            // Pin the issue order: after each MFMA, an even share of this
            // step's other memory instructions (fragment reads first, then
            // LDS write / global load pairs).
            {
                const int nr = FM + FN;
                const int nw = ks < kSlices ? ((ks + 1) * PA / kSlices - ks * PA / kSlices) +
                                                  ((ks + 1) * PB / kSlices - ks * PB / kSlices)
                                            : 0;
                const int total = nr + 2 * nw;
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
#pragma unroll
                    for (int o = m * total / NM; o < (m + 1) * total / NM; ++o) {
                        if (o < nr) {
                            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
                        } else if (((o - nr) & 1) == 0) {
                            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
                        } else {
                            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
                        }
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    // K-tiles go in pairs (stage 0, stage 1) with no branch between them.
    // When the count is odd the last pair's second K-tile lies past K: its
    // stage holds zeros, so its MFMAs add +0 to accumulators that are never
    // -0 (they start at +0), which leaves every bit unchanged.
    for (int kt = 0; kt < kt_count; kt += 2) {
        k_iter(S0{}, kt);
        k_iter(S1{}, kt + 1);
    }

    // Epilogue.  MFMA result layout: for 32x32 blocks, lane l register r
    // holds row 8*(r/4) + 4*(l/32) + r%4, column l%32; for 16x16 blocks,
    // row 4*(l/16) + r, column l%16.  With the swapped operands the row is n
    // and the column is m, so each group of 4 registers is 4 consecutive n.
    constexpr int kGroups = MB == 32 ? 4 : 1;
    const int quad = MB == 32 ? (lane >> 5) * 4 : (lane >> 4) * 4;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * TM + i * MB + frow;
        if (m >= p.m) continue;
        _Float16 *crow = p.c + (int64_t)m * p.n;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int g = 0; g < kGroups; ++g) {
                const int n = n0 + wn * TN + j * MB + 8 * g + quad;
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

using Cfg256 = Cfg<256, 256, 2, 2>;   // 4 waves, 128x128 each
using Cfg256w8 = Cfg<256, 256, 4, 2>; // 8 waves, 64x128 each
using Cfg256x128 = Cfg<256, 128, 2, 2>;
using Cfg128x256 = Cfg<128, 256, 2, 2>;
using Cfg128 = Cfg<128, 128, 2, 2>;
using Cfg128m16 = Cfg<128, 128, 2, 2, 16>;  // v_mfma_f32_16x16x32_f16
using Cfg64 = Cfg<64, 64, 2, 2>;

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
        default: return {64, 64};
    }
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int kNumCU = 256;

// Automatic block tile: the candidate with the best modelled throughput,
// (work per launch) / (rounds of 256 workgroups x per-tile efficiency).  A
// round is one workgroup per CU; the efficiency factors are relative
// per-CU throughputs of the tile shapes measured on MI355X (the bigger the
// tile, the fewer LDS and L2 bytes per flop).
static int auto_tile(int64_t m, int64_t n) {
    struct Cand {
        int id, bm, bn;
        double eff;
    };
    static const Cand cands[] = {
        {GEMM_F16_TILE_256x256, 256, 256, 1.00},
        {GEMM_F16_TILE_256x128, 256, 128, 0.90},
        {GEMM_F16_TILE_128x256, 128, 256, 0.90},
        {GEMM_F16_TILE_128x128, 128, 128, 0.75},
        {GEMM_F16_TILE_64x64, 64, 64, 0.35},
    };
    int best = GEMM_F16_TILE_64x64;
    double best_t = 1e300;
    for (const Cand &c : cands) {
        const int64_t tiles = cdiv(m, c.bm) * cdiv(n, c.bn);
        const int64_t rounds = cdiv(tiles, kNumCU);
        // time ~ rounds * (tile flops) / eff; tile flops ~ bm * bn
        const double t = (double)rounds * c.bm * c.bn / c.eff;
        if (t < best_t * 0.999) {
            best_t = t;
            best = c.id;
        }
    }
    return best;
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

template <class C>
static void launch(const Params &p, bool vec, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)p.num_m * p.num_n));
    if (vec)
        hipLaunchKernelGGL((gemm_f16_nt_kernel<C, true>), grid, dim3(C::kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((gemm_f16_nt_kernel<C, false>), grid, dim3(C::kThreads), 0, stream, p);
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
    if (o.tile < 0 || o.tile > GEMM_F16_TILE_LAST || o.swizzle < 0 || o.xcd < -1 || o.xcd > 1)
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
        case GEMM_F16_TILE_256x256: launch<Cfg256>(p, vec, s); break;
        case GEMM_F16_TILE_256x256_W8: launch<Cfg256w8>(p, vec, s); break;
        case GEMM_F16_TILE_256x128: launch<Cfg256x128>(p, vec, s); break;
        case GEMM_F16_TILE_128x256: launch<Cfg128x256>(p, vec, s); break;
        case GEMM_F16_TILE_128x128: launch<Cfg128>(p, vec, s); break;
        case GEMM_F16_TILE_128x128_M16: launch<Cfg128m16>(p, vec, s); break;
        default: launch<Cfg64>(p, vec, s); break;
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
