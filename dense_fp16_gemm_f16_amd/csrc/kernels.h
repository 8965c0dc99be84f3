// libgemm_f16: C = fp16(A * B^T), fp16 inputs, fp32 accumulation, for gfx950:
// the device code and the per-tile launch logic (instantiated per block tile
// in tile_*.hip and ring_*.hip).
//
// The operation is the one the Tilus tutorial "1. WGMMA: Hopper's
// Asynchronous Tensor Core" builds in "The Full Kernel": A is [M,K], B is
// [N,K], the fp32 accumulator starts at zero, the block tile walks K in
// block_k steps, and the accumulator is cast to fp16 and stored at the
// block's (m, n) offset.  The mechanism here is CDNA4's, not Hopper's:
//
//  * scheduler  a 1D grid, XCD-aware and swizzle-rasterized (tile_sched.h):
//               one workgroup per block tile, or, with more tiles than
//               CUs, one per CU walking tiles blockIdx.x, + gridDim.x, ...
//  * loader     for C = A B^T with K % 8 == 0 and 16-byte aligned operands,
//               buffer_load_dwordx4 ... lds straight into a 2-stage LDS ring
//               (KMajorDirect: 1 KB = 8 rows of 128 bytes per wave
//               instruction; lanes past K get an out-of-range offset and
//               land as zeros).  Otherwise 16-byte loads at 4-byte aligned
//               offsets (shifted into place on 2-byte aligned rows) staged
//               in VGPRs one K-tile ahead (KMajorOperand).  Buffer descriptors
//               bound each operand tile, so rows past M / N read as zero;
//  * LDS        direct path: 128-byte rows with the 16-byte chunks
//               swizzled by the row index, conflict-free fragment reads;
//               register-staged path: four 16-wide k planes of 32-byte
//               rows.  Every LDS address is one per-lane base register plus
//               an immediate offset;
//  * compute    4 waves in a 2 x 2 grid (8 on one tile), each owning a
//               (BM/WM) x (BN/WN) piece of C: v_mfma_f32_16x16x32_f16 with
//               the accumulators tied in AGPRs (inline asm) on the direct
//               path, v_mfma_f32_32x32x16_f16 on the register-staged one.
//               The fragments of K-tile t+1 are read during K-tile t
//               (gemm_f16_direct_ahead_kernel), behind a release and an
//               acquire barrier per K-tile;
//  * epilogue   fp32 -> fp16 round-to-nearest-even (or the fp32 value
//               itself), masked to [M, N]: staged through LDS so that 16
//               consecutive lanes store one contiguous row segment, or, in
//               gemm_f16_stream_kernel, stored straight from the
//               accumulators under the next tile's first MFMAs.
//
// The sum of each output runs over K-tiles in increasing order, and inside
// a K-tile over its k steps in increasing order, whatever the grid order:
// results do not depend on the rasterization options.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <type_traits>

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

// v_mfma_f32_16x16x32_f16 with the accumulator tied to itself in AGPRs.  The
// builtin's form lets the destination differ from srcC, and with 64
// accumulator blocks per wave the register allocator then rotates them
// through the AGPRs, with ~240 accumulator copies per K-loop iteration
// (measured in an LDS-fed MFMA loop on gfx950: 1403 TFLOP/s with the
// builtin, 1770 tied, uniform[-1,1] operands).  The compiler sees no MFMA in
// the asm, so it inserts no MFMA wait states for it: the kernel fences the
// accumulators itself (acc_fence) before the first and after the last one.
__device__ __forceinline__ void mfma16_tied(half8 a, half8 b, floatx4 &c) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

constexpr int kWave = 64;
constexpr uint32_t kOutOfRange = 0x80000000u;  // buffer offset past any num_records: reads 0

#ifndef GEMM_PLANE_PAD
#define GEMM_PLANE_PAD 32
#endif
// MFMA of the last k step after which the K-tile's workgroup barrier sits
// (a few MFMAs in, the wave's last fragment reads of the stage are done)
#ifndef GEMM_BAR_MFMA
#define GEMM_BAR_MFMA 2
#endif
// 1: the C = A B^T 16-byte path (K % 8 == 0, 16-byte aligned operands)
// loads straight into LDS (gemm_f16_direct_kernel, _ahead_kernel)
#ifndef GEMM_DIRECT
#define GEMM_DIRECT 1
#endif
// sixteenths of a K-tile's direct-to-LDS loads issued during step 0 of the
// following K-tile rather than right after the barrier
// (32x32x16 tiles, four 16-wide k steps per K-tile; the _M16 values are for
// 16x16x32 tiles, two 32-wide k steps)
#ifndef GEMM_DIRECT_TAIL
#define GEMM_DIRECT_TAIL 10
#endif
#ifndef GEMM_DIRECT_TAIL_M16
#define GEMM_DIRECT_TAIL_M16 4
#endif
// k steps of the following K-tile those loads are spread over
#ifndef GEMM_DIRECT_TAIL_STEPS
#define GEMM_DIRECT_TAIL_STEPS 2
#endif
// MFMA of the last k step after which the direct kernel's barrier sits
#ifndef GEMM_DIRECT_BAR_MFMA
#define GEMM_DIRECT_BAR_MFMA 1
#endif
#ifndef GEMM_DIRECT_BAR_MFMA_M16
#define GEMM_DIRECT_BAR_MFMA_M16 4
#endif
// 1: 16x16x32 direct-to-LDS tiles read fragments a K-tile ahead with two
// barriers per K-tile (gemm_f16_direct_ahead_kernel)
#ifndef GEMM_AHEAD
#define GEMM_AHEAD 1
#endif
#ifndef GEMM_AHEAD_REL_MFMA
#define GEMM_AHEAD_REL_MFMA 4
#endif
#ifndef GEMM_AHEAD_ACQ_MFMA
#define GEMM_AHEAD_ACQ_MFMA 4
#endif
// 1: more tiles than CUs -> one workgroup per CU walking several tiles
#ifndef GEMM_PERSIST
#define GEMM_PERSIST 1
#endif
// 1: C = A B^T's one-workgroup-per-CU kernel stores each tile's C under the
// MFMAs around the tile change (gemm_f16_stream_kernel)
#ifndef GEMM_STREAM
#define GEMM_STREAM 1
#endif
// 0: the stream kernel's store units run i (row block) fastest; 1: p
// (column pair) fastest, the two halves of a C line back to back
#ifndef GEMM_UNIT_P_FAST
#define GEMM_UNIT_P_FAST 0
#endif
// 1: the stream kernel's stores carry the streaming hint where the host
// asks for it (kStoreStream); 0: the default policy there instead
#ifndef GEMM_STREAM_NT
#define GEMM_STREAM_NT 1
#endif
// 1: the one-workgroup-per-CU kernels (stream, persistent) also serve
// K % 64 != 0 (a partial last K-tile per tile) and an odd K-tile count;
// 0: those shapes take one workgroup per tile
#ifndef GEMM_PARTIAL_K
#define GEMM_PARTIAL_K 1
#endif
// sixteenths of a K-tile's loads issued in step 0 (the rest in step 1)
#ifndef GEMM_AHEAD_STEP0_LOADS
#define GEMM_AHEAD_STEP0_LOADS 10
#endif
// staging register sets (1 or 2; a second set prefetches one more K-tile)
#ifndef GEMM_STAGE_SETS
#define GEMM_STAGE_SETS 1
#endif

// LDS poisoning (built only with -DGEMM_F16_POISON_LDS, a debug build of
// the library, never the library itself): every kernel fills its LDS with
// fp16 NaN (0x7E00) before its first load, and waits for it, so an MFMA
// operand read from LDS that no load (or zero-filling out-of-range load)
// has written turns its outputs into NaN, which the parity tests catch.
#ifdef GEMM_F16_POISON_LDS
__device__ __forceinline__ void poison_lds(char *smem, int bytes) {
    typedef int int4p __attribute__((ext_vector_type(4)));
    const int4p nan = {0x7E007E00, 0x7E007E00, 0x7E007E00, 0x7E007E00};
    for (int o = (int)threadIdx.x * 16; o < bytes; o += (int)blockDim.x * 16)
        *reinterpret_cast<int4p *>(smem + o) = nan;
    __syncthreads();
}
#define GEMM_POISON_LDS(smem) poison_lds(smem, (int)sizeof(smem))
#else
#define GEMM_POISON_LDS(smem)
#endif

// Timestamp trace (built only with -DGEMM_F16_TRACE, a profiling build of
// the library, never the library itself): the fragment-ahead and stream
// kernels record per wave, in this translation unit's copy of gemm_trace,
// the shader-clock counter (s_memtime) at their start, after the prologue's
// wait, after the K loop and after their last store has completed, the
// 100 MHz counter (s_memrealtime) at start and end, the cycles spent in the
// release and acquire barriers of the K loop, and the XCC and HW_ID
// registers; the stream kernel also the start of each of its first four
// tiles and, with -DGEMM_F16_TRACE_KTILES as well, of K-tiles kt-1 of its
// first tile and 0, 1 and 2 of its second (the first tile change; the low
// 32 bits of the counter; these take scalar registers that the K loop
// then spills to vector lanes).
// Slots of 24 words per wave, wave w of workgroup b at (4 b + w) * 24;
// workgroups past kTraceBlocks and waves past the fourth record nothing.
#ifdef GEMM_F16_TRACE
constexpr int kTraceBlocks = 2048, kTraceWords = 24;
static __device__ unsigned long long gemm_trace[kTraceBlocks * 4 * kTraceWords];
__device__ __forceinline__ uint64_t trace_clock() { return __builtin_amdgcn_s_memtime(); }
__device__ __forceinline__ uint64_t trace_realtime() { return __builtin_amdgcn_s_memrealtime(); }
struct TraceRecord {
    uint64_t t0 = 0, t1 = 0, rel = 0, acq = 0, acq_first = 0, tl = 0, r0 = 0, tiles = 0;
    uint64_t tile_start[4] = {0, 0, 0, 0};
#ifdef GEMM_F16_TRACE_KTILES
    // around the first tile change: the counter's low 32 bits (differences
    // of these are exact modulo 2^32)
    uint32_t kt_last = 0, kt0 = 0, kt1 = 0, kt2 = 0;
#endif
};
__device__ __forceinline__ void trace_write(const TraceRecord &r, int wave, int lane) {
    const uint64_t te = trace_clock(), re = trace_realtime();
    if (lane != 0 || wave >= 4 || blockIdx.x >= (unsigned)kTraceBlocks) return;
    unsigned long long *q = gemm_trace + ((size_t)blockIdx.x * 4 + wave) * kTraceWords;
    q[0] = r.t0;
    q[1] = r.t1;
    q[2] = r.rel;
    q[3] = r.acq;
    q[4] = r.acq_first;
    q[5] = r.tl;
    q[6] = te;
    q[7] = r.r0;
    q[8] = re;
    q[9] = r.tiles;
#pragma unroll
    for (int i = 0; i < 4; ++i) q[10 + i] = r.tile_start[i];
    q[14] = 0;
    q[15] = 0;
    q[16] = (unsigned)__builtin_amdgcn_s_getreg(20 | (3 << 11));  // XCC_ID[3:0]
    q[17] = (unsigned)__builtin_amdgcn_s_getreg(4 | (31 << 11));  // HW_ID
    q[18] = 0;
    q[19] = 0;
#ifdef GEMM_F16_TRACE_KTILES
    q[20] = r.kt_last;
    q[21] = r.kt0;
    q[22] = r.kt1;
    q[23] = r.kt2;
#else
    q[20] = q[21] = q[22] = q[23] = 0;
#endif
}
#define GEMM_TRACE_DO(...) __VA_ARGS__
#else
#define GEMM_TRACE_DO(...)
#endif

struct Params {
    const _Float16 *a;
    const _Float16 *b;
    void *c;               // fp16 C (NT) or fp32 D (NN)
    int32_t m, n, k;
    int32_t num_m, num_n;  // block tiles along M and N
    int32_t k_tiles;       // ceil(k / BK)
    int32_t swizzle;
    int32_t xcd;
    int32_t c_store;       // cache policy of the 16-byte C stores (CStore)
};

// Cache policy of the 16-byte C stores, decided by the host per call:
//   kStoreDevice  device scope (sc1): written through the XCD's L2 to the
//                 memory side, where the 256 MiB Infinity Cache takes the
//                 store bursts; chosen while A, B and C fit in it;
//   kStoreStream  streaming (nt): C lines do not displace the A and B lines
//                 that other workgroups of the XCD still read; for rows of
//                 whole 128-byte lines (rows ending inside a line measured
//                 slower with it);
//   kStoreDefault otherwise.
enum CStore : int32_t { kStoreDefault = 0, kStoreStream = 1, kStoreDevice = 2 };

// The cache-policy operand of a buffer store for a CStore (nt = bit 1,
// sc1 = bit 4).
__host__ __device__ constexpr int store_aux(int pol) {
    return pol == kStoreStream ? 2 : pol == kStoreDevice ? 16 : 0;
}

// A 16-byte global store at device scope (sc1).  No builtin carries the
// scope bits on a global store, hence the asm.
__device__ __forceinline__ void store_device_scope(void *dst, int4v v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(dst), "v"(v) : "memory");
}

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
    // staging register sets: with two, the loads of a K-tile are issued two
    // K-tiles before it is written to LDS.  Measured on gfx950 a second set
    // buys nothing (the loads are throughput-, not latency-bound), so the
    // default is one.
    static constexpr int kSets = GEMM_STAGE_SETS;
    static_assert(MB == 32 || MB == 16, "MFMA block edge");
    static_assert(TM % MB == 0 && TN % MB == 0, "wave tile must be whole MFMA blocks");
    static_assert(kRowsPerPass % 32 == 0, "passes must keep row bits 2-4 per lane");
};

// Which 16-byte half of a 32-byte plane row holds k-half h of row `row`:
// h ^ bit2(row) ^ bit3(row).  A fragment read touches 32 consecutive rows
// at one half; with this swap its ds_read_b128 is free of bank conflicts.
// The loader's 8-lane groups write one row's four planes; a 32-byte plane
// padding staggers those planes across banks so its ds_write_b128 is free
// of conflicts too (64 bytes, or none, costs 8-24 conflict cycles per
// write on gfx950, measured with SQ_LDS_BANK_CONFLICT).
__device__ __forceinline__ int half_swap(int row) { return ((row >> 2) ^ (row >> 3)) & 1; }

// Buffer descriptor (base, num_records).  Both are wave-uniform by
// construction; readfirstlane states it, so the descriptor lives in SGPRs
// and the loads need no per-lane loop over distinct descriptors.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    const uint64_t addr = (uint64_t)(uintptr_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    void *b = (void *)(uintptr_t)(((uint64_t)hi << 32) | lo);
    // word3 0x00020000: raw (untyped) 32-bit data format, as gfx9-family
    // buffer descriptors expect.
    return __builtin_amdgcn_make_buffer_rsrc(b, (short)0, (int)n, 0x00020000);
}

// LDS barrier that waits only for this wave's LDS traffic (lgkmcnt), not for
// the global loads still in flight for later K-tiles.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---- operands ---------------------------------------------------------------
//
// Both operand kinds share one interface, used by the K loop below:
//   init(...)          per-lane offsets, descriptors of the block tile
//   begin_tile(t)      descriptor (and lane mask) for K-tile t; a K-tile at
//                      or past K gets an empty range, so it reads zeros
//   load(i)            global -> staging registers, pass i of kPasses
//   store(smem, i, s)  staging registers -> LDS stage s, pass i
//   read(smem, s, ks, f)  MFMA fragment f of 16-wide k step ks from stage s:
//                      8 fp16 per lane, lane l holding k 8*(l/32)..+7 of
//                      row or column f*32 + l%32 (32x32x16), or k
//                      8*(l/16)..+7 of row f*16 + l%16 (16x16x32)

// Operand stored [rows, K] row-major in HBM: A, and B of the NT contract.
// LDS stage: kPlanes k planes of ROWS x 32 bytes (16 k per row) plus
// GEMM_PLANE_PAD bytes.  Each pass of the workgroup covers RPP rows of the
// K-tile (ROWS x 64 fp16 = ROWS x 8 chunks of 16 bytes); thread t owns
// chunk t % 8 of rows t / 8 + RPP * i, so every 8 consecutive lanes read one
// 128-byte row segment.  G says how the rows are aligned:
//   8: 16-byte aligned rows (K % 8 == 0): one 16-byte load per chunk;
//   2: 4-byte aligned rows (K even): one 16-byte load per chunk at a 4-byte
//      aligned offset;
//   1: 2-byte aligned rows (any K): the chunk's 16 bytes start 0 or 2 bytes
//      into a 4-byte aligned dword; a 16-byte load from there plus the dword
//      after it, shifted by those 0 or 2 bytes.
// With G < 8 a chunk can straddle K, and the bytes past K belong to the next
// row, so the elements past K are masked to zero on their way into LDS.
template <class C, int ROWS, int WROWS, int G, bool KFULL, int SETS>
struct KMajorOperand {
    static constexpr bool VEC = G == 8;
    static constexpr bool SHIFT = G == 1;
    static_assert(G == 8 || G == 2 || G == 1, "row alignment");
    static_assert(VEC || (SETS == 1 && !KFULL), "G < 8: one staging set, K-tiles masked against K");
    static constexpr int RPP = C::kRowsPerPass;
    static constexpr int kPasses = ROWS / RPP;
    static constexpr int kPlane = ROWS * 32 + GEMM_PLANE_PAD;
    static constexpr int kStage = C::kPlanes * kPlane;
    static constexpr int kLdsBytes = 2 * kStage;
    static constexpr int kPlanesPerStep = C::MK / 16;
    static_assert(ROWS % RPP == 0, "loader passes");
    // every pass moves a lane RPP rows on: an even number of rows keeps a
    // lane's chunks at one offset modulo 4 bytes whatever K is
    static_assert(RPP % 2 == 0, "rows per pass");
    // WROWS: rows of this operand one wave reads fragments from; the read
    // immediates reach stage + last plane + last fragment of the wave.
    static_assert(kStage + (C::kPlanes - 1) * kPlane + (WROWS - C::MB) * 32 < 65536,
                  "LDS immediates must fit the 16-bit offset field");

    int4v regs[SETS][kPasses];
    uint32_t next[SHIFT ? kPasses : 1];  // G == 1: the dword after each chunk's 16-byte load
    uint32_t voff[kPasses];  // byte offset of this lane's chunk (G < 8: of its 4-byte aligned start)
    int chunk, row0, k_elems, k_tiles;
    const char *tile;  // first row of the block tile (G < 8: rounded down to 4 bytes)
    uint32_t bytes;    // the block's rows (G < 8: from the rounded-down start, whole dwords)
    __amdgpu_buffer_rsrc_t rsrc0, rsrc_t, rsrc_none;
    uint32_t mask;     // G == 8, K % 64 != 0: the chunk past K
    uint32_t soff;     // KFULL: byte offset of the K-tile inside each row
    uint32_t shift;    // G == 1: bytes between the dword start and the chunk, 0 or 2
    int kvalid[2];     // G < 8: elements of the chunk inside K, for the K-tile of each LDS stage
    int k0;
    int w_lane, r_lane;

    // base: first row of the block tile; rows_valid: rows of it inside the
    // matrix; frag_row: first row this wave reads fragments from; lds: byte
    // offset of this operand's two stages.
    __device__ __forceinline__ void init(const _Float16 *base, int rows_valid, int K, int kt_count, int tid,
                                         int lane, int frag_row, int lds) {
        chunk = tid & 7;
        row0 = tid >> 3;
        k_elems = K;
        k_tiles = kt_count;
        if constexpr (VEC) {
            tile = reinterpret_cast<const char *>(base);
            bytes = (uint32_t)rows_valid * (uint32_t)K * 2u;
#pragma unroll
            for (int i = 0; i < kPasses; ++i) voff[i] = (uint32_t)((row0 + RPP * i) * K + chunk * 8) * 2u;
        } else {
            // The descriptor starts at the dword holding the block's first
            // element and ends with the dword holding its last one: a load
            // returns a dword only when all 4 of its bytes are in range, and
            // the dword holding an element lies in that element's page, so
            // the 2 bytes past the matrix it may hold are mapped.  Rows past
            // rows_valid get kOutOfRange and read zeros, as on the other
            // paths.
            const uint32_t lead = (uint32_t)((uintptr_t)base & 3u);  // 0, or 2 with G == 1
            tile = reinterpret_cast<const char *>(base) - lead;
            bytes = ((uint32_t)rows_valid * (uint32_t)K * 2u + lead + 3u) & ~3u;
            shift = ((uint32_t)row0 * (uint32_t)K * 2u + lead) & 2u;
#pragma unroll
            for (int i = 0; i < kPasses; ++i) {
                const int row = row0 + RPP * i;
                voff[i] = row < rows_valid ? (uint32_t)(row * K + chunk * 8) * 2u + lead - shift : kOutOfRange;
            }
        }
        rsrc0 = make_rsrc(tile, bytes);
        rsrc_none = make_rsrc(tile, 0u);
        w_lane = lds + (chunk >> 1) * kPlane + row0 * 32 + (((chunk & 1) ^ half_swap(row0)) * 16);
        // fragment reads: 32x32x16 lane l takes row l % 32, k half l / 32 of
        // the step's plane; 16x16x32 lane l takes row l % 16, plane 2 ks +
        // l / 32, half (l / 16) % 2.
        const int frow = lane % C::MB;
        const int fhalf = C::MB == 32 ? (lane >> 5) : ((lane >> 4) & 1);
        const int fplane = C::MB == 32 ? 0 : (lane >> 5);
        r_lane = lds + fplane * kPlane + (frag_row + frow) * 32 + ((fhalf ^ half_swap(frow)) * 16);
    }

    // KFULL (K % BK == 0, VEC): the block's descriptor for every K-tile,
    // the K-tile's byte offset in soffset, and an empty descriptor for the
    // K-tiles past K.  Otherwise a descriptor per K-tile whose range ends
    // with the block's last row, and reads past the last K-tile get an
    // empty range.  With G == 8 (K % 8 == 0) a chunk is wholly inside or
    // wholly past K, and the chunks past K get kOutOfRange; with G < 8 the
    // store masks each chunk against K.  All of these read zeros wherever
    // the tile leaves the matrix.
    __device__ __forceinline__ void begin_tile(int t) {
        k0 = t * C::BK;
        if constexpr (VEC && KFULL) {
            rsrc_t = t < k_tiles ? rsrc0 : rsrc_none;
            soff = (uint32_t)k0 * 2u;
            mask = 0;
        } else {
            const uint32_t skip = (uint32_t)t * (C::BK * 2);
            const bool live = t < k_tiles;
            rsrc_t = make_rsrc(tile + (live ? skip : 0u), (live && bytes > skip) ? bytes - skip : 0u);
            soff = 0;
            mask = (k0 + chunk * 8 >= k_elems) ? kOutOfRange : 0u;
            // With one staging set, K-tile t is stored into LDS stage t % 2,
            // after begin_tile(t) and before begin_tile(t + 2).
            if constexpr (!VEC) kvalid[t & 1] = k_elems - (k0 + chunk * 8);
        }
    }

    __device__ __forceinline__ void load(int i, int set) {
        if constexpr (VEC) {
            if constexpr (KFULL)
                regs[set][i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_t, voff[i], soff, 0);
            else
                regs[set][i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_t, voff[i] | mask, 0, 0);
        } else {
            regs[set][i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_t, voff[i], 0, 0);
            if constexpr (SHIFT) next[i] = __builtin_amdgcn_raw_buffer_load_b32(rsrc_t, voff[i] + 16u, 0, 0);
        }
    }

    __device__ __forceinline__ void store(char *smem, int i, int stage, int set) const {
        int4v v = regs[set][i];
        if constexpr (!VEC) {
            if constexpr (SHIFT) {
                const uint32_t w4 = next[i];
                v = int4v{(int)__builtin_amdgcn_alignbyte((uint32_t)v[1], (uint32_t)v[0], shift),
                          (int)__builtin_amdgcn_alignbyte((uint32_t)v[2], (uint32_t)v[1], shift),
                          (int)__builtin_amdgcn_alignbyte((uint32_t)v[3], (uint32_t)v[2], shift),
                          (int)__builtin_amdgcn_alignbyte(w4, (uint32_t)v[3], shift)};
            }
            // element e of the chunk is kept when e < kv (fp16 e sits in
            // the low half of dword e / 2 when e is even)
            const int kv = stage ? kvalid[1] : kvalid[0];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[j] &= (kv > 2 * j + 1) ? -1 : (kv > 2 * j) ? 0xffff : 0;
        }
        *reinterpret_cast<int4v *>(smem + w_lane + stage * kStage + i * RPP * 32) = v;
    }

    __device__ __forceinline__ half8 read(const char *smem, int stage, int ks, int f) const {
        return *reinterpret_cast<const half8 *>(smem + r_lane + stage * kStage +
                                                ks * kPlanesPerStep * kPlane + f * C::MB * 32);
    }
};

// B of the second contract, stored [K, N] row-major in HBM (the layout of
// the day-78 listing "wgmma_gemm.cu").  LDS stage: the K-tile as 64 rows of
// BN fp16 (n contiguous), each row padded by 64 bytes.  A 32x32x16 fragment
// needs 8 consecutive k of one column per lane; two ds_read_b64_tr_b16 give
// exactly that: within each 16-lane group, lane j reads 4 consecutive n of
// k-row j/4 and the hardware hands lane i the 4 k values of column i.  With
// the 64-byte row padding the 4 k-rows of a group and the two groups of a
// half-wave fall on disjoint banks.  Each pass covers RPP k-rows; thread t
// owns 16-byte chunk t % (BN/8) of k-row t / (BN/8) + RPP * i, so
// consecutive lanes read consecutive n (coalesced).
// VEC: N % 8 == 0 and a 16-byte aligned B, one 16-byte load per chunk.
// Otherwise the k-rows are 2-byte aligned: as in KMajorOperand with G == 1,
// a 16-byte load at the 4-byte aligned offset below the chunk and the dword
// after it, shifted into place.  The elements of a chunk past N are left as
// they come (the next k-row's): column n of B reaches only column n of D,
// and D's columns past N are never stored.  k-rows past K are zeroed.
template <class C, bool VEC, int SETS>
struct NMajorB {
    static constexpr int BN = C::BN, BK = C::BK;
    static constexpr int kCpr = BN / 8;  // 16-byte chunks per k-row
    static constexpr int RPP = C::kThreads / kCpr;
    static constexpr int kPasses = BK / RPP;
    static constexpr int kPitch = BN * 2 + 64;
    static constexpr int kStage = BK * kPitch;
    static constexpr int kLdsBytes = 2 * kStage;
    static_assert(C::MB == 32, "the transposed B path feeds 32x32x16 MFMAs");
    static_assert(C::kThreads % kCpr == 0 && BK % RPP == 0, "loader passes");
    static_assert(15 * kPitch + 4 * kPitch + BN * 2 < 65536, "LDS immediates");
    static_assert(VEC || SETS == 1, "unaligned rows: one staging set, k-rows masked against K");
    // an even number of k-rows per pass keeps a lane's chunks at one offset
    // modulo 4 bytes whatever N is
    static_assert(RPP % 2 == 0, "rows per pass");

    int4v regs[SETS][kPasses];
    uint32_t next[VEC ? 1 : kPasses];  // !VEC: the dword after each chunk's 16-byte load
    // byte offset from the K-tile's first row (!VEC: of the 4-byte aligned
    // start); VEC: bit 31 set past N
    uint32_t voff[kPasses];
    int chunk, row0, n_total, k_elems, k_tiles, n0;
    const char *b;     // !VEC: rounded down to 4 bytes
    uint32_t lead;     // bytes b was rounded down by
    uint32_t shift;    // !VEC: bytes between the dword start and the chunk, 0 or 2
    int krows[2];      // !VEC: k-rows inside K of the K-tile of each LDS stage
    __amdgpu_buffer_rsrc_t rsrc_t;
    int k0;
    int w_lane, r_lane[2];

    __device__ __forceinline__ void init(const _Float16 *bmat, int n_first, int N, int K, int kt_count, int tid,
                                         int lane, int frag_col, int lds) {
        chunk = tid % kCpr;
        row0 = tid / kCpr;
        n_total = N;
        k_elems = K;
        k_tiles = kt_count;
        n0 = n_first;
        if constexpr (VEC) {
            lead = 0;
            const uint32_t col_mask = (n0 + chunk * 8 >= N) ? kOutOfRange : 0u;  // N % 8 == 0
#pragma unroll
            for (int i = 0; i < kPasses; ++i)
                voff[i] = ((uint32_t)((row0 + RPP * i) * N + n0 + chunk * 8) * 2u) | col_mask;
        } else {
            // A chunk wholly past N reads the block's first chunk instead:
            // its columns are never stored.  Then every offset is below
            // 64 * N * 2 + 20 < 2^32 (N < 2^25), and a multiple of 4: the
            // chunk's column is a multiple of 8, and RPP is even.
            lead = (uint32_t)((uintptr_t)bmat & 3u);
            shift = ((uint32_t)row0 * (uint32_t)N * 2u + lead) & 2u;
            const int nc = n0 + chunk * 8 < N ? n0 + chunk * 8 : n0;
#pragma unroll
            for (int i = 0; i < kPasses; ++i)
                voff[i] = (uint32_t)((row0 + RPP * i) * N + nc) * 2u + lead - shift;
        }
        b = reinterpret_cast<const char *>(bmat) - lead;
        w_lane = lds + row0 * kPitch + chunk * 16;
        const int g = lane >> 4, j = lane & 15;
        const int base = lds + (8 * (lane >> 5) + (j >> 2)) * kPitch + (frag_col + 16 * (g & 1) + 4 * (j & 3)) * 2;
        r_lane[0] = base;
        r_lane[1] = base + kStage;
    }

    // K-tile t: k-rows t*BK .. ; the range ends at the last k-row inside K
    // (!VEC: with the dword that holds its last element).
    __device__ __forceinline__ void begin_tile(int t) {
        k0 = t * BK;
        const int rows = t < k_tiles ? min(BK, k_elems - k0) : 0;
        const uint32_t span = (uint32_t)rows * (uint32_t)n_total * 2u;
        rsrc_t = make_rsrc(b + (t < k_tiles ? (int64_t)k0 * n_total * 2 : 0),
                           VEC || rows == 0 ? span : (span + lead + 3u) & ~3u);
        // With one staging set, K-tile t is stored into LDS stage t % 2,
        // after begin_tile(t) and before begin_tile(t + 2).
        if constexpr (!VEC) krows[t & 1] = rows;
    }

    __device__ __forceinline__ void load(int i, int set) {
        regs[set][i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc_t, voff[i], 0, 0);
        if constexpr (!VEC) next[i] = __builtin_amdgcn_raw_buffer_load_b32(rsrc_t, voff[i] + 16u, 0, 0);
    }

    __device__ __forceinline__ void store(char *smem, int i, int stage, int set) const {
        int4v v = regs[set][i];
        if constexpr (!VEC) {
            const uint32_t w4 = next[i];
            v = int4v{(int)__builtin_amdgcn_alignbyte((uint32_t)v[1], (uint32_t)v[0], shift),
                      (int)__builtin_amdgcn_alignbyte((uint32_t)v[2], (uint32_t)v[1], shift),
                      (int)__builtin_amdgcn_alignbyte((uint32_t)v[3], (uint32_t)v[2], shift),
                      (int)__builtin_amdgcn_alignbyte(w4, (uint32_t)v[3], shift)};
            // a k-row past K can hold the element that shares the last
            // element's dword: it must not meet A's zeros as a NaN
            if (row0 + RPP * i >= (stage ? krows[1] : krows[0])) v = int4v{0, 0, 0, 0};
        }
        *reinterpret_cast<int4v *>(smem + w_lane + stage * kStage + i * RPP * kPitch) = v;
    }

    __device__ __forceinline__ half8 read(const char *smem, int stage, int ks, int f) const {
        typedef __fp16 fp16x4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
        typedef __attribute__((address_space(3))) fp16x4 lds_fp16x4;
        char *p0 = const_cast<char *>(smem) + r_lane[stage] + ks * 16 * kPitch + f * 64;
        // address-space casts of pointers into the __shared__ array
        const fp16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)p0);
        const fp16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4 *)(p0 + 4 * kPitch));
        half8 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            r[e] = (_Float16)lo[e];
            r[4 + e] = (_Float16)hi[e];
        }
        return r;
    }
};

// Epilogue: the accumulators of one wave to C (fp16, rounded to nearest
// even) or D (fp32).  smem is the workgroup's LDS of kLds bytes, free once
// every wave is past the K loop.
// Rows of each staging pass for a wave with kWaveBytes of LDS.
template <class C, bool NN, int kWaveBytes>
constexpr int staging_rows() {
    constexpr int RB = C::TN * (NN ? 4 : 2);
    return C::TM * RB <= kWaveBytes         ? C::TM
           : (C::TM / 2) * RB <= kWaveBytes ? C::TM / 2
           : (C::TM / 4) * RB <= kWaveBytes ? C::TM / 4
                                            : C::TM / 8;
}

// A wave's TM x TN piece of C on its way out: it goes through LDS in passes
// of SR rows.  Row r of a pass holds TN outputs (CPR chunks of 16 bytes,
// chunk c at slot c ^ (r % CPR)); lane l then takes chunk l % CPR of row
// l / CPR, so CPR consecutive lanes hold one contiguous row segment of C.
template <class C, bool NN, int kWaveBytes>
struct CStaging {
    static constexpr int TM = C::TM, TN = C::TN, FM = C::FM, FN = C::FN, MB = C::MB;
    using Out = std::conditional_t<NN, float, _Float16>;
    using Out4 = std::conditional_t<NN, floatx4, half4>;
    using Acc = typename Mfma<MB>::Acc;
    static constexpr int ES = (int)sizeof(Out);
    static constexpr int kGroups = MB == 32 ? 4 : 1;
    static constexpr int RB = TN * ES, CPR = RB / 16;
    static constexpr int SR = staging_rows<C, NN, kWaveBytes>();
    static constexpr int kPasses = TM / SR;
    static constexpr int kPerPass = SR * CPR / kWave;  // 16-byte chunks per lane and pass
    static_assert(SR * RB <= kWaveBytes && SR % MB == 0 && (SR * CPR) % kWave == 0, "staging");

    // MFMA result layout: for 32x32 blocks, lane l register r holds row
    // 8*(r/4) + 4*(l/32) + r%4, column l%32; for 16x16 blocks, row
    // 4*(l/16) + r, column l%16.  With the swapped operands the row is n and
    // the column is m, so each group of 4 registers is 4 consecutive n.
    // erow: this lane's row in a block (lane % MB), from an opaque zero so
    // the staging addresses are not computed early, where they would only
    // hold registers.
    static __device__ __forceinline__ void write_pass(const Acc (&acc)[FN][FM], char *stg, int pass, int erow,
                                                      int lane) {
        const int quad = MB == 32 ? (lane >> 5) * 4 : (lane >> 4) * 4;
#pragma unroll
        for (int i = pass * (SR / MB); i < (pass + 1) * (SR / MB); ++i) {
            const int rl = (i - pass * (SR / MB)) * MB + erow;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
#pragma unroll
                for (int g = 0; g < kGroups; ++g) {
                    Out4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = (Out)acc[j][i][4 * g + e];  // fp16: round to nearest even
                    const int byte = (j * MB + 8 * g + quad) * ES;
                    *reinterpret_cast<Out4 *>(stg + rl * RB + (((byte >> 4) ^ (rl % CPR)) << 4) + (byte & 15)) = o;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    static __device__ __forceinline__ int4v read_chunk(const char *stg, int s, int lane) {
        const int idx = s * kWave + lane;
        const int r = idx / CPR, c = idx % CPR;
        return *reinterpret_cast<const int4v *>(stg + r * RB + ((c ^ (r % CPR)) << 4));
    }

    // chunk s of pass `pass` into C; chunks wholly past N store nothing, only
    // a chunk that straddles N (or an unaligned C) takes the per-element path
    static __device__ __forceinline__ void store_chunk(const Params &p, int m0, int n0, int wm, int wn, int pass,
                                                       int s, int lane, int4v v, bool vec16) {
        const int idx = s * kWave + lane;
        const int r = idx / CPR, c = idx % CPR;
        const int m = m0 + wm * TM + pass * SR + r;
        const int n = n0 + wn * TN + c * (16 / ES);
        if (m < p.m && n < p.n) {
            Out *crow = static_cast<Out *>(p.c) + (int64_t)m * p.n;
            if (vec16 && n + 16 / ES - 1 < p.n) {
                // the host's cache policy (CStore; past the cache the second
                // contract keeps the default)
                if (p.c_store == kStoreDevice)
                    store_device_scope(crow + n, v);
                else if (!NN && p.c_store == kStoreStream)
                    __builtin_nontemporal_store(v, reinterpret_cast<int4v *>(crow + n));
                else
                    *reinterpret_cast<int4v *>(crow + n) = v;
            } else {
                union {
                    int4v v;
                    Out e[16 / ES];
                } u;
                u.v = v;
#pragma unroll
                for (int e = 0; e < 16 / ES; ++e)
                    if (n + e < p.n) crow[n + e] = u.e[e];
            }
        }
    }

    static __device__ __forceinline__ bool vec16(const Params &p) {
        return (p.n % (16 / ES)) == 0 && ((uintptr_t)p.c % 16) == 0;
    }

    static __device__ __forceinline__ int opaque_row(int lane) {
        int lz;
        asm volatile("v_mov_b32 %0, 0" : "=v"(lz));
        return lane % MB + lz;
    }
};

// The wave's piece of C from its accumulators, staged through kWaveBytes of
// LDS at stg (the caller makes sure no other wave uses them meanwhile).
template <class C, bool NN, int kWaveBytes>
__device__ __forceinline__ void store_tile_at(const typename Mfma<C::MB>::Acc (&acc)[C::FN][C::FM], char *stg,
                                              const Params &p, int m0, int n0, int wm, int wn, int lane) {
    using CS = CStaging<C, NN, kWaveBytes>;
    const int erow = CS::opaque_row(lane);
    const bool vec16 = CS::vec16(p);
#pragma unroll
    for (int pass = 0; pass < CS::kPasses; ++pass) {
        CS::write_pass(acc, stg, pass, erow, lane);
#pragma unroll
        for (int s = 0; s < CS::kPerPass; ++s)
            CS::store_chunk(p, m0, n0, wm, wn, pass, s, lane, CS::read_chunk(stg, s, lane), vec16);
    }
}

// The whole workgroup's C tile, each wave staging through its share of the
// kLds bytes at smem once every wave is done with the operand stages.
template <class C, bool NN, int kLds>
__device__ __forceinline__ void store_tile(const typename Mfma<C::MB>::Acc (&acc)[C::FN][C::FM], char *smem,
                                           const Params &p, int m0, int n0, int wm, int wn, int wave, int lane) {
    constexpr int kWaveBytes = kLds / C::kWaves;
    constexpr int SR = staging_rows<C, NN, kWaveBytes>();
    lds_barrier();
    store_tile_at<C, NN, kWaveBytes>(acc, smem + wave * (SR * C::TN * (NN ? 4 : 2)), p, m0, n0, wm, wn, lane);
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, class F>
__device__ __forceinline__ void static_range(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_range<B + 1, E>(f);
    }
}

// A k step's memory operations in issue order R0 W0 L0 R1 W1 L1 ... (nr
// fragment reads R, nw LDS writes W each followed by its global load L);
// kind 0 = R, 1 = W, 2 = L, and the index within its kind.
constexpr int step_op_kind(int o, int nr, int nw) {
    for (int t = 0;; ++t) {
        if (t < nr) {
            if (o == 0) return 0;
            --o;
        }
        if (t < nw) {
            if (o == 0) return 1;
            if (o == 1) return 2;
            o -= 2;
        }
    }
}
constexpr int step_op_index(int o, int nr, int nw) {
    for (int t = 0;; ++t) {
        if (t < nr) {
            if (o == 0) return t;
            --o;
        }
        if (t < nw) {
            if (o <= 1) return t;
            o -= 2;
        }
    }
}

// ---- the kernel -----------------------------------------------------------
//
// NN == false: C fp16 [M,N] = A [M,K] * B[N,K]^T (the tutorial's contract).
// NN == true:  D fp32 [M,N] = A [M,K] * B[K,N]   (the day-78 listing's).
// G: row alignment of the K-major operands (8, 2 or 1; KMajorOperand);
// KFULL: G == 8 and K a multiple of the K-tile (one descriptor per
// operand).
template <class C, int G, bool NN, bool KFULL>
__global__ __launch_bounds__(C::kThreads)
__attribute__((amdgpu_waves_per_eu(C::kMinWavesPerEU, C::kMinWavesPerEU)))
void gemm_f16_kernel(const Params p) {
    constexpr int BM = C::BM, BN = C::BN, KS = C::KS;
    constexpr int TM = C::TM, TN = C::TN, FM = C::FM, FN = C::FN, MB = C::MB;
    // with rows not 16-byte aligned the loads and the masks against K keep
    // too many registers live for a second staging set
    constexpr bool VEC = G == 8;
    static_assert(!NN || G == 8 || G == 1, "D = A B: 16-byte aligned rows, or any");
    constexpr int SETS = VEC ? C::kSets : 1;
    using OpA = KMajorOperand<C, BM, TM, G, KFULL, SETS>;
    using OpB = std::conditional_t<NN, NMajorB<C, VEC, SETS>, KMajorOperand<C, BN, TN, G, KFULL, SETS>>;
    constexpr int PA = OpA::kPasses, PB = OpB::kPasses;
    constexpr int kLdsB = OpA::kLdsBytes;
    static_assert(OpA::kLdsBytes + OpB::kLdsBytes <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(1024))) char smem[OpA::kLdsBytes + OpB::kLdsBytes];
    GEMM_POISON_LDS(smem);

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave / C::WN;
    const int wn = wave % C::WN;

    const TileCoord tc = tile_coord<uint32_t>(blockIdx.x, p.num_m, p.num_n, p.swizzle, p.xcd != 0);
    const int m0 = (int)tc.m_block * BM;
    const int n0 = (int)tc.n_block * BN;
    const int kt_count = p.k_tiles;
    if (kt_count == 0) return;  // never launched with K == 0

    // Per-tile buffer descriptors: rows past M (N) lie beyond num_records.
    OpA opa;
    OpB opb;
    opa.init(p.a + (int64_t)m0 * p.k, min(BM, p.m - m0), p.k, kt_count, tid, lane, wm * TM, 0);
    if constexpr (NN)
        opb.init(p.b, n0, p.n, p.k, kt_count, tid, lane, wn * TN, kLdsB);
    else
        opb.init(p.b + (int64_t)n0 * p.k, min(BN, p.n - n0), p.k, kt_count, tid, lane, wn * TN, kLdsB);

    using M = Mfma<MB>;
    typename M::Acc acc[FN][FM];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i) acc[j][i] = typename M::Acc{};

    half8 af[2][FM];
    half8 bf[2][FN];
    auto read_frags = [&](int buf, int stage, int ks) {
        // in the order the MFMAs consume them: B0, A0..A(FM-1), B1..
        bf[buf][0] = opb.read(smem, stage, ks, 0);
#pragma unroll
        for (int i = 0; i < FM; ++i) af[buf][i] = opa.read(smem, stage, ks, i);
#pragma unroll
        for (int j = 1; j < FN; ++j) bf[buf][j] = opb.read(smem, stage, ks, j);
    };

    // Prologue: K-tile 0 into stage 0; K-tiles 1 .. SETS (zeros past K) into
    // the staging register sets, K-tile x in set x % SETS.
    static_range<0, SETS + 1>([&](auto x_c) {
        constexpr int x = decltype(x_c)::value;
        opa.begin_tile(x);
        opb.begin_tile(x);
#pragma unroll
        for (int i = 0; i < PA; ++i) opa.load(i, x % SETS);
#pragma unroll
        for (int i = 0; i < PB; ++i) opb.load(i, x % SETS);
        if constexpr (x == SETS - 1) {
#pragma unroll
            for (int i = 0; i < PA; ++i) opa.store(smem, i, 0, 0);
#pragma unroll
            for (int i = 0; i < PB; ++i) opb.store(smem, i, 0, 0);
        }
    });
    lds_barrier();
    read_frags(0, 0, 0);

    // One K-tile of work, as KS k steps (MK wide) on stage STAGE, which also
    // moves the staged K-tile kt+1 into the other stage and refills its
    // staging registers with K-tile kt+1+SETS.  Past the last K-tile those moves
    // carry zeros that are never read, so every iteration is the same
    // branch-free block.  Its issue order is fixed instruction by
    // instruction: step ks puts after each of its MFMAs an even share of
    //   ks < KS-1: the fragment reads for step ks+1 and a slice of the LDS
    //              writes and global loads, as (read, write, load) triples;
    //   ks = KS-1: after the first MFMA, a wait for this wave's LDS traffic
    //              and the workgroup barrier, then the fragment reads for
    //              step 0 of K-tile kt+1.
    // LDS writes placed between fragment reads cost almost nothing, where a
    // run of writes after a run of reads stalls the MFMAs by about ten
    // cycles per write (measured on gfx950); hence the triples.
    constexpr int kSlices = KS - 1;
    constexpr int NM = FM * FN;
    constexpr int NR = FM + FN;  // fragment reads per step (calls)
    constexpr int kBarAt = GEMM_BAR_MFMA < NM ? GEMM_BAR_MFMA : NM - 1;
    auto read_frag = [&](int buf, int stage, int ks, int r) {
        // in the order the MFMAs consume them: B0, A0..A(FM-1), B1..
        if (r == 0)
            bf[buf][0] = opb.read(smem, stage, ks, 0);
        else if (r <= FM)
            af[buf][r - 1] = opa.read(smem, stage, ks, r - 1);
        else
            bf[buf][r - FM] = opb.read(smem, stage, ks, r - FM);
    };
    auto k_iter = [&](auto stage_tag, int kt) {
        constexpr int STAGE = decltype(stage_tag)::value;
        constexpr int NXT = STAGE ^ 1;
        constexpr int SET = SETS == 2 ? NXT : 0;  // (kt + 1) % SETS
        opa.begin_tile(kt + 1 + SETS);
        opb.begin_tile(kt + 1 + SETS);
        static_range<0, KS>([&](auto ks_c) {
            constexpr int ks = decltype(ks_c)::value;
            constexpr int cur = ks & 1;
            constexpr bool last = ks + 1 == KS;
            constexpr int rstage = last ? NXT : STAGE;
            constexpr int rks = last ? 0 : ks + 1;
            constexpr int a0 = ks * PA / kSlices, a1 = last ? a0 : (ks + 1) * PA / kSlices;
            constexpr int b0 = ks * PB / kSlices, b1 = last ? b0 : (ks + 1) * PB / kSlices;
            constexpr int nw = (a1 - a0) + (b1 - b0);
            constexpr int total = NR + 2 * nw;
            static_range<0, NM>([&](auto m_c) {
                constexpr int m = decltype(m_c)::value;
                // B fragments feed the MFMA's A operand and A fragments its
                // B operand, so each result block is C^T: a lane then holds
                // 4 consecutive n of one m row, which store as one vector.
                // snake order: odd rows of blocks run backwards, so each row
                // starts on the A fragment the previous row ended with (one
                // operand stays put across every pair of consecutive MFMAs)
                constexpr int j = m / FM, i = (j & 1) ? FM - 1 - m % FM : m % FM;
                acc[j][i] = M::run(bf[cur][j], af[cur][i], acc[j][i]);
                if constexpr (last && m == kBarAt) {
                    // The other stage is complete for everyone, and everyone
                    // has read its last fragments of this stage.
                    lds_barrier();
                }
                constexpr int first = last ? kBarAt : 0;  // ops ride after MFMAs first..NM-1
                constexpr int lo = m < first ? 0 : (m - first) * total / (NM - first);
                constexpr int hi = m < first ? 0 : (m - first + 1) * total / (NM - first);
                static_range<lo, hi>([&](auto o_c) {
                    constexpr int o = decltype(o_c)::value;
                    constexpr int kind = step_op_kind(o, NR, nw), idx = step_op_index(o, NR, nw);
                    if constexpr (kind == 0) {
                        read_frag(cur ^ 1, rstage, rks, idx);
                    } else {
                        constexpr bool is_a = idx < a1 - a0;
                        constexpr int pass = is_a ? a0 + idx : b0 + idx - (a1 - a0);
                        if constexpr (kind == 1) {
                            if constexpr (is_a) opa.store(smem, pass, NXT, SET);
                            else opb.store(smem, pass, NXT, SET);
                        } else {
                            if constexpr (is_a) opa.load(pass, SET);
                            else opb.load(pass, SET);
                        }
                    }
                });
                __builtin_amdgcn_sched_barrier(0);
            });
            // keep this step's fragments live to the end of the step, so the
            // next step's reads land in other registers
#pragma unroll
            for (int j = 0; j < FN; ++j) asm volatile("" ::"v"(bf[cur][j]));
#pragma unroll
            for (int i = 0; i < FM; ++i) asm volatile("" ::"v"(af[cur][i]));
        });
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

    store_tile<C, NN, OpA::kLdsBytes + OpB::kLdsBytes>(acc, smem, p, m0, n0, wm, wn, wave, lane);
}


// ---- direct-to-LDS variant (C = A B^T, K % 8 == 0, 16-byte aligned) -------
//
// The loads go straight from the buffer unit into LDS (buffer_load_dwordx4
// with the lds bit: lane l's 16 bytes land at M0 + 16 l), so no staging
// registers and no ds_write: the data does not cross the VGPR file on its
// way in, which saves issue slots and, on a power-limited part, energy.

// Wait until at most V of this wave's global loads are in flight and its LDS
// traffic is done, then the workgroup barrier.  A direct-to-LDS load counts
// on vmcnt until its data is in LDS.
template <int V>
__device__ __forceinline__ void vm_barrier() {
    static_assert(V >= 0 && V < 64, "vmcnt range");
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt((V & 15) | (7 << 4) | (0 << 8) | ((V >> 4) << 14));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Operand stored [rows, K] row-major, K % 64 == 0.  LDS stage: ROWS rows of
// 128 bytes (the K-tile's 64 fp16); the 16-byte chunk c (k 8c..8c+7) of row
// r sits at slot c ^ sw(r).  A load instruction of one wave fills a 1 KB
// block = 8 rows: lane l writes slot l % 8 of row l / 8 and so fetches the
// chunk that belongs there; the 8 lanes of a row still read one 128-byte
// segment.  A fragment read puts 16 rows at one chunk on every 16 lanes; two
// rows fill a 256-byte bank window, so the read is free of bank conflicts
// when those 16 rows take 16 distinct (row parity, slot) pairs.
//  * PERM false: fragment f, lane l reads row 16 f + l % 16 (consecutive
//    rows; 32x32x16: row 32 f + l % 32), and sw(r) = (r >> 1) & 7.
//  * PERM true (16x16x32 only): within each pair of fragments (2p, 2p + 1)
//    the rows are interleaved by fours: fragment 2p + s, lane l reads row
//    32 p + 8 ((l % 16) / 4) + 4 s + l % 4, and sw(r) = ((r >> 1) & 1) |
//    ((r >> 3) & 3) << 1.  As the MFMA's first operand this puts 8
//    consecutive rows (n of C) of one output row in a lane's two result
//    blocks 2p and 2p + 1, so C leaves in 16-byte stores straight from the
//    accumulators.
// Fragments: 32x32x16 lane l takes chunk 2 ks + l / 32 (k step ks of 16);
// 16x16x32 lane l takes chunk 4 ks + l / 16 (k step ks of 32).
// KFULL: K % 64 == 0.  Otherwise (K % 8 == 0) the lanes whose chunk lies
// past K get an out-of-range offset; an out-of-range lane of a direct load
// writes zeros into LDS (measured on gfx950), so the partial last K-tile
// reads as zero-padded.  A lane's chunk index is the same in every load of
// every K-tile (the swizzle's row bits do not change between a wave's
// blocks), so the mask is one compare per K-tile.
template <class C, int ROWS, bool KFULL = true, bool PERM = false>
struct KMajorDirect {
    static constexpr int kRow = 128;
    static constexpr int kStage = ROWS * kRow;
    static constexpr int kLdsBytes = 2 * kStage;
    static constexpr int kBlocks = kStage / 1024;       // 1 KB blocks per stage
    static constexpr int kLoads = kBlocks / C::kWaves;  // per wave and K-tile
    static_assert(C::BK == 64, "a 64-wide K-tile: 8 chunks per row");
    static_assert(kBlocks % C::kWaves == 0, "whole blocks per wave");
    // rows of a wave's loads differ by multiples of 8 kWaves, which must
    // leave the swizzle's row bits (1-3, or 1, 3 and 4) alone
    static_assert(C::kWaves % (PERM ? 4 : 2) == 0, "a lane's chunk index is the same in all its loads");
    static_assert(!PERM || C::MB == 16, "interleaved fragment rows serve 16x16x32 tiles");

    static __device__ __forceinline__ int sw(int r) {
        return PERM ? (((r >> 1) & 1) | (((r >> 3) & 3) << 1)) : ((r >> 1) & 7);
    }

    uint32_t voff[kLoads];
    __amdgpu_buffer_rsrc_t rsrc0, rsrc_none;
    int k_tiles;
    int k_elems, kc;  // !KFULL: K, and k of this lane's chunk inside a K-tile
    int lds_w;     // this wave's first block of stage 0
    int r_lane[PERM ? 2 : 1][C::KS]; // fragment 0 (PERM: fragments 0 and 1) of k step ks in stage 0

    __device__ __forceinline__ void init(const _Float16 *base, int rows_valid, int K, int kt_count, int wave,
                                         int lane, int frag_row, int lds) {
        k_tiles = kt_count;
        k_elems = K;
        rsrc0 = make_rsrc(base, (uint32_t)rows_valid * (uint32_t)K * 2u);
        rsrc_none = make_rsrc(base, 0u);
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int row = (i * C::kWaves + wave) * 8 + (lane >> 3);
            const int c = (lane & 7) ^ sw(row);
            voff[i] = (uint32_t)(row * K + c * 8) * 2u;
            if (i == 0) kc = c * 8;
        }
        lds_w = lds + wave * 1024;
        const int q = lane / C::MB, l16 = lane % C::MB;
        constexpr int kChunksPerStep = C::MK / 8;
#pragma unroll
        for (int s = 0; s < (PERM ? 2 : 1); ++s) {
            const int frow = frag_row + (PERM ? 8 * (l16 >> 2) + 4 * s + (l16 & 3) : l16);
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks)
                r_lane[s][ks] = lds + frow * kRow + (((kChunksPerStep * ks + q) ^ sw(frow)) << 4);
        }
    }

    // load i of K-tile t into stage S; past K an empty range (reads 0)
    template <int S>
    __device__ __forceinline__ void load(char *smem, int t, int i) const {
        uint32_t vo = voff[i];
        if constexpr (!KFULL) vo |= (t * C::BK + kc >= k_elems) ? kOutOfRange : 0u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            t < k_tiles ? rsrc0 : rsrc_none,
            (__attribute__((address_space(3))) void *)(smem + lds_w + S * kStage + i * C::kWaves * 1024), 16,
            vo, (uint32_t)t * 128u, 0, 0);
    }

    // an opaque copy of the LDS base: the loads' M0 addresses are then
    // rebuilt where they are used instead of held in scalar registers
    __device__ __forceinline__ void refresh_lds() { asm volatile("" : "+s"(lds_w)); }

    // load i of K-tile t of the tile whose rows start at base (rows_bytes
    // of them inside the matrix: the descriptor's range) into stage S
    template <int S>
    __device__ __forceinline__ void load_tile(char *smem, const _Float16 *base, uint32_t rows_bytes, int t,
                                              int i) const {
        uint32_t vo = voff[i];
        if constexpr (!KFULL) vo |= (t * C::BK + kc >= k_elems) ? kOutOfRange : 0u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            make_rsrc(base, rows_bytes),
            (__attribute__((address_space(3))) void *)(smem + lds_w + S * kStage + i * C::kWaves * 1024), 16, vo,
            (uint32_t)t * 128u, 0, 0);
    }

    __device__ __forceinline__ half8 read(const char *smem, int stage, int ks, int f) const {
        if constexpr (PERM)
            return *reinterpret_cast<const half8 *>(smem + r_lane[f & 1][ks] + stage * kStage + (f >> 1) * 32 * kRow);
        else
            return *reinterpret_cast<const half8 *>(smem + r_lane[0][ks] + stage * kStage + f * C::MB * kRow);
    }
};

typedef __fp16 fp16x4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) fp16x4 lds_fp16x4;

// ds_read_b64_tr_b16 through a restrict pointer.  The alias scope that the
// restrict parameter gives the read keeps the compiler from waiting for every
// direct-to-LDS load in flight (vmcnt 0) before it, which it does for a read
// it cannot tell apart from them; the kernels order these reads after the
// loads that fill their stage with their own waits and barriers, as they do
// for plain LDS reads.
static __device__ __forceinline__ fp16x4 lds_read_tr16(lds_fp16x4 *__restrict__ p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4f16(p);
}

// B of the second contract ([K, N] row-major) for 16x16x32 tiles, loaded
// straight into LDS.  Stage: the K-tile as 64 k-rows of BN fp16, unpadded
// (a direct load fills 1 KB, 1024 / (2 BN) whole k-rows); the 16-byte chunk
// c of k-row r sits at slot c ^ sw(r), sw(r) = 2 ((r & 3) | ((r >> 1) & 4)).
// A 16x16x32 fragment needs 8 consecutive k of one column per lane: two
// ds_read_b64_tr_b16 give it (in each 16-lane group, lane j reads 4
// consecutive n of k-row j / 4 and the hardware hands lane i the 4 k values
// of column i); a half-wave of such a read touches 8 k-rows, r and r + 8
// among them, whose 32-byte segments the swizzle puts on distinct banks.
// The swizzle of a lane's rows is the same in every k step (rows differ by
// multiples of 4 and by 8 g), but not additive across fragments, so each
// fragment column has its own address register.  Rows past K lie beyond
// the K-tile's descriptor; chunks past N (N % 8 == 0) get an out-of-range
// offset.
template <class C, bool KFULL>
struct NMajorDirect {
    static constexpr int BN = C::BN, BK = C::BK, FN = C::FN;
    static constexpr int CPR = BN / 8;  // 16-byte chunks per k-row
    static constexpr int kRowB = BN * 2;
    static constexpr int kStage = BK * kRowB;
    static constexpr int kLdsBytes = 2 * kStage;
    static constexpr int kRowsPerBlock = 1024 / kRowB;
    static constexpr int kBlocks = kStage / 1024;
    static constexpr int kLoads = kBlocks / C::kWaves;  // per wave and K-tile
    static_assert(C::MB == 16 && C::KS == 2 && BK == 64, "16x16x32 fragments of a 64-wide K-tile");
    static_assert(CPR >= 16 && CPR <= 64, "the swizzle needs 16..64 chunks per k-row");
    static_assert(kBlocks % C::kWaves == 0, "whole blocks per wave");

    static __device__ __forceinline__ int sw(int r) { return 2 * ((r & 3) | ((r >> 1) & 4)); }

    // loads i and i + 2 take the same chunk of their rows (rows 16 apart)
    static_assert((2 * C::kWaves * kRowsPerBlock) % 16 == 0, "chunk index periodic in the load index");

    uint32_t voff[kLoads];  // this lane's chunk in its rows of the K-tile, bit 31 set past N
    int ccol[2];            // column of that chunk in the tile, loads of even / odd index
    const _Float16 *b;      // B + n0: column n0 of k-row 0
    int n_total, k_elems, k_tiles, n0;
    int lds_w;        // this wave's first block of stage 0
    int r_lane[FN];   // fragment f, k step 0, first half, stage 0

    __device__ __forceinline__ void init(const _Float16 *bmat, int n_first, int N, int K, int kt_count, int wave,
                                         int lane, int frag_col, int lds) {
        // the tile's columns start at b; uniform values pinned to scalar registers
        const uint64_t addr = (uint64_t)(uintptr_t)(bmat + n_first);
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
        b = (const _Float16 *)(uintptr_t)(((uint64_t)hi << 32) | lo);
        n_total = __builtin_amdgcn_readfirstlane(N);
        k_elems = K;
        k_tiles = kt_count;
        n0 = __builtin_amdgcn_readfirstlane(n_first);
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int r = (i * C::kWaves + wave) * kRowsPerBlock + lane / CPR;
            const int c = (lane % CPR) ^ sw(r);
            voff[i] = ((uint32_t)(r * N + c * 8) * 2u) | ((n0 + c * 8 >= N) ? kOutOfRange : 0u);
            if (i < 2) ccol[i] = c * 8;
        }
        lds_w = lds + wave * 1024;
        const int g = lane >> 4, j = lane & 15;
        const int row = 8 * g + (j >> 2);     // + 32 ks + 4 h
        const int fsw = sw(row) >> 1;         // the same for every ks, h
#pragma unroll
        for (int f = 0; f < FN; ++f)
            r_lane[f] = lds + row * kRowB + ((((frag_col >> 4) + f) ^ fsw) << 5) + (((j >> 1) & 1) << 4) +
                        ((j & 1) << 3);
    }

    // load i of K-tile t into stage S: k-rows t BK .. of columns n0 ..
    template <int S>
    __device__ __forceinline__ void load(char *smem, int t, int i) const {
        // past the last K-tile: an empty range at the last one's base
        const bool live = t < k_tiles;
        const int k0 = (live ? t : k_tiles - 1) * BK;
        const uint32_t bytes = live ? (uint32_t)(min(BK, k_elems - k0) * n_total - n0) * 2u : 0u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            make_rsrc(b + (int64_t)k0 * n_total, bytes),
            (__attribute__((address_space(3))) void *)(smem + lds_w + S * kStage + i * C::kWaves * 1024), 16,
            voff[i], 0, 0, 0);
    }

    // an opaque copy of the LDS base (see KMajorDirect::refresh_lds)
    __device__ __forceinline__ void refresh_lds() { asm volatile("" : "+s"(lds_w)); }

    // load i of K-tile t of the tile whose columns start at tile_b = B +
    // tile_n0; bytes: the range of a whole K-tile from there (0: the loads
    // read zeros).  !KFULL: the range ends with the k-rows inside K (none
    // past the last K-tile).  The offsets were masked for columns past N
    // from column 0 in init; this adds the tile's own mask.
    template <int S>
    __device__ __forceinline__ void load_tile(char *smem, const _Float16 *tile_b, int tile_n0, uint32_t bytes, int t,
                                              int i) const {
        if constexpr (!KFULL) {
            const int rows = min(BK, k_elems - t * BK);
            bytes = bytes != 0u && rows > 0 ? (uint32_t)(rows * n_total - tile_n0) * 2u : 0u;
        }
        const uint32_t vo = voff[i] | ((tile_n0 + ccol[i & 1] >= n_total) ? kOutOfRange : 0u);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            make_rsrc(tile_b + (int64_t)t * BK * n_total, bytes),
            (__attribute__((address_space(3))) void *)(smem + lds_w + S * kStage + i * C::kWaves * 1024), 16, vo, 0,
            0, 0);
    }

    __device__ __forceinline__ half8 read(const char *smem, int stage, int ks, int f) const {
        char *p0 = const_cast<char *>(smem) + r_lane[f] + stage * kStage + ks * 32 * kRowB;
        // address-space casts of pointers into the __shared__ array
        const fp16x4 lo = lds_read_tr16((lds_fp16x4 *)p0);
        const fp16x4 hi = lds_read_tr16((lds_fp16x4 *)(p0 + 4 * kRowB));
        half8 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            r[e] = (_Float16)lo[e];
            r[4 + e] = (_Float16)hi[e];
        }
        return r;
    }
};

// Orders every accumulator after a stretch of s_nop: all accesses of acc
// before the call happen before the nops, all after it after them.  24 wait
// states cover the MFMA result latency (the hazards between an
// accumulator's VALU write and an MFMA reading it as srcC, and between an
// MFMA's result and a VALU read of it).
template <class Acc, int FN, int FM>
__device__ __forceinline__ void acc_fence(Acc (&acc)[FN][FM]) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i) asm volatile("" : "+a"(acc[j][i]));
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i) asm volatile("" : "+a"(acc[j][i]));
}

template <class C, bool KFULL>
__global__ __launch_bounds__(C::kThreads)
__attribute__((amdgpu_waves_per_eu(C::kMinWavesPerEU, C::kMinWavesPerEU)))
void gemm_f16_direct_kernel(const Params p) {
    constexpr int BM = C::BM, BN = C::BN, KS = C::KS;
    constexpr int TM = C::TM, TN = C::TN, FM = C::FM, FN = C::FN;
    using OpA = KMajorDirect<C, BM, KFULL>;
    using OpB = KMajorDirect<C, BN, KFULL>;
    constexpr int kLdsB = OpA::kLdsBytes;
    constexpr int kLds = OpA::kLdsBytes + OpB::kLdsBytes;
    constexpr int LA = OpA::kLoads, L = OpA::kLoads + OpB::kLoads;  // loads per wave and K-tile
    static_assert(kLds <= 160 * 1024, "LDS budget");
    static_assert(L < 64, "vmcnt range");
    static_assert(OpA::kStage + (FM - 1) * C::MB * 128 < 65536 && OpB::kStage + (FN - 1) * C::MB * 128 < 65536,
                  "LDS immediates must fit the 16-bit offset field");
    __shared__ __attribute__((aligned(1024))) char smem[kLds];
    GEMM_POISON_LDS(smem);

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / C::WN;
    const int wn = wave % C::WN;

    const TileCoord tc = tile_coord<uint32_t>(blockIdx.x, p.num_m, p.num_n, p.swizzle, p.xcd != 0);
    const int m0 = (int)tc.m_block * BM;
    const int n0 = (int)tc.n_block * BN;
    const int kt_count = p.k_tiles;
    if (kt_count == 0) return;  // never launched with K == 0

    OpA opa;
    OpB opb;
    opa.init(p.a + (int64_t)m0 * p.k, min(BM, p.m - m0), p.k, kt_count, wave, lane, wm * TM, 0);
    opb.init(p.b + (int64_t)n0 * p.k, min(BN, p.n - n0), p.k, kt_count, wave, lane, wn * TN, kLdsB);

    using M = Mfma<C::MB>;
    typename M::Acc acc[FN][FM];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i) acc[j][i] = typename M::Acc{};

    constexpr bool kTied = C::MB == 16;
    if constexpr (kTied) acc_fence(acc);

    half8 af[2][FM];
    half8 bf[2][FN];
    auto read_frag = [&](int buf, int stage, int ks, int r) {
        // in the order the MFMAs consume them: B0, A0..A(FM-1), B1..
        if (r == 0)
            bf[buf][0] = opb.read(smem, stage, ks, 0);
        else if (r <= FM)
            af[buf][r - 1] = opa.read(smem, stage, ks, r - 1);
        else
            bf[buf][r - FM] = opb.read(smem, stage, ks, r - FM);
    };
    auto load = [&](auto s_c, int t, int i) {
        constexpr int S = decltype(s_c)::value;
        if (i < LA)
            opa.template load<S>(smem, t, i);
        else
            opb.template load<S>(smem, t, i - LA);
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    constexpr int NM = FM * FN;
    constexpr int NR = FM + FN;
    constexpr int kBarMfma = C::MB == 16 ? GEMM_DIRECT_BAR_MFMA_M16 : GEMM_DIRECT_BAR_MFMA;
    constexpr int kBarAt = kBarMfma < NM ? kBarMfma : NM - 1;
    // The loads of K-tile t+2 go out in two parts: the first LH right after
    // the barrier of K-tile t (their stage has just been released), the rest
    // during k step 0 of K-tile t+1.  Issuing all of them in the last step's
    // few MFMAs overfills the texture address queue and stalls the wave.
    constexpr int LH = L - L * (C::MB == 16 ? GEMM_DIRECT_TAIL_M16 : GEMM_DIRECT_TAIL) / 16;
    // k steps the rest is spread over (all but the last)
    constexpr int TS = GEMM_DIRECT_TAIL_STEPS < KS ? GEMM_DIRECT_TAIL_STEPS : KS - 1;
    static_assert(TS >= 1, "tail steps");

    // Prologue: K-tile 0, and the first part of K-tile 1; wait for K-tile 0.
#pragma unroll
    for (int i = 0; i < L; ++i) load(S0{}, 0, i);
#pragma unroll
    for (int i = 0; i < LH; ++i) load(S1{}, 1, i);
    vm_barrier<LH>();
#pragma unroll
    for (int r = 0; r < NR; ++r) read_frag(0, 0, 0, r);

    // K-tile t on stage S, KS k steps.  Step 0: its MFMAs with the fragment
    // reads of step 1 and the rest of K-tile t+1's loads (into stage S^1,
    // free since the previous barrier).  Steps 1..KS-2: MFMAs and the next
    // step's fragment reads.  Last step: after MFMA kBarAt, wait until this
    // wave's loads of K-tile t+1 are in LDS and its reads of stage S are
    // done, pass the workgroup barrier (then everyone's are), and spread
    // over the remaining MFMAs the fragment reads of step 0 of K-tile t+1
    // (stage S^1) and the first loads of K-tile t+2 into stage S.
    // op o of a group of nr reads and nl loads, in the order R0 L0 R1 L1 ...
    // (the reads first while both remain): kind (0 read, 1 load) and index
    auto k_iter = [&](auto s_c, int t) {
        constexpr int S = decltype(s_c)::value;
        constexpr int SN = S ^ 1;
        using SNc = std::integral_constant<int, SN>;
        static_range<0, KS>([&](auto ks_c) {
            constexpr int ks = decltype(ks_c)::value;
            constexpr int cur = ks & 1;
            constexpr bool last = ks + 1 == KS;
            constexpr int first = last ? kBarAt : 0;      // ops ride after MFMAs first..NM-1
            // tail loads of K-tile t+1: [tl0, tl1) of L, over the first TS steps
            constexpr int tl0 = ks < TS ? LH + (L - LH) * ks / TS : 0;
            constexpr int tl1 = ks < TS ? LH + (L - LH) * (ks + 1) / TS : 0;
            constexpr int nl = last ? LH : tl1 - tl0;
            constexpr int total = NR + nl, slots = NM - first;
            static_range<0, NM>([&](auto m_c) {
                constexpr int m = decltype(m_c)::value;
                constexpr int j = m / FM, i = (j & 1) ? FM - 1 - m % FM : m % FM;
                if constexpr (kTied)
                    mfma16_tied(bf[cur][j], af[cur][i], acc[j][i]);
                else
                    acc[j][i] = M::run(bf[cur][j], af[cur][i], acc[j][i]);
                if constexpr (last && m == kBarAt) vm_barrier<0>();
                if constexpr (m >= first) {
                    constexpr int q = m - first;
                    static_range<q * total / slots, (q + 1) * total / slots>([&](auto o_c) {
                        constexpr int o = decltype(o_c)::value;
                        constexpr int pairs = NR < nl ? NR : nl;
                        constexpr bool is_read = o < 2 * pairs ? (o % 2 == 0) : (NR > nl);
                        constexpr int idx = o < 2 * pairs ? o / 2 : o - pairs;
                        if constexpr (is_read) {
                            if constexpr (last)
                                read_frag(cur ^ 1, SN, 0, idx);
                            else
                                read_frag(cur ^ 1, S, ks + 1, idx);
                        } else if constexpr (last) {
                            load(s_c, t + 2, idx);
                        } else {
                            load(SNc{}, t + 1, tl0 + idx);
                        }
                    });
                }
                __builtin_amdgcn_sched_barrier(0);
            });
#pragma unroll
            for (int j = 0; j < FN; ++j) asm volatile("" ::"v"(bf[cur][j]));
#pragma unroll
            for (int i = 0; i < FM; ++i) asm volatile("" ::"v"(af[cur][i]));
        });
    };
    // K-tiles in pairs (stage 0, stage 1); an odd count ends with one more
    // K-tile on stage 0.  Loads past K fill stages that are never summed.
    int kt = 0;
    for (; kt + 1 < kt_count; kt += 2) {
        k_iter(S0{}, kt);
        k_iter(S1{}, kt + 1);
    }
    if (kt < kt_count) k_iter(S0{}, kt);

    vm_barrier<0>();  // no load is still writing LDS when the epilogue stages C there
    if constexpr (kTied) acc_fence(acc);
    store_tile<C, false, kLds>(acc, smem, p, m0, n0, wm, wn, wave, lane);
}

// Wait until this wave's LDS reads are done (its global loads may still be
// in flight), then the workgroup barrier.
__device__ __forceinline__ void lgkm_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wait until at most V of this wave's global loads are in flight (its LDS
// reads may still be pending), then the workgroup barrier.
template <int V>
__device__ __forceinline__ void vm_only_barrier() {
    static_assert(V >= 0 && V < 64, "vmcnt range");
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt((V & 15) | (7 << 4) | (15 << 8) | ((V >> 4) << 14));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Direct-to-LDS kernel for 16x16x32 tiles (two 32-wide k steps per K-tile)
// with the fragment reads a whole K-tile ahead and two barriers per K-tile.
// Stage S holds K-tile t.  Both of its steps' fragments are read during
// step 1 of K-tile t-1, so S is free from the start of K-tile t:
//   step 0: release barrier (every wave's reads of S are done), then the
//           MFMAs of step 0 with the first loads of K-tile t+2 into S;
//   step 1: acquire barrier (every wave's loads of K-tile t+1 into S^1 are
//           done), then the MFMAs of step 1 with the reads of both steps of
//           K-tile t+1 from S^1 and the rest of K-tile t+2's loads.
// The loads of a K-tile thus spread over a whole K-tile, a steady stream
// instead of a burst after one barrier, and the last of them still have a k
// step to land.  Fragments rotate over three register buffers: step 0 always
// uses buffer 0, step 1 uses buffer 1 on stage 0 and buffer 2 on stage 1.
template <class C, bool KFULL, bool NN>
__global__ __launch_bounds__(C::kThreads)
__attribute__((amdgpu_waves_per_eu(C::kMinWavesPerEU, C::kMinWavesPerEU)))
void gemm_f16_direct_ahead_kernel(const Params p) {
    constexpr int BM = C::BM, BN = C::BN;
    constexpr int TM = C::TM, TN = C::TN, FM = C::FM, FN = C::FN;
    static_assert(C::MB == 16 && C::KS == 2, "two 32-wide k steps per K-tile");
    using OpA = KMajorDirect<C, BM, KFULL>;
    using OpB = std::conditional_t<NN, NMajorDirect<C, KFULL>, KMajorDirect<C, BN, KFULL>>;
    constexpr int kLdsB = OpA::kLdsBytes;
    constexpr int kLds = OpA::kLdsBytes + OpB::kLdsBytes;
    constexpr int LA = OpA::kLoads, L = OpA::kLoads + OpB::kLoads;
    static_assert(kLds <= 160 * 1024, "LDS budget");
    static_assert(2 * L < 64, "vmcnt range");
    static_assert(OpA::kStage + (FM - 1) * C::MB * 128 < 65536 && OpB::kStage + (FN - 1) * C::MB * 128 < 65536 &&
                      OpB::kStage + 36 * (BN * 2) < 65536,
                  "LDS immediates must fit the 16-bit offset field");
    __shared__ __attribute__((aligned(1024))) char smem[kLds];
    GEMM_POISON_LDS(smem);

    GEMM_TRACE_DO(TraceRecord tr; tr.t0 = trace_clock(); tr.r0 = trace_realtime(); tr.tiles = 1;)
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / C::WN;
    const int wn = wave % C::WN;

    const TileCoord tc = tile_coord<uint32_t>(blockIdx.x, p.num_m, p.num_n, p.swizzle, p.xcd != 0);
    const int m0 = (int)tc.m_block * BM;
    const int n0 = (int)tc.n_block * BN;
    const int kt_count = p.k_tiles;
    if (kt_count == 0) return;  // never launched with K == 0

    OpA opa;
    OpB opb;
    opa.init(p.a + (int64_t)m0 * p.k, min(BM, p.m - m0), p.k, kt_count, wave, lane, wm * TM, 0);
    if constexpr (NN)
        opb.init(p.b, n0, p.n, p.k, kt_count, wave, lane, wn * TN, kLdsB);
    else
        opb.init(p.b + (int64_t)n0 * p.k, min(BN, p.n - n0), p.k, kt_count, wave, lane, wn * TN, kLdsB);

    floatx4 acc[FN][FM];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i) acc[j][i] = floatx4{};
    acc_fence(acc);

    half8 af[3][FM];
    half8 bf[3][FN];
    constexpr int NR = FM + FN;  // fragment reads per k step
    // read r of the 2 NR reads of K-tile t+1: step r / NR, in the order the
    // MFMAs consume them (B0, A0..A(FM-1), B1..)
    auto read_frag = [&](int buf, int stage, int ks, int r) {
        if (r == 0)
            bf[buf][0] = opb.read(smem, stage, ks, 0);
        else if (r <= FM)
            af[buf][r - 1] = opa.read(smem, stage, ks, r - 1);
        else
            bf[buf][r - FM] = opb.read(smem, stage, ks, r - FM);
    };
    auto load = [&](auto s_c, int t, int i) {
        constexpr int S = decltype(s_c)::value;
        if (i < LA)
            opa.template load<S>(smem, t, i);
        else
            opb.template load<S>(smem, t, i - LA);
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    constexpr int NM = FM * FN;
    constexpr int kRelAt = GEMM_AHEAD_REL_MFMA < NM ? GEMM_AHEAD_REL_MFMA : NM - 1;
    constexpr int kAcqAt = GEMM_AHEAD_ACQ_MFMA < NM ? GEMM_AHEAD_ACQ_MFMA : NM - 1;
    constexpr int L0 = L * GEMM_AHEAD_STEP0_LOADS / 16;  // loads of K-tile t+2 in step 0

    // Prologue: K-tiles 0 and 1 into stages 0 and 1; both steps' fragments
    // of K-tile 0 into buffers 0 and 1.
#pragma unroll
    for (int i = 0; i < L; ++i) load(S0{}, 0, i);
#pragma unroll
    for (int i = 0; i < L; ++i) load(S1{}, 1, i);
    vm_barrier<L>();
    GEMM_TRACE_DO(tr.t1 = trace_clock();)
#pragma unroll
    for (int r = 0; r < NR; ++r) read_frag(0, 0, 0, r);
#pragma unroll
    for (int r = 0; r < NR; ++r) read_frag(1, 0, 1, r);

    auto k_iter = [&](auto s_c, int t) {
        constexpr int S = decltype(s_c)::value;
        constexpr int SN = S ^ 1;
        constexpr int B1 = S == 0 ? 1 : 2;   // this K-tile's step-1 buffer
        constexpr int NB1 = S == 0 ? 2 : 1;  // the next K-tile's
        // step 0
        static_range<0, NM>([&](auto m_c) {
            constexpr int m = decltype(m_c)::value;
            constexpr int j = m / FM, i = (j & 1) ? FM - 1 - m % FM : m % FM;
            mfma16_tied(bf[0][j], af[0][i], acc[j][i]);
            if constexpr (m == kRelAt) {
                GEMM_TRACE_DO(const uint64_t tb = trace_clock();)
                lgkm_barrier();
                GEMM_TRACE_DO(tr.rel += trace_clock() - tb;)
            }
            if constexpr (m >= kRelAt) {
                constexpr int q = m - kRelAt, slots = NM - kRelAt;
                static_range<q * L0 / slots, (q + 1) * L0 / slots>(
                    [&](auto o_c) { load(s_c, t + 2, decltype(o_c)::value); });
            }
            __builtin_amdgcn_sched_barrier(0);
        });
#pragma unroll
        for (int j = 0; j < FN; ++j) asm volatile("" ::"v"(bf[0][j]));
#pragma unroll
        for (int i = 0; i < FM; ++i) asm volatile("" ::"v"(af[0][i]));
        // step 1
        static_range<0, NM>([&](auto m_c) {
            constexpr int m = decltype(m_c)::value;
            constexpr int j = m / FM, i = (j & 1) ? FM - 1 - m % FM : m % FM;
            mfma16_tied(bf[B1][j], af[B1][i], acc[j][i]);
            if constexpr (m == kAcqAt) {
                GEMM_TRACE_DO(const uint64_t tb = trace_clock();)
                vm_only_barrier<L0>();
                GEMM_TRACE_DO(tr.acq += trace_clock() - tb;)
            }
            if constexpr (m >= kAcqAt) {
                constexpr int nl = L - L0, total = 2 * NR + nl, slots = NM - kAcqAt, q = m - kAcqAt;
                // R R L R R L ...: the reads first while both remain
                static_range<q * total / slots, (q + 1) * total / slots>([&](auto o_c) {
                    constexpr int o = decltype(o_c)::value;
                    constexpr int groups = (2 * NR) / 2 < nl ? (2 * NR) / 2 : nl;  // (R, R, L) groups
                    constexpr bool in_groups = o < 3 * groups;
                    constexpr bool is_read = in_groups ? (o % 3 != 2) : (2 * NR > 2 * groups);
                    constexpr int idx = in_groups ? (is_read ? (o / 3) * 2 + (o % 3) : o / 3)
                                                  : (is_read ? 2 * groups + (o - 3 * groups) : groups + (o - 3 * groups));
                    if constexpr (is_read) {
                        constexpr int ks = idx / NR, r = idx % NR;
                        read_frag(ks == 0 ? 0 : NB1, SN, ks, r);
                    } else {
                        load(s_c, t + 2, L0 + idx);
                    }
                });
            }
            __builtin_amdgcn_sched_barrier(0);
        });
#pragma unroll
        for (int j = 0; j < FN; ++j) asm volatile("" ::"v"(bf[B1][j]));
#pragma unroll
        for (int i = 0; i < FM; ++i) asm volatile("" ::"v"(af[B1][i]));
    };
    // K-tiles in pairs (stage 0, stage 1); an odd count ends with one more
    // K-tile on stage 0.  Loads past K fill stages that are never summed.
    int kt = 0;
    for (; kt + 1 < kt_count; kt += 2) {
        k_iter(S0{}, kt);
        k_iter(S1{}, kt + 1);
    }
    if (kt < kt_count) k_iter(S0{}, kt);

    vm_barrier<0>();  // no load is still writing LDS when the epilogue stages C there
    GEMM_TRACE_DO(tr.tl = trace_clock();)
    acc_fence(acc);
    store_tile<C, NN, kLds>(acc, smem, p, m0, n0, wm, wn, wave, lane);
    GEMM_TRACE_DO(__builtin_amdgcn_s_waitcnt(0); trace_write(tr, wave, lane);)
}

// The fragment-ahead kernel with one workgroup per CU walking several tiles
// (blockIdx.x, + gridDim.x, ...), for at least 3 K-tiles, and C with N % 8
// == 0 and a 16-byte aligned base; NN: B [K,N] and D fp32.  KFULL: K a
// multiple of the K-tile with an even count; otherwise the chunks past K
// read zeros and an odd count is rounded up by a K-tile of zeros (as in
// gemm_f16_stream_kernel).  The K-tile stream runs on across tiles:
// the last two K-tiles of a tile load the next tile's K-tiles 0 and 1 as
// their "K-tile t+2"; the last one reads no fragments ahead.  Each wave then
// stages its C through its share of the LDS beyond the two stages and stores
// it with 16-byte buffer stores whose out-of-range lanes are dropped by
// their offsets, so every wave issues exactly kStores of them on every tile.
// They go out after the loads of the next tile's K-tiles 0 and 1, so the
// waits that follow (K-tile 0 before its fragment reads, K-tile 1 at the next
// tile's first acquire barrier) can leave them in flight (the wait counter
// is in order): the store burst drains under the next tile's MFMAs.
template <class C, bool NN, bool KFULL = true>
__global__ __launch_bounds__(C::kThreads)
__attribute__((amdgpu_waves_per_eu(C::kMinWavesPerEU, C::kMinWavesPerEU)))
void gemm_f16_persistent_kernel(const Params p) {
    constexpr int BM = C::BM, BN = C::BN;
    constexpr int TM = C::TM, TN = C::TN, FM = C::FM, FN = C::FN;
    static_assert(C::MB == 16 && C::KS == 2, "two 32-wide k steps per K-tile");
    using OpA = KMajorDirect<C, BM, KFULL>;
    using OpB = std::conditional_t<NN, NMajorDirect<C, KFULL>, KMajorDirect<C, BN, KFULL>>;
    constexpr int kLdsB = OpA::kLdsBytes;
    constexpr int kLds = OpA::kLdsBytes + OpB::kLdsBytes;
    constexpr int LA = OpA::kLoads, L = OpA::kLoads + OpB::kLoads;
    // LDS beyond the two stages for the C staging: a quarter (fp16) or an
    // eighth (fp32) of a wave's piece of C per pass, within the 160 KB
    constexpr int ES = NN ? 4 : 2;
    constexpr int kPassRows = TM * 2 / (4 * ES) > C::MB ? TM * 2 / (4 * ES) : C::MB;
    constexpr int kWaveBytes = kPassRows * TN * ES;
    constexpr int kSpare = C::kWaves * kWaveBytes;
    using CS = CStaging<C, NN, kWaveBytes>;
    constexpr int kStores = CS::kPasses * CS::kPerPass;  // 16-byte chunks of a wave's piece of C
    // a wait may leave at most 63 operations in flight: past that it waits
    // for some of the stores as well
    constexpr int kLeave = L + kStores < 63 ? L + kStores : 63;
    static_assert(kLds + kSpare <= 160 * 1024, "LDS budget");
    static_assert(OpA::kStage + (FM - 1) * C::MB * 128 < 65536 && OpB::kStage + (FN - 1) * C::MB * 128 < 65536 &&
                      OpB::kStage + 36 * (BN * 2) < 65536,
                  "LDS immediates must fit the 16-bit offset field");
    __shared__ __attribute__((aligned(1024))) char smem[kLds + kSpare];
    GEMM_POISON_LDS(smem);

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / C::WN;
    const int wn = wave % C::WN;

    // K-tiles per tile: even and >= 4 (an odd count rounded up, !KFULL)
    const int kt_count = KFULL ? p.k_tiles : (p.k_tiles + 1) & ~1;
    const int ntiles = p.num_m * p.num_n;
    const int G = gridDim.x;
    int idx = blockIdx.x;

    // first rows of A, B and C of a tile and the bytes of its rows inside
    // the matrices (0 past the last tile: loads read zeros)
    struct TileRows {
        const _Float16 *a, *b;
        char *c;
        uint32_t a_bytes, b_bytes, c_bytes;
        int m0, n0;
    };
    auto tile_rows = [&](int id) {
        TileRows r;
        if (id < ntiles) {
            const TileCoord tc = tile_coord<uint32_t>(id, p.num_m, p.num_n, p.swizzle, p.xcd != 0);
            r.m0 = (int)tc.m_block * BM;
            r.n0 = (int)tc.n_block * BN;
            const uint32_t rows_a = (uint32_t)min(BM, p.m - r.m0), rows_b = (uint32_t)min(BN, p.n - r.n0);
            r.a = p.a + (int64_t)r.m0 * p.k;
            r.c = static_cast<char *>(p.c) + (int64_t)r.m0 * p.n * ES;
            r.a_bytes = rows_a * (uint32_t)p.k * 2u;
            r.c_bytes = rows_a * (uint32_t)p.n * (uint32_t)ES;
            if constexpr (NN) {  // B [K,N]: columns n0.. of a K-tile's k-rows
                r.b = p.b + r.n0;
                r.b_bytes = (uint32_t)(C::BK * p.n - r.n0) * 2u;
            } else {
                r.b = p.b + (int64_t)r.n0 * p.k;
                r.b_bytes = rows_b * (uint32_t)p.k * 2u;
            }
        } else {
            r.a = p.a;
            r.b = p.b;
            r.c = static_cast<char *>(p.c);
            r.a_bytes = r.b_bytes = r.c_bytes = 0u;
            r.m0 = r.n0 = 0;
        }
        // wave-uniform by construction; readfirstlane keeps them in scalar
        // registers through the K loop
        auto u32 = [](uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane(v); };
        auto uptr = [&](auto *q) {
            const uint64_t v = (uint64_t)(uintptr_t)q;
            return (decltype(q))(uintptr_t)(((uint64_t)u32((uint32_t)(v >> 32)) << 32) | u32((uint32_t)v));
        };
        r.a = uptr(r.a);
        r.b = uptr(r.b);
        r.c = uptr(r.c);
        r.a_bytes = u32(r.a_bytes);
        r.b_bytes = u32(r.b_bytes);
        r.c_bytes = u32(r.c_bytes);
        r.m0 = (int)u32((uint32_t)r.m0);
        r.n0 = (int)u32((uint32_t)r.n0);
        return r;
    };
    TileRows cur = tile_rows(idx);
    TileRows nxt = tile_rows(idx + G);

    OpA opa;
    OpB opb;
    opa.init(cur.a, 0, p.k, kt_count, wave, lane, wm * TM, 0);
    if constexpr (NN)
        opb.init(p.b, 0, p.n, p.k, kt_count, wave, lane, wn * TN, kLdsB);
    else
        opb.init(cur.b, 0, p.k, kt_count, wave, lane, wn * TN, kLdsB);

    floatx4 acc[FN][FM];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i) acc[j][i] = floatx4{};
    acc_fence(acc);

    half8 af[3][FM];
    half8 bf[3][FN];
    constexpr int NR = FM + FN;  // fragment reads per k step
    // in the order the MFMAs consume them: B0, A0..A(FM-1), B1..
    auto read_frag = [&](int buf, int stage, int ks, int r) {
        if (r == 0)
            bf[buf][0] = opb.read(smem, stage, ks, 0);
        else if (r <= FM)
            af[buf][r - 1] = opa.read(smem, stage, ks, r - 1);
        else
            bf[buf][r - FM] = opb.read(smem, stage, ks, r - FM);
    };
    // load i of K-tile u of the stream: K-tile u of this tile, or u -
    // kt_count of the next
    auto load = [&](auto s_c, int u, int i) {
        constexpr int S = decltype(s_c)::value;
        const bool next = u >= kt_count;
        const int t = next ? u - kt_count : u;
        if (i < LA)
            opa.template load_tile<S>(smem, next ? nxt.a : cur.a, next ? nxt.a_bytes : cur.a_bytes, t, i);
        else if constexpr (NN)
            opb.template load_tile<S>(smem, next ? nxt.b : cur.b, next ? nxt.n0 : cur.n0,
                                      next ? nxt.b_bytes : cur.b_bytes, t, i - LA);
        else
            opb.template load_tile<S>(smem, next ? nxt.b : cur.b, next ? nxt.b_bytes : cur.b_bytes, t, i - LA);
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using F = std::false_type;
    using T = std::true_type;
    constexpr int NM = FM * FN;
    constexpr int kRelAt = GEMM_AHEAD_REL_MFMA < NM ? GEMM_AHEAD_REL_MFMA : NM - 1;
    constexpr int kAcqAt = GEMM_AHEAD_ACQ_MFMA < NM ? GEMM_AHEAD_ACQ_MFMA : NM - 1;
    constexpr int L0 = L * GEMM_AHEAD_STEP0_LOADS / 16;  // loads of K-tile t+2 in step 0
    constexpr int kLeave0 = L0 + kStores < 63 ? L0 + kStores : 63;

    // Prologue: K-tiles 0 and 1 into stages 0 and 1, both in LDS before the
    // first K-tile (its acquire barrier then waits as after a tile change);
    // both steps' fragments of K-tile 0 into buffers 0 and 1.
#pragma unroll
    for (int i = 0; i < L; ++i) load(S0{}, 0, i);
#pragma unroll
    for (int i = 0; i < L; ++i) load(S1{}, 1, i);
    vm_barrier<0>();
#pragma unroll
    for (int r = 0; r < NR; ++r) read_frag(0, 0, 0, r);
#pragma unroll
    for (int r = 0; r < NR; ++r) read_frag(1, 0, 1, r);

    // first_c: K-tile 0 of a tile, whose acquire barrier may leave kStores
    // more operations (the previous tile's stores) in flight.  last_c: the
    // last K-tile of a tile: its loads, but no fragment reads ahead and so no
    // acquire barrier.
    auto k_iter = [&](auto s_c, int t, auto first_c, auto last_c) {
        constexpr int S = decltype(s_c)::value;
        constexpr bool FIRST = decltype(first_c)::value;
        constexpr bool LAST = decltype(last_c)::value;
        constexpr int SN = S ^ 1;
        opa.refresh_lds();
        opb.refresh_lds();
        constexpr int B1 = S == 0 ? 1 : 2;   // this K-tile's step-1 buffer
        constexpr int NB1 = S == 0 ? 2 : 1;  // the next K-tile's
        // step 0
        static_range<0, NM>([&](auto m_c) {
            constexpr int m = decltype(m_c)::value;
            constexpr int j = m / FM, i = (j & 1) ? FM - 1 - m % FM : m % FM;
            mfma16_tied(bf[0][j], af[0][i], acc[j][i]);
            if constexpr (m == kRelAt) lgkm_barrier();
            if constexpr (m >= kRelAt) {
                constexpr int q = m - kRelAt, slots = NM - kRelAt;
                static_range<q * L0 / slots, (q + 1) * L0 / slots>(
                    [&](auto o_c) { load(s_c, t + 2, decltype(o_c)::value); });
            }
            __builtin_amdgcn_sched_barrier(0);
        });
#pragma unroll
        for (int j = 0; j < FN; ++j) asm volatile("" ::"v"(bf[0][j]));
#pragma unroll
        for (int i = 0; i < FM; ++i) asm volatile("" ::"v"(af[0][i]));
        // step 1
        static_range<0, NM>([&](auto m_c) {
            constexpr int m = decltype(m_c)::value;
            constexpr int j = m / FM, i = (j & 1) ? FM - 1 - m % FM : m % FM;
            mfma16_tied(bf[B1][j], af[B1][i], acc[j][i]);
            if constexpr (!LAST && m == kAcqAt) vm_only_barrier<FIRST ? kLeave0 : L0>();
            if constexpr (LAST && m >= kAcqAt) {
                constexpr int nl = L - L0, slots = NM - kAcqAt, q = m - kAcqAt;
                static_range<q * nl / slots, (q + 1) * nl / slots>(
                    [&](auto o_c) { load(s_c, t + 2, L0 + decltype(o_c)::value); });
            }
            if constexpr (!LAST && m >= kAcqAt) {
                constexpr int nl = L - L0, total = 2 * NR + nl, slots = NM - kAcqAt, q = m - kAcqAt;
                // R R L R R L ...: the reads first while both remain
                static_range<q * total / slots, (q + 1) * total / slots>([&](auto o_c) {
                    constexpr int o = decltype(o_c)::value;
                    constexpr int groups = (2 * NR) / 2 < nl ? (2 * NR) / 2 : nl;  // (R, R, L) groups
                    constexpr bool in_groups = o < 3 * groups;
                    constexpr bool is_read = in_groups ? (o % 3 != 2) : (2 * NR > 2 * groups);
                    constexpr int idx2 = in_groups ? (is_read ? (o / 3) * 2 + (o % 3) : o / 3)
                                                   : (is_read ? 2 * groups + (o - 3 * groups) : groups + (o - 3 * groups));
                    if constexpr (is_read) {
                        constexpr int ks = idx2 / NR, r = idx2 % NR;
                        read_frag(ks == 0 ? 0 : NB1, SN, ks, r);
                    } else {
                        load(s_c, t + 2, L0 + idx2);
                    }
                });
            }
            __builtin_amdgcn_sched_barrier(0);
        });
#pragma unroll
        for (int j = 0; j < FN; ++j) asm volatile("" ::"v"(bf[B1][j]));
#pragma unroll
        for (int i = 0; i < FM; ++i) asm volatile("" ::"v"(af[B1][i]));
    };

    for (;;) {
        k_iter(S0{}, 0, T{}, F{});
        k_iter(S1{}, 1, F{}, F{});
        int kt = 2;
        for (; kt + 2 < kt_count; kt += 2) {
            k_iter(S0{}, kt, F{}, F{});
            k_iter(S1{}, kt + 1, F{}, F{});
        }
        k_iter(S0{}, kt, F{}, F{});
        k_iter(S1{}, kt + 1, F{}, T{});
        // C through this wave's staging area (no other wave uses it, and its
        // own last reads of it were a tile ago), each 16-byte chunk stored as
        // it is read back: a chunk past N gets an out-of-range offset, rows
        // past M lie beyond the descriptor's range.
        acc_fence(acc);
        {
            char *const stg = smem + kLds + wave * kWaveBytes;
            const __amdgpu_buffer_rsrc_t rc = make_rsrc(cur.c, cur.c_bytes);
            // an opaque zero: the staging and store addresses are computed
            // here, not kept live through the K loop as loop invariants
            int lz;
            asm volatile("v_mov_b32 %0, 0" : "=v"(lz));
            const int el = lane + lz;
            const int erow = el % C::MB;
#pragma unroll
            for (int pass = 0; pass < CS::kPasses; ++pass) {
                CS::write_pass(acc, stg, pass, erow, el);
#pragma unroll
                for (int q = 0; q < CS::kPerPass; ++q) {
                    const int e = q * kWave + el;
                    const int r = wm * TM + pass * CS::SR + e / CS::CPR;  // row inside the tile
                    const int n = cur.n0 + wn * TN + (e % CS::CPR) * (16 / ES);
                    const uint32_t off = (n < p.n) ? (uint32_t)(r * p.n + n) * (uint32_t)ES : kOutOfRange;
                    // the host's cache policy (CStore); the branch is uniform, and the
                    // cache-policy operand must be a constant
                    if (p.c_store == kStoreDevice)
                        __builtin_amdgcn_raw_buffer_store_b128(CS::read_chunk(stg, q, el), rc, off, 0,
                                                               store_aux(kStoreDevice));
                    else if (p.c_store == kStoreStream)
                        __builtin_amdgcn_raw_buffer_store_b128(CS::read_chunk(stg, q, el), rc, off, 0,
                                                               store_aux(kStoreStream));
                    else
                        __builtin_amdgcn_raw_buffer_store_b128(CS::read_chunk(stg, q, el), rc, off, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);  // one chunk at a time: few live registers
                }
            }
        }
        if (idx + G >= ntiles) break;
        // The next tile's K-tile 0 (loaded before its K-tile 1 and the
        // stores) is in LDS for every wave: its fragments into buffers 0, 1.
        vm_only_barrier<kLeave>();
#pragma unroll
        for (int r = 0; r < NR; ++r) read_frag(0, 0, 0, r);
#pragma unroll
        for (int r = 0; r < NR; ++r) read_frag(1, 0, 1, r);
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int i = 0; i < FM; ++i) acc[j][i] = floatx4{};
        acc_fence(acc);
        idx += G;
        cur = nxt;
        nxt = tile_rows(idx + G);
    }
    // the last tile's loads past the tile (zeros into LDS) are done before
    // the workgroup ends
    __builtin_amdgcn_s_waitcnt(0);
}

// v_mfma_f32_16x16x32_f16 with srcC = 0: the first MFMA of an accumulator
// block in a tile overwrites it.  The accumulator stays tied ("+a") so its
// registers do not move; the instruction does not read it.
__device__ __forceinline__ void mfma16_first(half8 a, half8 b, floatx4 &c) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "+a"(c) : "v"(a), "v"(b));
}

// C = A B^T with one workgroup per CU walking tiles (blockIdx.x, + gridDim.x,
// ...), like gemm_f16_persistent_kernel and under the same conditions, but
// with each tile's C leaving under the MFMAs around the tile change instead
// of in a pause between tiles.
//
// B's fragment rows are interleaved (KMajorDirect PERM), so a lane's result
// blocks (2p, i) and (2p + 1, i) hold 8 consecutive n of one row m of C:
// "unit" u = p FM + i, one 16-byte store.  The last K-tile of a tile reads
// the next tile's first fragments like any other, so the K-tile stream runs
// on unbroken; step 0 of a tile's first K-tile runs its MFMAs in unit order
// (blocks (2p, i), (2p + 1, i) back to back) with srcC = 0, and right before
// the MFMA that overwrites unit u (its MFMA 2u) the previous tile's unit u
// is read from the accumulators, rounded to fp16 (nearest even) and
// stored: one store every two MFMAs, each at least NM - 1 MFMAs after the
// unit's last MFMA (far more than the MFMA result latency).  Stores and
// loads share the in-order vmcnt counter, so the step-1 acquire barrier of
// that K-tile leaves the U stores in flight and the next K-tile's waits for
// them.  The last tile stores its units after the loop.  POL: the stores'
// cache policy (CStore), chosen by the host, so no store is behind a branch.
// KFULL: K a multiple of the K-tile; otherwise the chunks of every tile's
// last K-tile that lie past K get an out-of-range offset and read as zeros.
template <class C, int POL, bool KFULL = true>
__global__ __launch_bounds__(C::kThreads)
__attribute__((amdgpu_waves_per_eu(C::kMinWavesPerEU, C::kMinWavesPerEU)))
void gemm_f16_stream_kernel(const Params p) {
    constexpr int BM = C::BM, BN = C::BN;
    constexpr int TM = C::TM, TN = C::TN, FM = C::FM, FN = C::FN;
    static_assert(C::MB == 16 && C::KS == 2, "two 32-wide k steps per K-tile");
    static_assert(FN % 2 == 0, "B fragments in pairs");
    using OpA = KMajorDirect<C, BM, KFULL>;
    using OpB = KMajorDirect<C, BN, KFULL, true>;
    constexpr int kLdsB = OpA::kLdsBytes;
    constexpr int kLds = OpA::kLdsBytes + OpB::kLdsBytes;
    constexpr int LA = OpA::kLoads, L = OpA::kLoads + OpB::kLoads;
    constexpr int NM = FM * FN;  // MFMAs per k step
    constexpr int U = NM / 2;    // 16-byte store units per wave and tile
    static_assert(NM >= 16, "the store units need a window of several MFMAs");
    static_assert(kLds <= 160 * 1024, "LDS budget");
    static_assert(OpA::kStage + (FM - 1) * C::MB * 128 < 65536 && OpB::kStage + (FN / 2 - 1) * 32 * 128 < 65536,
                  "LDS immediates must fit the 16-bit offset field");
    __shared__ __attribute__((aligned(1024))) char smem[kLds];
    GEMM_POISON_LDS(smem);

    GEMM_TRACE_DO(TraceRecord tr; tr.t0 = trace_clock(); tr.r0 = trace_realtime();)
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / C::WN;
    const int wn = wave % C::WN;

    // K-tiles per tile: even and >= 4.  !KFULL rounds an odd count up: the
    // extra K-tile lies wholly past K and reads zeros, and its MFMAs add +0
    // to accumulators that are never -0 (they start at +0), which leaves
    // every bit unchanged.
    const int kt_count = KFULL ? p.k_tiles : (p.k_tiles + 1) & ~1;
    const int ntiles = p.num_m * p.num_n;
    const int G = gridDim.x;
    int idx = blockIdx.x;

    // first rows of A, B and C of a tile and the bytes of its rows inside
    // the matrices (0 past the last tile: loads read zeros)
    struct TileRows {
        const _Float16 *a, *b;
        _Float16 *c;
        uint32_t a_bytes, b_bytes, c_bytes;
        int n0;
    };
    auto tile_rows = [&](int id) {
        TileRows r;
        if (id < ntiles) {
            const TileCoord tc = tile_coord<uint32_t>(id, p.num_m, p.num_n, p.swizzle, p.xcd != 0);
            const int m0 = (int)tc.m_block * BM;
            r.n0 = (int)tc.n_block * BN;
            const uint32_t rows_a = (uint32_t)min(BM, p.m - m0), rows_b = (uint32_t)min(BN, p.n - r.n0);
            r.a = p.a + (int64_t)m0 * p.k;
            r.b = p.b + (int64_t)r.n0 * p.k;
            r.c = static_cast<_Float16 *>(p.c) + (int64_t)m0 * p.n;
            r.a_bytes = rows_a * (uint32_t)p.k * 2u;
            r.b_bytes = rows_b * (uint32_t)p.k * 2u;
            r.c_bytes = rows_a * (uint32_t)p.n * 2u;
        } else {
            r.a = p.a;
            r.b = p.b;
            r.c = static_cast<_Float16 *>(p.c);
            r.a_bytes = r.b_bytes = r.c_bytes = 0u;
            r.n0 = 0;
        }
        // wave-uniform by construction; readfirstlane keeps them in scalar
        // registers through the K loop
        auto u32 = [](uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane(v); };
        auto uptr = [&](auto *q) {
            const uint64_t v = (uint64_t)(uintptr_t)q;
            return (decltype(q))(uintptr_t)(((uint64_t)u32((uint32_t)(v >> 32)) << 32) | u32((uint32_t)v));
        };
        r.a = uptr(r.a);
        r.b = uptr(r.b);
        r.c = uptr(r.c);
        r.a_bytes = u32(r.a_bytes);
        r.b_bytes = u32(r.b_bytes);
        r.c_bytes = u32(r.c_bytes);
        r.n0 = (int)u32((uint32_t)r.n0);
        return r;
    };
    TileRows cur = tile_rows(idx);
    TileRows nxt = tile_rows(idx + G);
    TileRows prv = tile_rows(ntiles);  // before the first tile: nothing to store

    OpA opa;
    OpB opb;
    opa.init(cur.a, 0, p.k, kt_count, wave, lane, wm * TM, 0);
    opb.init(cur.b, 0, p.k, kt_count, wave, lane, wn * TN, kLdsB);

    // Every tile's first MFMA on a block takes srcC = 0, so the accumulators
    // are never cleared: defining them is enough.
    floatx4 acc[FN][FM];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i) asm volatile("" : "=a"(acc[j][i]));

    half8 af[3][FM];
    half8 bf[3][FN];
    constexpr int NR = FM + FN;  // fragment reads per k step
    // in the order the MFMAs consume them: B0, A0..A(FM-1), B1..
    auto read_frag = [&](int buf, int stage, int ks, int r) {
        if (r == 0)
            bf[buf][0] = opb.read(smem, stage, ks, 0);
        else if (r <= FM)
            af[buf][r - 1] = opa.read(smem, stage, ks, r - 1);
        else
            bf[buf][r - FM] = opb.read(smem, stage, ks, r - FM);
    };
    // load i of K-tile u of the stream: K-tile u of this tile, or u -
    // kt_count of the next
    auto load = [&](auto s_c, int u, int i) {
        constexpr int S = decltype(s_c)::value;
        const bool next = u >= kt_count;
        const int t = next ? u - kt_count : u;
        if (i < LA)
            opa.template load_tile<S>(smem, next ? nxt.a : cur.a, next ? nxt.a_bytes : cur.a_bytes, t, i);
        else
            opb.template load_tile<S>(smem, next ? nxt.b : cur.b, next ? nxt.b_bytes : cur.b_bytes, t, i - LA);
    };

    // Unit u = (p, i), i fastest by default: step 0 of a tile's first K-tile
    // then keeps one pair of B fragments for FM units in a row.  (p fastest
    // puts the two 64-byte halves of a 128-byte line of C, p = 2c and 2c + 1,
    // back to back; it measured 1-3% slower.)
    constexpr auto unit_p = [](int u) { return GEMM_UNIT_P_FAST ? u % (FN / 2) : u / FM; };
    constexpr auto unit_i = [](int u) { return GEMM_UNIT_P_FAST ? u / (FN / 2) : u % FM; };
    // Store unit u of tile t: lane l holds row 16 i + l % 16 of the wave's
    // rows and n = 32 p + 8 (l / 16) .. + 7 of its columns; the descriptor
    // starts at the tile's first row of C, so the offset adds the tile's
    // first column n0.  A chunk past N
    // (N % 8 == 0: wholly past) gets an out-of-range offset; rows past M lie
    // beyond the descriptor's range.
    const int col_l = wn * TN + 8 * (lane >> 4);
    const uint32_t lane_off = (uint32_t)((wm * TM + (lane & 15)) * p.n + col_l) * 2u;
    auto store_unit = [&](auto u_c, const TileRows &t, __amdgpu_buffer_rsrc_t rc) {
        constexpr int u = decltype(u_c)::value;
        constexpr int pp = unit_p(u), ii = unit_i(u);
        // redefine the unit's accumulators here, so their copies to VGPRs
        // happen here and not all at the top of the step
        asm volatile("" : "+a"(acc[2 * pp][ii]), "+a"(acc[2 * pp + 1][ii]));
        half8 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = (_Float16)acc[2 * pp][ii][e];  // round to nearest even
            v[4 + e] = (_Float16)acc[2 * pp + 1][ii][e];
        }
        // an opaque copy of the lane's offsets: computed here, not hoisted
        // out of the tile loop as 2 U loop invariants
        uint32_t lo = lane_off;
        int cl = col_l;
        asm volatile("" : "+v"(lo), "+v"(cl));
        const uint32_t off = (lo + (uint32_t)(16 * ii * p.n + t.n0 + 32 * pp) * 2u) |
                             (t.n0 + cl + 32 * pp < p.n ? 0u : kOutOfRange);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(int4v, v), rc, off, 0, store_aux(POL));
    };

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using F = std::false_type;
    using T = std::true_type;
    constexpr int kRelAt = GEMM_AHEAD_REL_MFMA < NM ? GEMM_AHEAD_REL_MFMA : NM - 1;
    constexpr int kAcqAt = GEMM_AHEAD_ACQ_MFMA < NM ? GEMM_AHEAD_ACQ_MFMA : NM - 1;
    constexpr int L0 = L * GEMM_AHEAD_STEP0_LOADS / 16;  // loads of K-tile t+2 in step 0
    static_assert(U + L0 < 64, "vmcnt range");

    // Prologue: K-tiles 0 and 1 into stages 0 and 1; wait for K-tile 0 only
    // (K-tile 1's loads went out first, so the first K-tile's acquire
    // barrier, vmcnt(U + L0), covers them); both steps' fragments of K-tile
    // 0 into buffers 0 and 1.
#pragma unroll
    for (int i = 0; i < L; ++i) load(S0{}, 0, i);
#pragma unroll
    for (int i = 0; i < L; ++i) load(S1{}, 1, i);
    vm_barrier<L>();
    GEMM_TRACE_DO(tr.t1 = trace_clock();)
#pragma unroll
    for (int r = 0; r < NR; ++r) read_frag(0, 0, 0, r);
#pragma unroll
    for (int r = 0; r < NR; ++r) read_frag(1, 0, 1, r);

    // One K-tile (as gemm_f16_persistent_kernel's).  FIRST: a tile's first
    // K-tile: step 0 in unit order with srcC = 0, storing the units of the
    // previous tile (ep, through rc_ep) as it overwrites them.
    auto k_iter = [&](auto s_c, int t, auto first_c, const TileRows &ep, __amdgpu_buffer_rsrc_t rc_ep) {
        constexpr int S = decltype(s_c)::value;
        constexpr bool FIRST = decltype(first_c)::value;
        constexpr int SN = S ^ 1;
#if defined(GEMM_F16_TRACE) && defined(GEMM_F16_TRACE_KTILES)
        if (tr.tiles == 1) {
            if (t == kt_count - 1) tr.kt_last = (uint32_t)trace_clock();
        } else if (tr.tiles == 2 && t < 3) {
            const uint32_t tk = (uint32_t)trace_clock();
            if (t == 0) tr.kt0 = tk;
            else if (t == 1) tr.kt1 = tk;
            else tr.kt2 = tk;
        }
#endif
        opa.refresh_lds();
        opb.refresh_lds();
        constexpr int B1 = S == 0 ? 1 : 2;   // this K-tile's step-1 buffer
        constexpr int NB1 = S == 0 ? 2 : 1;  // the next K-tile's
        // step 0
        static_range<0, NM>([&](auto m_c) {
            constexpr int m = decltype(m_c)::value;
            if constexpr (FIRST) {
                constexpr int u = m / 2, j = 2 * unit_p(u) + m % 2, i = unit_i(u);
                if constexpr (m % 2 == 0) store_unit(std::integral_constant<int, u>{}, ep, rc_ep);
                mfma16_first(bf[0][j], af[0][i], acc[j][i]);
            } else {
                constexpr int j = m / FM, i = (j & 1) ? FM - 1 - m % FM : m % FM;
                mfma16_tied(bf[0][j], af[0][i], acc[j][i]);
            }
            if constexpr (m == kRelAt) {
                GEMM_TRACE_DO(const uint64_t tb = trace_clock();)
                lgkm_barrier();
                GEMM_TRACE_DO(tr.rel += trace_clock() - tb;)
            }
            if constexpr (m >= kRelAt) {
                constexpr int q = m - kRelAt, slots = NM - kRelAt;
                static_range<q * L0 / slots, (q + 1) * L0 / slots>(
                    [&](auto o_c) { load(s_c, t + 2, decltype(o_c)::value); });
            }
            __builtin_amdgcn_sched_barrier(0);
        });
#pragma unroll
        for (int j = 0; j < FN; ++j) asm volatile("" ::"v"(bf[0][j]));
#pragma unroll
        for (int i = 0; i < FM; ++i) asm volatile("" ::"v"(af[0][i]));
        // step 1
        static_range<0, NM>([&](auto m_c) {
            constexpr int m = decltype(m_c)::value;
            constexpr int j = m / FM, i = (j & 1) ? FM - 1 - m % FM : m % FM;
            mfma16_tied(bf[B1][j], af[B1][i], acc[j][i]);
            // Acquire: this wave's loads of K-tile t+1 are in LDS; after
            // them went out the loads of K-tile t+2 of step 0 and, in a
            // tile's first K-tile, the previous tile's U stores.
            if constexpr (m == kAcqAt) {
                GEMM_TRACE_DO(const uint64_t tb = trace_clock();)
                vm_only_barrier<FIRST ? U + L0 : L0>();
                GEMM_TRACE_DO(const uint64_t dt = trace_clock() - tb; tr.acq += dt; if constexpr (FIRST) tr.acq_first += dt;)
            }
            if constexpr (m >= kAcqAt) {
                constexpr int nl = L - L0, total = 2 * NR + nl, slots = NM - kAcqAt, q = m - kAcqAt;
                // R R L R R L ...: the reads first while both remain
                static_range<q * total / slots, (q + 1) * total / slots>([&](auto o_c) {
                    constexpr int o = decltype(o_c)::value;
                    constexpr int groups = (2 * NR) / 2 < nl ? (2 * NR) / 2 : nl;  // (R, R, L) groups
                    constexpr bool in_groups = o < 3 * groups;
                    constexpr bool is_read = in_groups ? (o % 3 != 2) : (2 * NR > 2 * groups);
                    constexpr int idx2 = in_groups ? (is_read ? (o / 3) * 2 + (o % 3) : o / 3)
                                                   : (is_read ? 2 * groups + (o - 3 * groups) : groups + (o - 3 * groups));
                    if constexpr (is_read) {
                        constexpr int ks = idx2 / NR, r = idx2 % NR;
                        read_frag(ks == 0 ? 0 : NB1, SN, ks, r);
                    } else {
                        load(s_c, t + 2, L0 + idx2);
                    }
                });
            }
            __builtin_amdgcn_sched_barrier(0);
        });
#pragma unroll
        for (int j = 0; j < FN; ++j) asm volatile("" ::"v"(bf[B1][j]));
#pragma unroll
        for (int i = 0; i < FM; ++i) asm volatile("" ::"v"(af[B1][i]));
    };

    // Every tile runs the same code, with no branch around a K-tile (with
    // all registers in use, duplicated K-tiles on two paths make the
    // register allocator spill): the first tile stores the units of a
    // "previous tile" with an empty range, which are dropped, and the last
    // reads the fragments of a "next tile" past the grid, zeros.
    __amdgpu_buffer_rsrc_t rc_prv = make_rsrc(prv.c, 0u);
    for (;;) {
#ifdef GEMM_F16_TRACE
        {
            const uint64_t ts = trace_clock();
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (tr.tiles == (uint64_t)i) tr.tile_start[i] = ts;  // constant indexes: no scratch
            ++tr.tiles;
        }
#endif
        k_iter(S0{}, 0, T{}, prv, rc_prv);
        k_iter(S1{}, 1, F{}, prv, rc_prv);
        for (int kt = 2; kt < kt_count; kt += 2) {
            k_iter(S0{}, kt, F{}, prv, rc_prv);
            k_iter(S1{}, kt + 1, F{}, prv, rc_prv);
        }
        if (idx + G >= ntiles) break;
        prv = cur;
        rc_prv = make_rsrc(cur.c, cur.c_bytes);
        cur = nxt;
        idx += G;
        nxt = tile_rows(idx + G);
    }
    // the last tile's units
    GEMM_TRACE_DO(tr.tl = trace_clock();)
    acc_fence(acc);
    {
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(cur.c, cur.c_bytes);
        static_range<0, U>([&](auto u_c) {
            store_unit(u_c, cur, rc);
            __builtin_amdgcn_sched_barrier(0);
        });
    }
    // the last tile's loads past the tile (zeros into LDS) and its stores
    // are done before the workgroup ends
    __builtin_amdgcn_s_waitcnt(0);
    GEMM_TRACE_DO(trace_write(tr, wave, lane);)
}

// ---- configurable ring (the tuning sweep's other axes) -------------------------
//
// A one-tile-per-workgroup kernel for C = A B^T whose K-tile width (block_k
// 32 or 64), LDS ring depth (S stages) and wave roles are template
// parameters, so the sweep can measure the axes the default kernels fix
// (block_k 64, 2 stages, every wave loading): the "Pipeline Depth" and
// producer/consumer ("Two Consumer Warp Groups") variants of "4. Pipeline
// Abstraction and Two Consumer Warp Groups", on gfx950 terms.  16x16x32 MFMAs
// with tied accumulators; fragments read one 32-wide k step ahead; one
// workgroup barrier per K-tile, a few MFMAs into its last k step: before it
// every wave has finished reading the K-tile's stage and the loading waves
// have waited for their loads of the next K-tile, so after it the stage is
// free for the loads of K-tile t + S and the next K-tile is in LDS for
// everyone.  PROD: 4 more waves that only load (the MFMA waves then issue
// no global loads); otherwise every wave loads its share, spread over the
// MFMAs after the barrier.  K % BK == 0; the K-tile count is padded with
// all-zero K-tiles to a whole number of unrolled blocks (they add +0 to
// accumulators that are never -0, which leaves every bit as it was).

// Operand stored [rows, K] row-major: LDS stage of ROWS rows of BK fp16
// (2 BK bytes); the 16-byte chunk c of row r at slot c ^ sw(r).  A fragment
// read puts 16 consecutive rows at one chunk on 16 lanes, and a 256-byte
// bank window holds 256 / (2 BK) rows, so the read is free of bank
// conflicts when those rows take distinct (row mod rows-per-window, slot)
// pairs: sw(r) = (r >> 1) & 7 for BK 64, (r >> 2) & 3 for BK 32.  A load
// fills 1 KB: lane l writes slot l % (BK / 8) of row l / (BK / 8) and
// fetches the chunk that belongs there.  NLW waves load, load i of loading
// wave w covering rows (i NLW + w) 1024 / (2 BK) ..; those rows differ by
// multiples of 32, which leaves a lane's slot-to-chunk map the same in all
// its loads.
template <class C, int ROWS, int BK, int NLW>
struct RingOperand {
    static constexpr int kRow = 2 * BK, kCpr = BK / 8, kRowsPerLoad = 1024 / kRow;
    static constexpr int kStage = ROWS * kRow;
    static constexpr int kBlocks = kStage / 1024;
    static constexpr int kLoads = kBlocks / NLW;  // per loading wave and K-tile
    static constexpr int KS = BK / 32;            // 32-wide k steps per K-tile
    static_assert(BK == 32 || BK == 64, "block_k");
    static_assert(kBlocks % NLW == 0, "whole blocks per loading wave");
    static_assert((NLW * kRowsPerLoad) % 32 == 0, "a lane's chunk map is the same in all its loads");

    static __device__ __forceinline__ int sw(int r) { return BK == 64 ? ((r >> 1) & 7) : ((r >> 2) & 3); }

    uint32_t voff[kLoads];
    __amdgpu_buffer_rsrc_t rsrc, rsrc_none;
    int k_tiles;
    int lds_w;       // this loading wave's first block of stage 0
    int r_lane[KS];  // fragment 0 of k step ks, stage 0

    __device__ __forceinline__ void init_loads(const _Float16 *base, int rows_valid, int K, int kt, int lw, int lane,
                                               int lds) {
        k_tiles = kt;
        rsrc = make_rsrc(base, (uint32_t)rows_valid * (uint32_t)K * 2u);
        rsrc_none = make_rsrc(base, 0u);
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int row = (i * NLW + lw) * kRowsPerLoad + lane / kCpr;
            voff[i] = (uint32_t)(row * K + ((lane % kCpr) ^ sw(row)) * 8) * 2u;
        }
        lds_w = lds + lw * 1024;
    }

    __device__ __forceinline__ void init_reads(int frag_row, int lane, int lds) {
        const int frow = frag_row + lane % 16, q = lane / 16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) r_lane[ks] = lds + frow * kRow + (((4 * ks + q) ^ sw(frow)) << 4);
    }

    // load i of K-tile t into stage s (byte offset so); past K an empty range (reads 0)
    __device__ __forceinline__ void load(char *smem, int so, int t, int i) const {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            t < k_tiles ? rsrc : rsrc_none,
            (__attribute__((address_space(3))) void *)(smem + lds_w + so + i * NLW * 1024), 16, voff[i],
            (uint32_t)t * (uint32_t)kRow, 0, 0);
    }

    __device__ __forceinline__ void refresh_lds() { asm volatile("" : "+s"(lds_w)); }

    __device__ __forceinline__ half8 read(const char *smem, int so, int ks, int f) const {
        return *reinterpret_cast<const half8 *>(smem + r_lane[ks] + so + f * 16 * kRow);
    }
};

template <class C, int BK, int S, bool PROD>
__global__ __launch_bounds__(C::kThreads *(PROD ? 2 : 1))
__attribute__((amdgpu_waves_per_eu(PROD ? 2 : C::kMinWavesPerEU, PROD ? 2 : C::kMinWavesPerEU)))
void gemm_f16_ring_kernel(const Params p) {
    constexpr int BM = C::BM, BN = C::BN;
    constexpr int TM = C::TM, TN = C::TN, FM = C::FM, FN = C::FN;
    constexpr int NC = C::kWaves;        // MFMA waves
    constexpr int NLW = PROD ? 4 : NC;   // loading waves
    static_assert(C::MB == 16, "16x16x32 MFMAs");
    using OpA = RingOperand<C, BM, BK, NLW>;
    using OpB = RingOperand<C, BN, BK, NLW>;
    constexpr int KS = OpA::KS;
    constexpr int kStageAB = OpA::kStage + OpB::kStage;  // one stage: A then B
    constexpr int kLds = S * kStageAB;
    constexpr int LA = OpA::kLoads, L = OpA::kLoads + OpB::kLoads;  // per loading wave and K-tile
    constexpr int NM = FM * FN, NR = FM + FN;
    // K-tiles per unrolled block: S stages, and an even number of k steps
    // so that the fragment buffers alternate within it
    constexpr int kBlk = (S * KS) % 2 == 0 ? S : 2 * S;
    static_assert(S >= 2 && kLds <= 160 * 1024, "LDS budget");
    static_assert((S - 1) * L < 64, "vmcnt range");
    // (a stage offset past the 16-bit LDS immediate costs the compiler an
    // address add per read; deep rings of large stages pay it)
    __shared__ __attribute__((aligned(1024))) char smem[kLds];
    GEMM_POISON_LDS(smem);

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const bool mfma_wave = !PROD || wave < NC;
    const int lw = PROD ? wave - NC : wave;  // index among the loading waves
    const int wm = (wave % NC) / C::WN;
    const int wn = (wave % NC) % C::WN;

    const TileCoord tc = tile_coord<uint32_t>(blockIdx.x, p.num_m, p.num_n, p.swizzle, p.xcd != 0);
    const int m0 = (int)tc.m_block * BM;
    const int n0 = (int)tc.n_block * BN;
    const int kt = p.k / BK;                      // K % BK == 0 (the host's condition)
    const int tpad = (kt + kBlk - 1) / kBlk * kBlk;  // padded with all-zero K-tiles

    OpA opa;
    OpB opb;
    opa.init_loads(p.a + (int64_t)m0 * p.k, min(BM, p.m - m0), p.k, kt, lw, lane, 0);
    opb.init_loads(p.b + (int64_t)n0 * p.k, min(BN, p.n - n0), p.k, kt, lw, lane, OpA::kStage);
    opa.init_reads(wm * TM, lane, 0);
    opb.init_reads(wn * TN, lane, OpA::kStage);

    auto load = [&](int so, int t, int i) {
        if (i < LA)
            opa.load(smem, so, t, i);
        else
            opb.load(smem, so, t, i - LA);
    };

    if (PROD && !mfma_wave) {
        // Loading waves: K-tiles 0 .. S-1 into stages 0 .. S-1; then per
        // K-tile t, wait for K-tile t + 1 (after it went out K-tiles t + 2
        // .. t + S - 1), pass the barrier (everyone has read stage t % S)
        // and load K-tile t + S into it.
        for (int s = 0; s < S; ++s)
#pragma unroll
            for (int i = 0; i < L; ++i) load(s * kStageAB, s, i);
        vm_barrier<(S - 1) * L>();  // K-tile 0 in LDS: the MFMA waves' first reads
        for (int t = 0; t < tpad; ++t) {
            vm_only_barrier<(S - 2) * L>();
            const int so = (t % S) * kStageAB;
#pragma unroll
            for (int i = 0; i < L; ++i) load(so, t + S, i);
        }
        __builtin_amdgcn_s_waitcnt(0);
        lds_barrier();  // the MFMA waves' epilogue barrier; LDS is now theirs
        return;
    }

    floatx4 acc[FN][FM];
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int i = 0; i < FM; ++i) acc[j][i] = floatx4{};
    acc_fence(acc);

    half8 af[2][FM];
    half8 bf[2][FN];
    auto read_frag = [&](int buf, int so, int ks, int r) {
        if (r == 0)
            bf[buf][0] = opb.read(smem, so, ks, 0);
        else if (r <= FM)
            af[buf][r - 1] = opa.read(smem, so, ks, r - 1);
        else
            bf[buf][r - FM] = opb.read(smem, so, ks, r - FM);
    };

    // Prologue: K-tiles 0 .. S-1 into the S stages (the loading waves), then
    // K-tile 0's first fragments.
    if constexpr (!PROD) {
        for (int s = 0; s < S; ++s)
#pragma unroll
            for (int i = 0; i < L; ++i) load(s * kStageAB, s, i);
        vm_barrier<(S - 1) * L>();
    } else {
        vm_barrier<0>();
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) read_frag(0, 0, 0, r);

    constexpr int kBarAt = 4 < NM ? 4 : NM - 1;
    // k step `step` (0 .. kBlk KS - 1 of the block) of K-tile t = t0 + step / KS
    auto k_step = [&](auto step_c, int t0) {
        constexpr int step = decltype(step_c)::value;
        constexpr int tb = step / KS, ks = step % KS, cur = step & 1;
        constexpr int s = tb % S, sn = (tb + 1) % S;
        constexpr bool last = ks == KS - 1;
        const int t = t0 + tb;
        opa.refresh_lds();
        opb.refresh_lds();
        static_range<0, NM>([&](auto m_c) {
            constexpr int m = decltype(m_c)::value;
            constexpr int j = m / FM, i = (j & 1) ? FM - 1 - m % FM : m % FM;
            mfma16_tied(bf[cur][j], af[cur][i], acc[j][i]);
            if constexpr (!last) {
                // the next k step's fragments, same stage
                static_range<m * NR / NM, (m + 1) * NR / NM>(
                    [&](auto r_c) { read_frag(cur ^ 1, s * kStageAB, ks + 1, decltype(r_c)::value); });
            } else {
                if constexpr (m == kBarAt) {
                    // this wave's reads of stage s are done and (loading
                    // waves) its loads of K-tile t + 1 are in LDS: after them
                    // went out those of K-tiles t + 2 .. t + S - 1
                    if constexpr (PROD)
                        lgkm_barrier();
                    else
                        vm_barrier<(S - 2) * L>();
                }
                if constexpr (m >= kBarAt) {
                    constexpr int q = m - kBarAt, slots = NM - kBarAt;
                    // K-tile t + 1's first fragments from the next stage
                    static_range<q * NR / slots, (q + 1) * NR / slots>(
                        [&](auto r_c) { read_frag(cur ^ 1, sn * kStageAB, 0, decltype(r_c)::value); });
                    if constexpr (!PROD)  // K-tile t + S into the stage just released
                        static_range<q * L / slots, (q + 1) * L / slots>(
                            [&](auto o_c) { load(s * kStageAB, t + S, decltype(o_c)::value); });
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        });
#pragma unroll
        for (int j = 0; j < FN; ++j) asm volatile("" ::"v"(bf[cur][j]));
#pragma unroll
        for (int i = 0; i < FM; ++i) asm volatile("" ::"v"(af[cur][i]));
    };
    for (int t0 = 0; t0 < tpad; t0 += kBlk)
        static_range<0, kBlk * KS>([&](auto step_c) { k_step(step_c, t0); });

    __builtin_amdgcn_s_waitcnt(0);  // no load still writing LDS when C is staged there
    acc_fence(acc);
    store_tile<C, false, kLds>(acc, smem, p, m0, n0, wm, wn, wave, lane);
}

// ---- launch ----------------------------------------------------------------

using Cfg256 = Cfg<256, 256, 2, 2>;   // 4 waves, 128x128 each
// the same tile on v_mfma_f32_16x16x32_f16 with tied accumulators: the
// direct-to-LDS path of every 4-wave tile (measured 12-16% faster than
// 32x32x16 at 256x256 and 7-28% at the smaller tiles; the register-staged
// path keeps 32x32x16, whose builtin keeps its accumulators in place)
using Cfg256d = Cfg<256, 256, 2, 2, 16>;
using Cfg256w8 = Cfg<256, 256, 4, 2>; // 8 waves, 64x128 each
using Cfg256x128 = Cfg<256, 128, 2, 2>;
using Cfg256x128d = Cfg<256, 128, 2, 2, 16>;
using Cfg128x256 = Cfg<128, 256, 2, 2>;
using Cfg128x256d = Cfg<128, 256, 2, 2, 16>;
using Cfg128 = Cfg<128, 128, 2, 2>;
using Cfg128d = Cfg<128, 128, 2, 2, 16>;
using Cfg128m16 = Cfg128d;  // v_mfma_f32_16x16x32_f16 on the register-staged path too
using Cfg64 = Cfg<64, 64, 2, 2>;
using Cfg64d = Cfg<64, 64, 2, 2, 16>;
using Cfg64x128 = Cfg<64, 128, 2, 2>;
using Cfg64x128d = Cfg<64, 128, 2, 2, 16>;
using Cfg128x64 = Cfg<128, 64, 2, 2>;
using Cfg128x64d = Cfg<128, 64, 2, 2, 16>;

// One launch of a kernel that takes Params, returning the status of this
// launch itself (not an error some earlier HIP call left behind).
template <class Kernel>
inline hipError_t launch_kernel(Kernel kernel, dim3 grid, dim3 block, hipStream_t stream, const Params &p) {
    void *args[] = {const_cast<Params *>(&p)};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, args, 0, stream);
}

// The stream kernel with the host's C store policy: the policy is a
// template argument, so no store sits behind a branch.
template <class CD, bool KFULL>
inline hipError_t launch_stream(const Params &p, dim3 grid, dim3 block, hipStream_t stream) {
    if (p.c_store == kStoreDevice)
        return launch_kernel(gemm_f16_stream_kernel<CD, kStoreDevice, KFULL>, grid, block, stream, p);
    if (p.c_store == kStoreStream && GEMM_STREAM_NT)
        return launch_kernel(gemm_f16_stream_kernel<CD, kStoreStream, KFULL>, grid, block, stream, p);
    return launch_kernel(gemm_f16_stream_kernel<CD, kStoreDefault, KFULL>, grid, block, stream, p);
}

// Launch of block tile C.  CD: the configuration of the direct-to-LDS kernels
// (16-byte loads); C: the register-staged kernel's.  g: the operands' row
// alignment (8: 16 bytes, 2: 4 bytes, 1: 2 bytes; KMajorOperand); cus: the
// device's compute units (0 if unknown: no one-workgroup-per-CU kernel).
// The 256x256 register-staged kernels exist only for 16-byte loads: with
// narrower ones their staging registers spill, so the host runs those
// operands on the 128x256 tile instead and this returns an error.
template <class C, bool NN, class CD = C>
hipError_t launch(const Params &p, int g, int cus, hipStream_t stream) {
    static_assert(CD::BM == C::BM && CD::BN == C::BN, "one block tile");
    const dim3 grid((unsigned)((int64_t)p.num_m * p.num_n));
    const int64_t tiles = (int64_t)p.num_m * p.num_n;
    const bool full = p.k % CD::BK == 0;
    if constexpr (NN && GEMM_DIRECT && GEMM_AHEAD && CD::MB == 16 && CD::BN >= 128) {
        // B [K,N] straight into LDS: 16-byte chunks of a k-row, a K-tile's
        // byte offsets below 2^31
        if (g == 8 && (int64_t)CD::BK * p.n * 2 < (int64_t(1) << 31)) {
            const dim3 block(CD::kThreads);
            // an even count of at least 4 whole K-tiles, or (KFULL = false)
            // at least 3 K-tiles of any kind
            const bool whole = full && p.k_tiles % 2 == 0 && p.k_tiles >= 4;
            const bool partial = GEMM_PARTIAL_K && p.k_tiles >= 3;
            if (GEMM_PERSIST && (whole || partial) && cus > 0 && tiles > cus && ((uintptr_t)p.c % 16) == 0 &&
                (int64_t)CD::BM * p.n * 4 < (int64_t(1) << 31))
                return whole ? launch_kernel(gemm_f16_persistent_kernel<CD, true, true>, dim3((unsigned)cus), block,
                                             stream, p)
                             : launch_kernel(gemm_f16_persistent_kernel<CD, true, false>, dim3((unsigned)cus), block,
                                             stream, p);
            return full ? launch_kernel(gemm_f16_direct_ahead_kernel<CD, true, true>, grid, block, stream, p)
                        : launch_kernel(gemm_f16_direct_ahead_kernel<CD, false, true>, grid, block, stream, p);
        }
    }
    if constexpr (!NN && GEMM_DIRECT) {
        if (g == 8) {
            const dim3 block(CD::kThreads);
            if constexpr (GEMM_AHEAD && CD::MB == 16) {
                // more tiles than CUs: one workgroup per CU walking several
                // tiles, where its conditions hold (the stream kernel also
                // takes a partial last K-tile)
                constexpr bool kStream = GEMM_STREAM && CD::FM * CD::FN >= 16;
                // an even count of at least 4 whole K-tiles; the KFULL =
                // false copies also take a partial last K-tile, and an odd
                // count of at least 3 (rounded up)
                const bool whole = full && p.k_tiles % 2 == 0 && p.k_tiles >= 4;
                const bool partial = GEMM_PARTIAL_K && p.k_tiles >= 3;
                if (GEMM_PERSIST && (whole || partial) && cus > 0 && tiles > cus && p.n % 8 == 0 &&
                    ((uintptr_t)p.c % 16) == 0 && (int64_t)CD::BM * p.n * 2 < (int64_t(1) << 31)) {
                    const dim3 g1((unsigned)cus);
                    if constexpr (kStream)
                        return whole ? launch_stream<CD, true>(p, g1, block, stream)
                                     : launch_stream<CD, false>(p, g1, block, stream);
                    else
                        return whole ? launch_kernel(gemm_f16_persistent_kernel<CD, false, true>, g1, block, stream, p)
                                     : launch_kernel(gemm_f16_persistent_kernel<CD, false, false>, g1, block, stream,
                                                     p);
                }
                return full ? launch_kernel(gemm_f16_direct_ahead_kernel<CD, true, false>, grid, block, stream, p)
                            : launch_kernel(gemm_f16_direct_ahead_kernel<CD, false, false>, grid, block, stream, p);
            } else {
                return full ? launch_kernel(gemm_f16_direct_kernel<CD, true>, grid, block, stream, p)
                            : launch_kernel(gemm_f16_direct_kernel<CD, false>, grid, block, stream, p);
            }
        }
    }
    const dim3 block(C::kThreads);
    if (g == 8) {
        // C = A B^T with 16-byte loads always takes a direct path above
        if constexpr (NN || !GEMM_DIRECT)
            return full ? launch_kernel(gemm_f16_kernel<C, 8, NN, true>, grid, block, stream, p)
                        : launch_kernel(gemm_f16_kernel<C, 8, NN, false>, grid, block, stream, p);
        else
            return hipErrorInvalidValue;
    }
    if constexpr (!(C::BM == 256 && C::BN == 256)) {
        if constexpr (!NN) {
            if (g == 2) return launch_kernel(gemm_f16_kernel<C, 2, NN, false>, grid, block, stream, p);
        }
        return launch_kernel(gemm_f16_kernel<C, 1, NN, false>, grid, block, stream, p);
    } else {
        return hipErrorInvalidValue;
    }
}

// The ring kernel's variants (gemm_f16_options.variant 1..7): (block_k,
// stages, loader waves).  A variant whose LDS does not fit, or whose MFMA
// waves would not fit their registers next to loader waves, is not
// compiled; the host refuses it before launching.
template <class CD, int BK, int S, bool PROD>
constexpr bool ring_fits() {
    constexpr int stage = (CD::BM + CD::BN) * 2 * BK;
    // with loader waves the MFMA waves have 256 registers: a 128x64 wave tile
    // fits a 2-stage ring, a 3-stage one's extra stage addresses spill
    return CD::MB == 16 && CD::kWaves == 4 && S * stage <= 160 * 1024 &&
           (!PROD || CD::FM * CD::FN <= (S == 2 ? 32 : 16));
}

template <class CD, int BK, int S, bool PROD>
hipError_t launch_ring_variant(const Params &p, hipStream_t stream) {
    if constexpr (ring_fits<CD, BK, S, PROD>()) {
        const dim3 grid((unsigned)((int64_t)p.num_m * p.num_n));
        return launch_kernel(gemm_f16_ring_kernel<CD, BK, S, PROD>, grid, dim3(CD::kThreads * (PROD ? 2 : 1)),
                             stream, p);
    } else {
        return hipErrorInvalidValue;
    }
}

template <class CD>
hipError_t launch_ring(int variant, const Params &p, hipStream_t stream) {
    switch (variant) {
        case 1: return launch_ring_variant<CD, 64, 2, false>(p, stream);
        case 2: return launch_ring_variant<CD, 64, 3, false>(p, stream);
        case 3: return launch_ring_variant<CD, 32, 2, false>(p, stream);
        case 4: return launch_ring_variant<CD, 32, 3, false>(p, stream);
        case 5: return launch_ring_variant<CD, 32, 4, false>(p, stream);
        case 6: return launch_ring_variant<CD, 64, 2, true>(p, stream);
        case 7: return launch_ring_variant<CD, 64, 3, true>(p, stream);
        default: return hipErrorInvalidValue;
    }
}

// One function per block tile, each in a translation unit of its own so the
// kernels compile in parallel.  nn selects the contract (false: C fp16 =
// A B^T; true: D fp32 = A B with B [K,N]); the 128x128 16x16x32 tile serves
// C = A B^T only.
hipError_t launch_256x256(bool nn, const Params &p, int g, int cus, hipStream_t s);
hipError_t launch_256x256_w8(bool nn, const Params &p, int g, int cus, hipStream_t s);
hipError_t launch_256x128(bool nn, const Params &p, int g, int cus, hipStream_t s);
hipError_t launch_128x256(bool nn, const Params &p, int g, int cus, hipStream_t s);
hipError_t launch_128x128(bool nn, const Params &p, int g, int cus, hipStream_t s);
hipError_t launch_128x128_m16(const Params &p, int g, int cus, hipStream_t s);
hipError_t launch_64x64(bool nn, const Params &p, int g, int cus, hipStream_t s);
hipError_t launch_64x128(bool nn, const Params &p, int g, int cus, hipStream_t s);
hipError_t launch_128x64(bool nn, const Params &p, int g, int cus, hipStream_t s);
// the ring kernel's variants on the 256x256, 256x128, 128x256 and 128x128 tiles
hipError_t launch_ring_256x256(int variant, const Params &p, hipStream_t s);
hipError_t launch_ring_256x128(int variant, const Params &p, hipStream_t s);
hipError_t launch_ring_128x256(int variant, const Params &p, hipStream_t s);
hipError_t launch_ring_128x128(int variant, const Params &p, hipStream_t s);

}  // namespace gemm_f16
