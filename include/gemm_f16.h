/*
 * gemm_f16.h - C ABI of the MI355X (gfx950) fp16 GEMM library libgemm_f16.so.
 *
 * The operation is the tiled dense GEMM of the Tilus Hopper matmul tutorial,
 * "1. WGMMA: Hopper's Asynchronous Tensor Core", section "The Full Kernel":
 *
 *     C[m][n] = fp16( sum_{k<K} A[m][k] * B[n][k] )      0 <= m < M, 0 <= n < N
 *
 * with A viewed as [M,K] and B as [N,K] (the product uses B transposed), an
 * fp32 accumulator that starts at zero, and one cast of the accumulator to
 * fp16 (round to nearest, ties to even) before C is stored.  C is
 * overwritten; there is no alpha/beta.
 *
 * Layouts (all dense, no strides):
 *   a  fp16 [M,K] row-major      element (m,k) at a[m*K + k]
 *   b  fp16 [N,K] row-major      element (n,k) at b[n*K + k]   ("K-major")
 *   c  fp16 [M,N] row-major      element (m,n) at c[m*N + n]
 * fp16 is IEEE 754 binary16.  Pointers are device pointers (memory the HIP
 * runtime allocated on the current device, e.g. through PyTorch).
 *
 * Ownership: the caller owns every buffer.  The library allocates no device
 * memory, keeps no pointer after the call returns and needs no workspace.
 * c must not overlap a or b.
 *
 * Asynchrony: the work is enqueued on `stream` (a hipStream_t passed as
 * void*; NULL is the null stream) and the call returns without waiting.
 * Completion is the caller's business (stream or event synchronisation).
 *
 * Threads: every entry point may be called from several host threads at
 * once.  The only state the library keeps is a per-device cache of the
 * device's architecture and compute-unit count, filled on first use, and
 * per host thread the XCD setting of the last grid of one tile per CU
 * (gemm_f16_select_xcd).
 *
 * Errors: every entry point returns 0 on success or one of the negative
 * GEMM_F16_E* codes below; gemm_f16_status_string() names them.  Argument
 * checks run before any HIP call, so an invalid call has no effect.  The
 * library never exits the process.
 */
#ifndef GEMM_F16_H
#define GEMM_F16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    GEMM_F16_OK = 0,
    GEMM_F16_EINVAL = -1,     /* negative size, M or N >= 2^30, M*N >= 2^47, K >= 2^22, bad option */
    GEMM_F16_ENULL = -2,      /* null pointer with a non-empty extent */
    GEMM_F16_EALIGN = -3,     /* pointer not aligned to its element size (2 or 4 bytes) */
    GEMM_F16_EDEVICE = -4,    /* current device is not gfx950 */
    GEMM_F16_EHIP = -5,       /* a HIP runtime call or the kernel launch failed */
    GEMM_F16_EOVERLAP = -6    /* the output overlaps a or b */
};

/*
 * C = fp16(A * B^T) with fp32 accumulation (see the top of this file).
 *
 * m, n, k >= 0; m, n < 2^30; m*n < 2^47; k < 2^22.
 * m == 0 or n == 0: returns GEMM_F16_OK and launches nothing.
 * k == 0: C is filled with +0 (the zero accumulator is stored).
 * Sizes that are not multiples of the block tile are handled: elements of A
 * and B outside [M,K] / [N,K] are read as zero and elements of C outside
 * [M,N] are never written.
 * Speed: K % 8 == 0 with 16-byte aligned A and B loads the operands straight
 * into LDS; any other K or alignment goes through registers, at roughly
 * 0.55-0.7 of that speed on large shapes.
 */
int gemm_f16_nt(int64_t m, int64_t n, int64_t k, const void *a, const void *b,
                void *c, void *stream);

/*
 * Launch options for gemm_f16_nt_ex (tuning, determinism tests).
 *   tile     0 = automatic choice by shape; otherwise one of the
 *            GEMM_F16_TILE_* block-tile configurations.
 *   swizzle  tile-columns per rasterization group (the swizzle_size of
 *            "4. Pipeline Abstraction and Two Consumer Warp Groups", section
 *            "Tile Rasterization"); 0 = library default, 1 = plain grid.
 *   xcd      1 = give each of the 8 XCDs a contiguous run of tiles,
 *            0 = hardware dispatch order, -1 = library default
 *            (gemm_f16_select_xcd).
 *   variant  0 = the library's kernels.  1..7 = a kernel whose K-tile width
 *            (block_k), LDS ring depth and wave roles are those of the
 *            GEMM_F16_VARIANT_* below, one tile per workgroup (the tuning
 *            sweep's axes; "4. Pipeline Abstraction and Two Consumer Warp
 *            Groups", sections "Pipeline Depth" and "Two Consumer Warp
 *            Groups").  A variant needs C = A B^T, an explicit block tile of
 *            256x256 (variants 1, 3, 4, 5 only), 256x128 or 128x256 (not
 *            variant 7), or 128x128, K a positive multiple of its block_k,
 *            and 16-byte aligned A and B; otherwise the call returns
 *            GEMM_F16_EINVAL.
 * Every option but the variant changes only the schedule: the fp32 sum of
 * each output is taken in the same order, so results are bitwise identical
 * across options that select the same block tile.
 */
typedef struct {
    int32_t tile;
    int32_t swizzle;
    int32_t xcd;
    int32_t variant;
} gemm_f16_options;

enum {
    GEMM_F16_VARIANT_DEFAULT = 0,
    GEMM_F16_VARIANT_BK64_S2 = 1,      /* block_k 64, 2 LDS stages, every wave loads */
    GEMM_F16_VARIANT_BK64_S3 = 2,      /* block_k 64, 3 stages */
    GEMM_F16_VARIANT_BK32_S2 = 3,      /* block_k 32, 2 stages */
    GEMM_F16_VARIANT_BK32_S3 = 4,      /* block_k 32, 3 stages */
    GEMM_F16_VARIANT_BK32_S4 = 5,      /* block_k 32, 4 stages */
    GEMM_F16_VARIANT_PRODUCER_S2 = 6,  /* block_k 64, 2 stages, 4 loader waves + 4 MFMA waves */
    GEMM_F16_VARIANT_PRODUCER_S3 = 7,  /* block_k 64, 3 stages, 4 loader waves + 4 MFMA waves */
    GEMM_F16_VARIANT_LAST = 7
};

enum {
    GEMM_F16_TILE_AUTO = 0,
    GEMM_F16_TILE_256x256 = 1,     /* 4 waves, each 128x128 of C */
    GEMM_F16_TILE_128x128 = 2,     /* 4 waves, each 64x64 of C */
    GEMM_F16_TILE_64x64 = 3,       /* 4 waves, each 32x32 of C */
    GEMM_F16_TILE_256x256_W8 = 4,  /* 8 waves, each 64x128 of C */
    GEMM_F16_TILE_256x128 = 5,     /* 4 waves, each 128x64 of C */
    GEMM_F16_TILE_128x256 = 6,     /* 4 waves, each 64x128 of C */
    GEMM_F16_TILE_128x128_M16 = 7, /* 4 waves, each 64x64 of C, on v_mfma_f32_16x16x32_f16 */
    GEMM_F16_TILE_64x128 = 8,      /* 4 waves, each 32x64 of C */
    GEMM_F16_TILE_128x64 = 9,      /* 4 waves, each 64x32 of C */
    GEMM_F16_TILE_LAST = 9
};

/* gemm_f16_nt with explicit options; opt == NULL means all defaults. */
int gemm_f16_nt_ex(int64_t m, int64_t n, int64_t k, const void *a, const void *b,
                   void *c, void *stream, const gemm_f16_options *opt);

/*
 * The second contract, that of the day-78 listing "wgmma_gemm.cu" (its
 * kernel, its B layout and its fp32 output):
 *
 *     D[m][n] = sum_{k<K} A[m][k] * B[k][n]      fp32 accumulation, fp32 out
 *
 *   a  fp16 [M,K] row-major      element (m,k) at a[m*K + k]
 *   b  fp16 [K,N] row-major      element (k,n) at b[k*N + n]
 *   d  fp32 [M,N] row-major      element (m,n) at d[m*N + n], 4-byte aligned
 *
 * D is the fp32 accumulator itself (no rounding to fp16).  Same sizes,
 * ownership, asynchrony and error rules as gemm_f16_nt, plus n < 2^25;
 * k == 0 fills D with +0.  Options as for gemm_f16_nt_ex, except that
 * GEMM_F16_TILE_128x128_M16 is not available (GEMM_F16_EINVAL).
 */
int gemm_f16_nn_f32(int64_t m, int64_t n, int64_t k, const void *a, const void *b,
                    void *d, void *stream);
int gemm_f16_nn_f32_ex(int64_t m, int64_t n, int64_t k, const void *a, const void *b,
                       void *d, void *stream, const gemm_f16_options *opt);

/* Static message for a status code (never NULL). */
const char *gemm_f16_status_string(int status);

/*
 * Host-side copy of the block-tile scheduler the kernels run (same source):
 * workgroup index `pid` of a grid of num_m*num_n tiles -> (m_block, n_block).
 * With xcd != 0 the dispatch index is first remapped so each of the 8 XCDs
 * gets a contiguous run of tiles; the tiles are then grouped `swizzle`
 * tile-columns wide and handed out row-major inside a group ("4. Pipeline
 * Abstraction and Two Consumer Warp Groups", section "Tile Rasterization").
 * Returns GEMM_F16_EINVAL for num_m or num_n below 1, a grid of 2^63
 * tiles or more, pid outside the grid or swizzle < 1.
 * Pure host function: no HIP call.
 */
int gemm_f16_tile_coord(int64_t pid, int64_t num_m, int64_t num_n, int32_t swizzle,
                        int32_t xcd, int64_t *m_block, int64_t *n_block);

/*
 * Block tile the automatic choice would use for (m, n, k) on the current
 * device: one of GEMM_F16_TILE_*, or a negative status for invalid sizes.
 * Asks HIP for the device's compute-unit count (once per device); with no
 * device it assumes 256.
 */
int gemm_f16_select_tile(int64_t m, int64_t n, int64_t k);

/*
 * The xcd option that xcd = -1 stands for, on a grid of num_m x num_n
 * block tiles rasterized `swizzle` tile-columns wide, on a device of `cus`
 * compute units: 1 (remap) except on a grid of exactly `cus` tiles whose
 * dispatch order leaves no XCD more operand panels (distinct tile rows
 * plus tile columns) than the remap does; then 0.  Returns
 * GEMM_F16_EINVAL for num_m, num_n or swizzle below 1, cus below 0, or a
 * grid of 2^31 tiles or more.  Pure host function: no HIP call.
 */
int gemm_f16_select_xcd(int64_t num_m, int64_t num_n, int32_t swizzle, int32_t cus);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_F16_H */
