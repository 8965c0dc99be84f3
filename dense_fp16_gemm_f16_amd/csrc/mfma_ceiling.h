/*
 * mfma_ceiling.h - C ABI of libmfma_ceiling.so, a measurement probe (not part
 * of the GEMM): the sustained v_mfma_f32_32x32x16_f16 and
 * v_mfma_f32_16x16x32_f16 rates of the device with no global memory traffic
 * in the loop, on operand values the caller chooses.
 * It is the practical ceiling against which the GEMM's fraction of the
 * published dense fp16 peak is read (the MFMA clock falls with the switching
 * activity of the operands).
 */
#ifndef MFMA_CEILING_H
#define MFMA_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* entries of 8 fp16 values (16 bytes) in the operand table: 64 KB */
#define MFMA_CEILING_TABLE_ENTRIES 4096

/*
 * Enqueue one launch on `stream` (hipStream_t as void*; NULL = null stream):
 * `workgroups` workgroups of 4 waves (use one per CU), each wave running
 * `iters` iterations on a 128x128 fp32 tile.  Variants 0 and 1: an iteration
 * is two 16-wide k steps of 16 v_mfma_f32_32x32x16_f16; variants 2 and 3:
 * one 32-wide k step of 64 v_mfma_f32_16x16x32_f16 with the accumulators
 * tied in AGPRs (the same flops).  Variants 0 and 2 re-read the operand
 * fragments from LDS every k step; 1 and 3 keep them in registers.
 *   table  device pointer, 16-byte aligned, MFMA_CEILING_TABLE_ENTRIES x 16
 *          bytes of fp16 operand values (copied to LDS, read by every wave)
 *   out    device pointer, workgroups * 256 floats (sums that keep the
 *          accumulators live; their values carry no meaning)
 * Returns 0, -1 for a bad variant / count, -2 for a null pointer, -3 for a
 * misaligned pointer, -5 if the launch failed.  Asynchronous; allocates
 * nothing.
 */
int mfma_ceiling_launch(int variant, int64_t iters, int32_t workgroups, const void *table,
                        float *out, void *stream);

/* Floating-point operations of one launch with these arguments (2 per MAC). */
double mfma_ceiling_flops(int64_t iters, int32_t workgroups);

#ifdef __cplusplus
}
#endif

#endif /* MFMA_CEILING_H */
