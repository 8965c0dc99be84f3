// libmfma_ceiling: the sustained v_mfma_f32_32x32x16_f16 throughput of one
// MI355X with no global memory traffic, as the practical MFMA ceiling the
// GEMM's roofline fraction is read against.
//
// One workgroup of 4 waves per CU; each wave holds a 128x128 fp32
// accumulator tile (4 x 4 blocks of 32x32, 256 AGPRs, as in the GEMM) and
// runs 16 MFMAs per 16-wide k step in the GEMM's snake order.  Variant 0
// re-reads the step's 4 + 4 operand fragments from LDS every step (double
// buffered, as the GEMM's fragment reads are); variant 1 keeps them in
// registers.  Variants 2 and 3 are the same on v_mfma_f32_16x16x32_f16
// (8 x 8 blocks of 16x16 per wave, 64 MFMAs per 32-wide k step) with the
// accumulators tied in AGPRs, as the GEMM's 256x256 direct-to-LDS kernel
// runs them.  The operands are whatever the caller's table holds (random
// fp16 values, zeros, ...): the MFMA clock depends on their switching
// activity.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "mfma_ceiling.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kTable = MFMA_CEILING_TABLE_ENTRIES;  // 16-byte entries, 64 KB

template <bool LDS_READS>
__global__ __launch_bounds__(256) void ceiling_kernel(const half8 *table, float *out, int64_t iters) {
    __shared__ half8 lds[kTable];
    for (int i = threadIdx.x; i < kTable; i += 256) lds[i] = table[(i + blockIdx.x * 97) & (kTable - 1)];
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int base = (wave * 1024 + lane) & (kTable - 1);
    half8 af[2][4], bf[2][4];
    floatx16 acc[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = floatx16{};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        af[0][q] = lds[(base + 64 * q) & (kTable - 1)];
        bf[0][q] = lds[(base + 256 + 64 * q) & (kTable - 1)];
    }
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            // the fragments of the next step, from another part of the table
            const int nxt = (base + (int)((it * 2 + s + 1) & 7) * 512) & (kTable - 1);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (LDS_READS) {
                    af[s ^ 1][q] = lds[(nxt + 64 * q) & (kTable - 1)];
                    bf[s ^ 1][q] = lds[(nxt + 256 + 64 * q) & (kTable - 1)];
                } else {
                    af[s ^ 1][q] = af[s][q];
                    bf[s ^ 1][q] = bf[s][q];
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int i = (j & 1) ? 3 - ii : ii;
                    acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[s][j], af[s][i], acc[j][i], 0, 0, 0);
                }
        }
    }
    // one value per thread keeps every accumulator live
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) sum += acc[j][i][r];
    out[blockIdx.x * 256 + threadIdx.x] = sum;
}

// v_mfma_f32_16x16x32_f16 with the accumulator tied to itself in AGPRs (the
// builtin's untied form makes the register allocator rotate 64 accumulator
// blocks through the AGPRs with copies).  The compiler sees no MFMA in the
// asm: fence() puts 24 wait states between the accumulators' other
// accesses and the first / after the last MFMA.
__device__ __forceinline__ void mfma16(half8 a, half8 b, floatx4 &c) {
    asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

__device__ __forceinline__ void fence(floatx4 (&acc)[8][8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) asm volatile("" : "+a"(acc[j][i]));
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) asm volatile("" : "+a"(acc[j][i]));
}

// One iteration = one 32-wide k step: 64 MFMAs, the same flops as two
// 16-wide steps of the 32x32x16 kernel.
template <bool LDS_READS>
__global__ __launch_bounds__(256) void ceiling16_kernel(const half8 *table, float *out, int64_t iters) {
    __shared__ half8 lds[kTable];
    for (int i = threadIdx.x; i < kTable; i += 256) lds[i] = table[(i + blockIdx.x * 97) & (kTable - 1)];
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int base = (wave * 1024 + lane) & (kTable - 1);
    half8 af[2][8], bf[2][8];
    floatx4 acc[8][8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[j][i] = floatx4{};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        af[0][q] = lds[(base + 64 * q) & (kTable - 1)];
        bf[0][q] = lds[(base + 512 + 64 * q) & (kTable - 1)];
    }
    fence(acc);
    auto step = [&](int s, int64_t it) {
        const int nxt = (base + (int)((it + 1) & 7) * 512) & (kTable - 1);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (LDS_READS) {
                af[s ^ 1][q] = lds[(nxt + 64 * q) & (kTable - 1)];
                bf[s ^ 1][q] = lds[(nxt + 512 + 64 * q) & (kTable - 1)];
            } else {
                af[s ^ 1][q] = af[s][q];
                bf[s ^ 1][q] = bf[s][q];
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int ii = 0; ii < 8; ++ii) {
                const int i = (j & 1) ? 7 - ii : ii;
                mfma16(bf[s][j], af[s][i], acc[j][i]);
            }
    };
    int64_t it = 0;
    for (; it + 1 < iters; it += 2) {
        step(0, it);
        step(1, it + 1);
    }
    if (it < iters) step(0, it);
    fence(acc);
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) sum += acc[j][i][r];
    out[blockIdx.x * 256 + threadIdx.x] = sum;
}

}  // namespace

extern "C" int mfma_ceiling_launch(int variant, int64_t iters, int32_t workgroups, const void *table,
                                   float *out, void *stream) {
    if (variant < 0 || variant > 3 || iters < 1 || workgroups < 1) return -1;
    if (!table || !out) return -2;
    if (((uintptr_t)table & 15) || ((uintptr_t)out & 3)) return -3;
    hipStream_t s = (hipStream_t)stream;
    const dim3 grid((unsigned)workgroups), block(256);
    const half8 *t = (const half8 *)table;
    switch (variant) {
        case 0: hipLaunchKernelGGL(ceiling_kernel<true>, grid, block, 0, s, t, out, iters); break;
        case 1: hipLaunchKernelGGL(ceiling_kernel<false>, grid, block, 0, s, t, out, iters); break;
        case 2: hipLaunchKernelGGL(ceiling16_kernel<true>, grid, block, 0, s, t, out, iters); break;
        default: hipLaunchKernelGGL(ceiling16_kernel<false>, grid, block, 0, s, t, out, iters); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" double mfma_ceiling_flops(int64_t iters, int32_t workgroups) {
    // per wave and iteration: 2 k steps x 16 MFMAs x 2*32*32*16 flop
    return (double)iters * 2.0 * 16.0 * 32768.0 * 4.0 * (double)workgroups;
}
