// Block-tile scheduler: 1D workgroup index -> (m_block, n_block).
//
// Shared by the kernels (device) and by gemm_f16_tile_coord (host), so the
// host-side tests check the very code the GPU runs.
//
// Two steps:
//  1. XCD remap (this library's addition).  The command processor hands
//     workgroups to the 8 XCDs of an MI355X round-robin, so dispatch index
//     p runs on XCD p % 8, and each XCD has its own L2.  Remapping p so that
//     XCD x owns the contiguous logical run [start_x, start_x + count_x)
//     makes the tiles that run together on one XCD neighbours in the
//     rasterized order below, so they share A and B strips in that XCD's L2.
//  2. Swizzled rasterization, from "4. Pipeline Abstraction and Two Consumer
//     Warp Groups" (Tilus tutorial), section "Tile Rasterization": the N axis
//     of the tile grid is cut into groups of `swizzle` tile-columns, tiles of
//     one group are handed out row-major (n fastest), and a narrower last
//     group keeps the map a bijection.  swizzle == 1 is the plain grid that
//     walks down M first.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define GEMM_HD __host__ __device__ __forceinline__
#else
#define GEMM_HD inline
#endif

namespace gemm_f16 {

constexpr int kNumXcd = 8;

// Dispatch index -> logical index (bijection on [0, grid)).
GEMM_HD int64_t xcd_remap(int64_t pid, int64_t grid) {
    const int64_t q = grid / kNumXcd;
    const int64_t r = grid % kNumXcd;
    const int64_t x = pid % kNumXcd;
    const int64_t start = x * q + (x < r ? x : r);
    return start + pid / kNumXcd;
}

struct TileCoord {
    int64_t m_block;
    int64_t n_block;
};

GEMM_HD TileCoord tile_coord(int64_t pid, int64_t num_m, int64_t num_n, int32_t swizzle, bool xcd) {
    const int64_t grid = num_m * num_n;
    const int64_t logical = xcd ? xcd_remap(pid, grid) : pid;
    const int64_t per_group = num_m * swizzle;
    const int64_t group = logical / per_group;
    const int64_t first_n = group * swizzle;
    const int64_t rest = num_n - first_n;
    const int64_t width = rest < swizzle ? rest : swizzle;
    const int64_t within = logical - group * per_group;
    TileCoord t;
    t.m_block = within / width;
    t.n_block = first_n + within % width;
    return t;
}

}  // namespace gemm_f16
