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

// Dispatch index -> logical index (bijection on [0, grid)).  I: the integer
// type of the arithmetic (the kernels take uint32_t: the host refuses grids
// of 2^31 tiles or more, and 64-bit division is a long instruction sequence
// on the GPU).
template <class I>
GEMM_HD I xcd_remap(I pid, I grid) {
    const I q = grid / kNumXcd;
    const I r = grid % kNumXcd;
    const I x = pid % kNumXcd;
    const I start = x * q + (x < r ? x : r);
    return start + pid / kNumXcd;
}

struct TileCoord {
    int64_t m_block;
    int64_t n_block;
};

template <class I>
GEMM_HD TileCoord tile_coord(I pid, I num_m, I num_n, I swizzle, bool xcd) {
    const I grid = num_m * num_n;
    const I logical = xcd ? xcd_remap<I>(pid, grid) : pid;
    // a group wider than the grid is the grid (same map), and keeps
    // num_m * swizzle within the grid's range
    if (swizzle > num_n) swizzle = num_n;
    const I per_group = num_m * swizzle;
    const I group = logical / per_group;
    const I first_n = group * swizzle;
    const I rest = num_n - first_n;
    const I width = rest < swizzle ? rest : swizzle;
    const I within = logical - group * per_group;
    TileCoord t;
    t.m_block = (int64_t)(within / width);
    t.n_block = (int64_t)(first_n + within % width);
    return t;
}

}  // namespace gemm_f16
