// tile_order.h -- work-group id -> output tile, shared by the tiled kernels.
// Plain C++ when compiled without hipcc, so host tests can check the mapping.
#pragma once

#if defined(__HIPCC__)
#define SGEMM_HD __host__ __device__
#else
#define SGEMM_HD
#endif

namespace sgemm {

// Work-groups of one launch are handed to the 8 XCDs of the chip round-robin
// (work-group id p runs on XCD p % 8), and each XCD has its own L2.  This maps
// hardware id p of a launch of n work-groups to a virtual id such that every
// XCD owns one contiguous run of virtual ids.  A bijection on [0, n).
SGEMM_HD inline int xcd_remap(int pid, int n) {
    const int xcd = pid & 7, slot = pid >> 3;
    const int per = n >> 3, rem = n & 7;
    return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

// Virtual tile index -> (tile row, tile column), walking `group_m` tile-rows at
// a time so that consecutive indices share rows of A and columns of B.  A
// bijection from [0, tiles_m*tiles_n) onto the tile grid.
SGEMM_HD inline void group_tile(int logical, int tiles_m, int tiles_n, int group_m, int *tm,
                                int *tn) {
    const int group = group_m * tiles_n;
    const int g = logical / group;
    const int first_m = g * group_m;
    const int rows = tiles_m - first_m < group_m ? tiles_m - first_m : group_m;
    const int in_group = logical - g * group;
    *tm = first_m + in_group % rows;
    *tn = in_group / rows;
}

// One work-group per tile: the tiles resident on one XCD at a time form compact
// groups of C.  A bijection from [0, tiles_m*tiles_n) onto the tile grid.
SGEMM_HD inline void tile_order(int pid, int tiles_m, int tiles_n, int group_m, int *tm,
                                int *tn) {
    group_tile(xcd_remap(pid, tiles_m * tiles_n), tiles_m, tiles_n, group_m, tm, tn);
}

// The element of C owned by work-item (tx, ty) of work-group `block` in the
// rungs that compute one element per work-item (naive and LDS-tiled).  The
// work-groups cover C with tile_m x tile_n tiles numbered row by row, tiles_n
// to a tile row, so the 1-D id stands for the 2-D block (x = block % tiles_n,
// y = block / tiles_n); then, as in the tiled kernels of the pages, the row is
// y * tile_m + ty and the column x * tile_n + tx (page "【infra之路】Tiled
// Matrix Multiplication详解", the walk-through of the index computation: with
// a tile of 4, block (1, 2) and thread (3, 1) own row 9, column 7).
SGEMM_HD inline void element_of(int block, int tiles_n, int tile_m, int tile_n, int tx, int ty,
                                int *row, int *col) {
    const int bx = block % tiles_n, by = block / tiles_n;
    *row = by * tile_m + ty;
    *col = bx * tile_n + tx;
}

}  // namespace sgemm
