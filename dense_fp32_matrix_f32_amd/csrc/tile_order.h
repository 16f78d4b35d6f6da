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
// the hardware order to a logical tile order in which every XCD owns one
// contiguous run of logical ids, and walks the logical ids in groups of
// `group_m` tile-rows so that the tiles resident on one XCD at a time share
// rows of A and columns of B.  The map is a bijection on [0, tiles_m*tiles_n).
SGEMM_HD inline void tile_order(int pid, int tiles_m, int tiles_n, int group_m,
                                int *tm, int *tn) {
    const int nwg = tiles_m * tiles_n;
    const int xcd = pid & 7, slot = pid >> 3;
    const int per = nwg >> 3, rem = nwg & 7;
    const int logical = xcd < rem ? xcd * (per + 1) + slot
                                  : rem * (per + 1) + (xcd - rem) * per + slot;
    const int group = group_m * tiles_n;
    const int g = logical / group;
    const int first_m = g * group_m;
    const int rows = tiles_m - first_m < group_m ? tiles_m - first_m : group_m;
    const int in_group = logical - g * group;
    *tm = first_m + in_group % rows;
    *tn = in_group / rows;
}

}  // namespace sgemm
