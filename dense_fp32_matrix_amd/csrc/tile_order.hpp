// Output-tile order of the tiled kernels, shared with the host-side check
// (tests/layout_check.cpp), which compiles this header as plain C++.
#pragma once

#if defined(__HIPCC__)
#define SGEMM_TILE_HD __host__ __device__ __forceinline__
#else
#define SGEMM_TILE_HD inline
#endif

namespace sgemm_impl {

// Workgroup -> output tile.  Consecutive workgroup ids are dispatched
// round-robin over the chip's 8 XCDs (each with its own L2), so id b is first
// renumbered so that every XCD receives one contiguous range of logical
// tiles; logical tiles are then walked in groups of group_m tile rows,
// column by column, so the tiles one XCD holds at a time share rows of A
// and columns of B.  group_m == 0 selects the plain row-major order instead
// (tile b is row b / tiles_n, column b % tiles_n), for comparison.
SGEMM_TILE_HD void tile_coords(int bid, int tiles_m, int tiles_n, int group_m, int* tm, int* tn) {
    if (group_m == 0) {
        *tm = bid / tiles_n;
        *tn = bid - *tm * tiles_n;
        return;
    }
    const int total = tiles_m * tiles_n;
    const int xcd = bid % 8;
    const int local = bid / 8;
    const int per = total / 8;
    const int rem = total % 8;
    const int t = xcd * per + (xcd < rem ? xcd : rem) + local;
    const int span = group_m * tiles_n;
    const int group = t / span;
    const int first_m = group * group_m;
    const int gm = tiles_m - first_m < group_m ? tiles_m - first_m : group_m;
    const int within = t - group * span;
    *tm = first_m + within % gm;
    *tn = within / gm;
}

}  // namespace sgemm_impl
