// Block-to-tile mapping of the GEMM kernels. Plain integer arithmetic with no
// device dependency, so that the mapping itself can be compiled and checked on
// the host (a bijection onto the tiles for every grid shape, the working tiles of
// a leading row range spread over the XCDs).
#pragma once

namespace cfm {

constexpr int GROUP_M = 4;   // block-rows per group of the tile walk

__host__ __device__ inline void tile_of(int bid, int nblocks, int tm, int tn, bool spread, int& mt, int& nt) {
    // The hardware deals block ids round-robin to the 8 XCDs (XCD x runs the ids
    // with id % 8 == x). With all rows valid, XCD x is given a contiguous range of
    // walk positions (a bijection for any block count), so it runs neighbouring
    // groups. With a device row count (spread: packed variable-length batches,
    // stopped guidance lanes) only a leading part of the rows does work; then the
    // walk position is the block id itself, so the working tiles, which come first
    // in the walk, are dealt evenly to all XCDs (and an XCD still sees one block-row
    // of each group against half of its columns when tn is even).
    const int q = nblocks / 8, rem = nblocks % 8;
    const int xcd = bid % 8, idx = bid / 8;
    const int b = spread ? bid : xcd * q + (xcd < rem ? xcd : rem) + idx;
    // the walk: groups of GROUP_M block-rows, column by column inside a group
    const int group = GROUP_M * tn;
    const int g = b / group, first_m = g * GROUP_M;
    const int gm = tm - first_m < GROUP_M ? tm - first_m : GROUP_M;
    const int in = b - g * group;
    mt = first_m + in % gm;
    nt = in / gm;
}

}  // namespace cfm
