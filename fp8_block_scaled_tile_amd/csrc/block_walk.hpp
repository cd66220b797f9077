// block_walk.hpp -- the order in which the quantizers' work-groups take the
// 128x128 blocks of a matrix (nrb block rows, ncb block columns).
//
// Every quantizer kernel launches one work-group per block on a 1-D grid;
// a block's codes and scales do not depend on the order, only the memory
// traffic of the work-groups in flight together does.  Two walks:
//
//   grouped:  groups of `group_rows` block rows, column block by column block
//             inside a group, so the work-groups in flight read a few
//             contiguous row bands and write contiguous runs of the
//             transposed copy.  A plain row- or column-major walk
//             concentrates the reads or the transposed writes on a few HBM
//             channels when rows are 8 KB or more apart.
//
//   XCD tiles: the MI355X deals the work-groups of a launch round-robin to
//             its 8 XCDs (accelerator complexes, each with its own L2), so
//             work-group b runs on XCD b % 8.  XCD x walks its own tile of
//             tile_rows x tile_cols blocks, rows first; the 8 tiles sit
//             side by side as xcd_rows x (8 / xcd_rows) tiles, and these
//             super tiles walk across a band of block rows, then the next
//             band.  Each XCD then writes runs of both the row codes and
//             the transposed codes from one L2, where the grouped walk
//             deals the pieces of one transposed run to eight.  Measured on
//             32768-row activations: dual quantizer 3-10% faster at 6144 to
//             16384 columns, column-only 9-12%, row-only from 3% slower
//             (6144) to 4% faster (16384); no gain at 2048 columns, which
//             keep the grouped walk.
//
// Both are permutations of the blocks (a host-side check covers the shapes
// the launchers pick them for); on a device that deals work-groups
// differently the XCD walk is still a valid order, only a slower one.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace puro {

struct BlockRC {
    int64_t rb, cb;
};

struct BlockWalk {
    int group_rows;      // grouped walk (used when tile_rows == 0)
    int tile_rows;       // XCD walk: blocks per XCD tile, down the rows
    int tile_cols;       //           and across the columns
    int xcd_rows;        //           XCD tiles stacked along rows: 1, 2, 4 or 8
};

// Group height of the grouped walk (measured on MI355X): 4 for weights, 16
// for activations up to 2048 columns, 8 for wider ones.
inline int quant_group_rows(bool weight, int64_t cols)
{
    if (weight)
        return 4;
    return cols <= 2048 ? 16 : 8;
}

// The walk for an activation-shaped launch of nrb x ncb blocks: XCD tiles of
// 4 x 4 blocks, stacked 1 high from 64 block columns on (8192 columns and
// wider) and 2 high from 32 (6144), when the blocks divide into whole super
// tiles; otherwise the grouped walk with `group_rows`.
inline BlockWalk act_walk(int group_rows, int64_t nrb, int64_t ncb)
{
    BlockWalk w{group_rows, 0, 0, 0};
    if (ncb < 32)
        return w;
    const int xr = ncb >= 64 ? 1 : 2;
    const int tr = 4, tc = 4;
    if (nrb % (tr * xr) == 0 && ncb % (tc * (8 / xr)) == 0) {
        w.tile_rows = tr;
        w.tile_cols = tc;
        w.xcd_rows = xr;
    }
    return w;
}

__host__ __device__ inline BlockWalk grouped_walk(int group_rows)
{
    return BlockWalk{group_rows, 0, 0, 0};
}

// Block (rb, cb) taken by work-group `bid` of the nrb x ncb launch.
__host__ __device__ inline BlockRC block_of(int64_t bid, int64_t nrb, int64_t ncb, const BlockWalk& w)
{
    if (w.tile_rows > 0) {
        const int64_t x = bid & 7;                 // the XCD
        const int64_t p = bid >> 3;                // its position in the XCD's sequence
        const int64_t per_tile = (int64_t)w.tile_rows * w.tile_cols;
        const int64_t tile = p / per_tile, k = p - tile * per_tile;
        const int64_t xc = 8 / w.xcd_rows;
        const int64_t st_rows = (int64_t)w.tile_rows * w.xcd_rows;
        const int64_t st_cols = (int64_t)w.tile_cols * xc;
        const int64_t per_band = ncb / st_cols;
        const int64_t band = tile / per_band, sc = tile - band * per_band;
        return BlockRC{band * st_rows + (x % w.xcd_rows) * w.tile_rows + k % w.tile_rows,
                       sc * st_cols + (x / w.xcd_rows) * w.tile_cols + k / w.tile_rows};
    }
    const int64_t per_group = (int64_t)w.group_rows * ncb;
    const int64_t group = bid / per_group;
    const int64_t j = bid - group * per_group;
    const int64_t left = nrb - group * w.group_rows;
    const int64_t gr = left < w.group_rows ? left : w.group_rows;
    const int64_t cb = j / gr;
    return BlockRC{group * w.group_rows + (j - cb * gr), cb};
}

}  // namespace puro
