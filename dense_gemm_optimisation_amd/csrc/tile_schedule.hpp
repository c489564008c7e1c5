// Workgroup -> output-tile mapping for the GEMM kernels.
//
// The grid is one-dimensional: one workgroup per (batch, tile row, tile
// column).  Two remappings improve cache reuse; both are bijections for every
// grid, so each output tile is computed exactly once.
//
// 1. XCD grouping.  MI355X has 8 accelerator complex dies (XCDs), each with
//    its own L2, and the dispatcher hands consecutive workgroup ids to the
//    XCDs round-robin (id % 8).  Workgroup w is therefore re-numbered so that
//    the ids one XCD receives form one contiguous range of logical tiles:
//    neighbouring tiles, which share rows of A and columns of B, then run on
//    the same L2.
// 2. Grouped rasterisation.  Logical tiles are walked in groups of `group_m`
//    tile rows: down a column of the group first, then to the next column.
//    A group of G rows by the grid's width reuses G panels of A from L2
//    instead of one.  This is the thread-block swizzle of section 1 of the
//    hgemm sm120 article (wingedge777.com) and the rasterisation discussed in
//    "GPU GEMM 优化完全拆解（三）" (pinghaoyang.com.cn), section on
//    rasterization and split-K.  The article's formula assumes a grid width
//    that is a multiple of the swizzle width; here the last group is allowed
//    to be partial, which keeps the map a bijection for any grid.
#pragma once

#include <cstdint>

#if !defined(__HIPCC__)
#ifndef __host__
#define __host__
#endif
#ifndef __device__
#define __device__
#endif
#endif

namespace libgemm {

struct TileGrid {
    int64_t tiles_m;  // tile rows    (ceil(M / BM))
    int64_t tiles_n;  // tile columns (ceil(N / BN))
    int64_t batch;
    int32_t group_m;  // tile rows per rasterisation group (>= 1)
    int32_t xcds;     // XCDs workgroups are dealt to round-robin (>= 1)

    __host__ __device__ int64_t per_batch() const { return tiles_m * tiles_n; }
    __host__ __device__ int64_t count() const { return tiles_m * tiles_n * batch; }
};

struct TileCoord {
    int64_t batch;
    int64_t tm;  // tile row
    int64_t tn;  // tile column
};

// XCD x receives ids x, x + X, x + 2X, ...: it gets q or q + 1 of them
// (q = total / X, the first `total % X` XCDs one more).  The k-th id an XCD
// receives becomes logical id start(x) + k, so each XCD owns one contiguous
// block of logical ids.
__host__ __device__ inline int64_t xcd_remap(int64_t wg, int64_t total, int32_t xcds) {
    if (xcds <= 1) return wg;
    const int64_t x = wg % xcds;
    const int64_t k = wg / xcds;
    const int64_t q = total / xcds;
    const int64_t r = total % xcds;
    const int64_t start = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
    return start + k;
}

__host__ __device__ inline TileCoord tile_of(const TileGrid &g, int64_t wg) {
    const int64_t id = xcd_remap(wg, g.count(), g.xcds);
    TileCoord t;
    const int64_t pb = g.per_batch();
    t.batch = id / pb;
    const int64_t local = id - t.batch * pb;
    const int64_t gm = g.group_m < 1 ? 1 : g.group_m;
    const int64_t in_group = gm * g.tiles_n;          // tiles in one full group
    const int64_t group = local / in_group;
    const int64_t first_m = group * gm;
    const int64_t rows = g.tiles_m - first_m < gm ? g.tiles_m - first_m : gm;  // last group may be short
    const int64_t r = local - group * in_group;
    t.tm = first_m + r % rows;
    t.tn = r / rows;
    return t;
}

}  // namespace libgemm
