// Work items of the tiled grouped GEMM and the order the persistent
// workgroups take them in.  Plain C++ (host and device), so the same code
// that the kernels run can be checked for coverage on the CPU.
//
// A stage's work is every (block, weight slice) whose block holds valid rows
// (the row predicate of "Fused MoE GEMM 提交说明", 完整算子代码: a block
// with no rows does no work).  Blocks are taken two at a time: an expert's
// live blocks form ceil(live / 2) entries, a pair of consecutive blocks
// (256 tokens) or, for an odd count, its lone last block (run with the
// second half of the tile empty).  The item list is entry x weight slice,
// rectangle by rectangle of RMOE_TILE_GROUP slices, entries in expert order
// within a rectangle, the slices innermost, so that workgroups running
// neighbouring items share weight slices and token rows in L2.  Each
// locality group (XCD) owns a contiguous part of the list, taken round robin
// (or from a queue) by its workgroups.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define RMOE_HD __host__ __device__ __forceinline__
#else
#define RMOE_HD inline
#endif

#ifndef RMOE_TILE_GROUP
#define RMOE_TILE_GROUP 8  // weight slices per locality rectangle
#endif

namespace rmoe {

constexpr int kItemRows = 128;  // rows per contract block

struct TileItem {
    int nt;     // weight slice
    int e;      // expert
    int bx;     // first block
    int off;    // row offset of block bx inside its expert's rows
    int rows0;  // valid rows of block bx (>= 1)
    int rows1;  // valid rows of block bx + 1, 0 for a lone block
};

struct TileSeq {
    int NT;     // weight slices of the stage
    int P;      // entries (pairs and lone blocks) over all experts
    int lo, n;  // this group's part of the item list
};

// A position in the walk over experts: `base` entries belong to the experts
// before `e`.
struct TileCursor {
    int e = 0, base = 0;
};

RMOE_HD int live_blocks(const int32_t *gs, int e) { return (gs[e] + kItemRows - 1) / kItemRows; }
RMOE_HD int entries_of(const int32_t *gs, int e) { return (live_blocks(gs, e) + 1) / 2; }

// The part of locality group grp (of ngrp).
RMOE_HD TileSeq tile_seq(const int32_t *gs, int E, int NT, int grp, int ngrp) {
    TileSeq s;
    s.NT = NT;
    s.P = 0;
    for (int e = 0; e < E; ++e) s.P += entries_of(gs, e);
    const int tot = s.P * NT, per = (tot + ngrp - 1) / ngrp;
    s.lo = grp * per;
    s.n = tot - s.lo < per ? tot - s.lo : per;
    s.n = s.n < 0 ? 0 : s.n;
    return s;
}

// Item i of the group's part.  The cursor only moves forward while i does
// (and starts over when the entry index steps back, at a new rectangle), so
// a workgroup's walk over the experts is amortised over its items.
RMOE_HD TileItem tile_item(const int32_t *gs, const int32_t *gpo, const TileSeq &s, int i, TileCursor &c) {
    TileItem it;
    const int q = s.lo + i;
    const int gsz = RMOE_TILE_GROUP * s.P;
    const int g = q / gsz, r = q - g * gsz;
    const int width = s.NT - g * RMOE_TILE_GROUP < RMOE_TILE_GROUP ? s.NT - g * RMOE_TILE_GROUP : RMOE_TILE_GROUP;
    const int p = r / width;
    it.nt = g * RMOE_TILE_GROUP + (r - p * width);
    if (p < c.base) c = TileCursor();
    while (p >= c.base + entries_of(gs, c.e)) {
        c.base += entries_of(gs, c.e);
        ++c.e;
    }
    const int qq = p - c.base, n = gs[c.e];
    it.e = c.e;
    it.off = 2 * kItemRows * qq;
    it.bx = gpo[c.e] / kItemRows + 2 * qq;
    it.rows0 = n - it.off < kItemRows ? n - it.off : kItemRows;
    const int r1 = n - it.off - kItemRows;
    it.rows1 = r1 < 0 ? 0 : (r1 > kItemRows ? kItemRows : r1);
    return it;
}

}  // namespace rmoe
