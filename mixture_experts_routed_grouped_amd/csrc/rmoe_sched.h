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

// ---- Single launch with the hidden hand-over kept inside one locality
// group (XCD).  Every entry (a pair of blocks or a lone last block) belongs
// to exactly one group, which runs all of its gate/up slices and then all of
// its down slices, so the hidden rows a down tile reads were written by the
// same XCD and never have to leave its L2.  Groups own contiguous runs of
// entries in expert order, cut where the running cost crosses g * C / ngrp
// (cost of an entry: 2 + its 32-row token tiles, a fixed part for the item's
// prologue and epilogue plus the MFMA work).  A group's entries are taken in
// units of RMOE_FUSED_UNIT consecutive entries; a unit's gate/up tickets
// run slice by slice over its entries (so neighbouring workgroups share a
// weight slice), then, RMOE_FUSED_LAG units later in the queue, its down
// tickets the same way: the gate/up tickets of the first `lag` units, then
// for each later unit v its gate/up tickets followed by the down tickets of
// unit v - lag, then the remaining down tickets.  So every gate/up ticket
// of an entry comes before any of its down tickets in the same queue: a
// workgroup that holds a down ticket waits only for tickets already handed
// to running workgroups of its own group.  The last unit is padded to the
// unit size with void tickets (entries past the group's run) that do nothing.
#ifndef RMOE_FUSED_UNIT
#define RMOE_FUSED_UNIT 2
#endif
#ifndef RMOE_FUSED_LAG
#define RMOE_FUSED_LAG 1
#endif

struct FusedSeq {
    int NT1, NT2;  // gate/up and down slices per entry
    int lo, J;     // this group's entries: global entries lo .. lo + J - 1
    int NU;        // units of RMOE_FUSED_UNIT entries (the last one padded)
    int n;         // tickets: NU * RMOE_FUSED_UNIT * (NT1 + NT2)
};

struct FusedTicket {
    bool down;  // false: a gate/up slice, true: a down slice
    int j;      // entry within the group (>= J: a void ticket of the padded last unit)
    int nt;     // slice
};

RMOE_HD int entry_cost(int n, int qq) {
    const int off = 2 * kItemRows * qq;
    int r0 = n - off, r1 = n - off - kItemRows;
    r0 = r0 > kItemRows ? kItemRows : r0;
    r1 = r1 < 0 ? 0 : (r1 > kItemRows ? kItemRows : r1);
    return 2 + (r0 + 31) / 32 + (r1 + 31) / 32;
}

RMOE_HD FusedSeq fused_seq(const int32_t *gs, int E, int NT1, int NT2, int grp, int ngrp) {
    FusedSeq s;
    s.NT1 = NT1;
    s.NT2 = NT2;
    int64_t C = 0;
    for (int e = 0; e < E; ++e)
        for (int qq = 0; qq < entries_of(gs, e); ++qq) C += entry_cost(gs[e], qq);
    s.lo = 0;
    s.J = 0;
    int64_t run = 0;
    int q = 0;
    for (int e = 0; e < E; ++e)
        for (int qq = 0; qq < entries_of(gs, e); ++qq, ++q) {
            const int g = (int)(run * ngrp / (C > 0 ? C : 1));  // group of the entry starting at `run`
            if (g < grp) s.lo = q + 1;
            if (g == grp) ++s.J;
            run += entry_cost(gs[e], qq);
        }
    s.NU = (s.J + RMOE_FUSED_UNIT - 1) / RMOE_FUSED_UNIT;
    s.n = s.NU * RMOE_FUSED_UNIT * (NT1 + NT2);
    return s;
}

RMOE_HD FusedTicket fused_ticket(const FusedSeq &s, int t) {
    constexpr int U = RMOE_FUSED_UNIT;
    const int L = s.NU < RMOE_FUSED_LAG ? s.NU : RMOE_FUSED_LAG;
    const int g1 = U * s.NT1, g2 = U * s.NT2;  // tickets of one unit's gate/up, down
    int v, i;                                   // unit, ticket within that unit's stage
    FusedTicket k;
    if (t < L * g1) {
        k.down = false;
        v = t / g1;
        i = t % g1;
    } else if ((t -= L * g1) < (s.NU - L) * (g1 + g2)) {
        const int r = t % (g1 + g2);
        k.down = r >= g1;
        v = L + t / (g1 + g2) - (k.down ? L : 0);
        i = k.down ? r - g1 : r;
    } else {
        t -= (s.NU - L) * (g1 + g2);
        k.down = true;
        v = s.NU - L + t / g2;
        i = t % g2;
    }
    // slice by slice over the unit's entries
    k.nt = i / U;
    k.j = v * U + i % U;
    return k;
}

// Global entry q (in expert order) as a work item of slice nt; the cursor
// only moves forward while q does and starts over when q steps back.
RMOE_HD TileItem entry_item(const int32_t *gs, const int32_t *gpo, int q, int nt, TileCursor &c) {
    if (q < c.base) c = TileCursor();
    while (q >= c.base + entries_of(gs, c.e)) {
        c.base += entries_of(gs, c.e);
        ++c.e;
    }
    TileItem it;
    const int qq = q - c.base, n = gs[c.e];
    it.nt = nt;
    it.e = c.e;
    it.off = 2 * kItemRows * qq;
    it.bx = gpo[c.e] / kItemRows + 2 * qq;
    it.rows0 = n - it.off < kItemRows ? n - it.off : kItemRows;
    const int r1 = n - it.off - kItemRows;
    it.rows1 = r1 < 0 ? 0 : (r1 > kItemRows ? kItemRows : r1);
    return it;
}

}  // namespace rmoe
