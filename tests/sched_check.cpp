// Host check of the tiled kernels' work sequence (csrc/rmoe_sched.h, the
// same code the kernels run): every (block with valid rows, weight slice)
// must be computed exactly once, by an item whose rows match the block.
// Input on stdin: E NT ngrp lanes, then the E group sizes.  Prints
// "ok <items> <largest part>" or "FAIL <reason>".
#include <cstdio>
#include <vector>

#include "../mixture_experts_routed_grouped_amd/csrc/rmoe_sched.h"

using namespace rmoe;

int main() {
    int E, NT, ngrp, lanes;
    if (std::scanf("%d %d %d %d", &E, &NT, &ngrp, &lanes) != 4) return 2;
    std::vector<int32_t> gs(E), gpo(E + 1, 0);
    for (int e = 0; e < E; ++e)
        if (std::scanf("%d", &gs[e]) != 1) return 2;
    // padded starts: each expert owns floor(count / 128) + 1 blocks
    for (int e = 0; e < E; ++e) gpo[e + 1] = gpo[e] + (gs[e] / kItemRows + 1) * kItemRows;
    const int M = gpo[E] / kItemRows;
    std::vector<int> hits((size_t)M * NT, 0);
    long items = 0;
    int largest = 0;
    for (int g = 0; g < ngrp; ++g) {
        const TileSeq s = tile_seq(gs.data(), E, NT, g, ngrp);
        largest = s.n > largest ? s.n : largest;
        // walk as the workgroups do: lane l takes l, l + lanes, ... with its
        // own cursors; then again in one increasing walk (a queue) that
        // revisits from 0 to exercise the cursor reset
        for (int pass = 0; pass < 2; ++pass) {
            for (int l = 0; l < (pass == 0 ? lanes : 1); ++l) {
                TileCursor c;
                for (int i = l; i < s.n; i += (pass == 0 ? lanes : 1)) {
                    const TileItem it = tile_item(gs.data(), gpo.data(), s, i, c);
                    if (it.nt < 0 || it.nt >= NT || it.e < 0 || it.e >= E) {
                        std::printf("FAIL range g=%d i=%d\n", g, i);
                        return 1;
                    }
                    const int nblk = it.rows1 > 0 ? 2 : 1;
                    for (int b = 0; b < nblk; ++b) {
                        const int bx = it.bx + b;
                        const int rel = bx - gpo[it.e] / kItemRows;
                        const int off = kItemRows * rel;
                        int rows = gs[it.e] - off;
                        rows = rows < 0 ? 0 : (rows > kItemRows ? kItemRows : rows);
                        const int got = b ? it.rows1 : it.rows0;
                        if (rel < 0 || bx >= M || rows <= 0 || got != rows ||
                            (b == 0 && it.off != off)) {
                            std::printf("FAIL rows g=%d i=%d bx=%d rows=%d got=%d\n", g, i, bx, rows, got);
                            return 1;
                        }
                        if (pass == 0) hits[(size_t)bx * NT + it.nt] += 1;
                    }
                    // a lone block is its expert's last live block
                    if (it.rows1 == 0 && it.rows0 + it.off != gs[it.e]) {
                        std::printf("FAIL lone block not last g=%d i=%d\n", g, i);
                        return 1;
                    }
                    if (pass == 0) ++items;
                }
            }
        }
    }
    for (int bx = 0; bx < M; ++bx) {
        int e = 0;
        while (e + 1 < E && gpo[e + 1] <= bx * kItemRows) ++e;
        const int off = bx * kItemRows - gpo[e];
        const int live = gs[e] - off > 0 ? 1 : 0;
        for (int nt = 0; nt < NT; ++nt)
            if (hits[(size_t)bx * NT + nt] != live) {
                std::printf("FAIL coverage bx=%d nt=%d hits=%d want=%d\n", bx, nt,
                            hits[(size_t)bx * NT + nt], live);
                return 1;
            }
    }
    std::printf("ok %ld %d\n", items, largest);
    return 0;
}
