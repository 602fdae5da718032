// Host check of the single-launch forward's work queues (csrc/rmoe_sched.h,
// the same code the fused kernel runs), for both hand-over modes.
//
// Input on stdin: E NT1 NT2 mode seed, then per group its number of
// resident workgroups (8 numbers), then the E group sizes.  mode 1 = LOCAL
// (each XCD runs whole entries), mode 2 = GLOBAL (a pair's slices over all
// queues).  Prints "ok <tickets> <max wait depth>" or "FAIL <reason>",
// or "UNREACHABLE <detail>" when a down ticket was handed out while a
// gate/up ticket it needs sat in a queue that no running workgroup serves.
//
// Checked:
//   * coverage: every (block with valid rows, gate/up slice) and (block,
//     down slice) is run exactly once over all queues, with the right rows;
//   * LOCAL: the groups own disjoint, contiguous runs of entries covering
//     all of them, and every gate/up ticket of an entry comes before all of
//     its down tickets in the same queue;
//   * progress: a discrete-event run of the queues -- each resident
//     workgroup takes tickets of its own queue in order, a gate/up item
//     ends after a random time and counts into done[bx], a down item of the
//     pair at bx starts only once done[bx] reaches NT1 -- must finish every
//     ticket.  A queue with no resident workgroup is served, in LOCAL mode,
//     by the last workgroup out after all others have finished (as the
//     kernel does); in GLOBAL mode nobody serves it while the others wait.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../mixture_experts_routed_grouped_amd/csrc/rmoe_sched.h"

using namespace rmoe;

namespace {

constexpr int kGroups = 8;

struct Tk {
    bool down;
    TileItem it;
};

// The ticket list of queue g, exactly as serve_queue derives it.
std::vector<Tk> queue_of(int mode, const std::vector<int32_t> &gs, const std::vector<int32_t> &gpo,
                         int E, int NT1, int NT2, int g) {
    std::vector<Tk> q;
    if (mode == 1) {
        const FusedSeq fq = fused_seq(gs.data(), E, NT1, NT2, g, kGroups);
        TileCursor c1, c2;
        for (int t = 0; t < fq.n; ++t) {
            const FusedTicket k = fused_ticket(fq, t);
            if (k.j >= fq.J) continue;  // void ticket of the padded last unit (the kernel skips it)
            Tk x;
            x.down = k.down;
            x.it = entry_item(gs.data(), gpo.data(), fq.lo + k.j, k.nt, k.down ? c2 : c1);
            q.push_back(x);
        }
    } else {
        const TileSeq s1 = tile_seq(gs.data(), E, NT1, g, kGroups), s2 = tile_seq(gs.data(), E, NT2, g, kGroups);
        TileCursor c;
        for (int t = 0; t < s1.n + s2.n; ++t) {
            Tk x;
            x.down = t >= s1.n;
            x.it = x.down ? tile_item(gs.data(), gpo.data(), s2, t - s1.n, c)
                          : tile_item(gs.data(), gpo.data(), s1, t, c);
            q.push_back(x);
        }
    }
    return q;
}

}  // namespace

int main() {
    int E, NT1, NT2, mode;
    unsigned seed;
    if (std::scanf("%d %d %d %d %u", &E, &NT1, &NT2, &mode, &seed) != 5) return 2;
    int resident[kGroups];
    for (int g = 0; g < kGroups; ++g)
        if (std::scanf("%d", &resident[g]) != 1) return 2;
    std::vector<int32_t> gs(E), gpo(E + 1, 0);
    for (int e = 0; e < E; ++e)
        if (std::scanf("%d", &gs[e]) != 1) return 2;
    for (int e = 0; e < E; ++e) gpo[e + 1] = gpo[e] + (gs[e] / kItemRows + 1) * kItemRows;
    const int M = gpo[E] / kItemRows;

    std::vector<std::vector<Tk>> Q(kGroups);
    long tickets = 0;
    for (int g = 0; g < kGroups; ++g) {
        Q[g] = queue_of(mode, gs, gpo, E, NT1, NT2, g);
        tickets += (long)Q[g].size();
    }

    // ---- coverage of both stages
    std::vector<int> hit1((size_t)M * NT1, 0), hit2((size_t)M * NT2, 0);
    for (int g = 0; g < kGroups; ++g)
        for (const Tk &x : Q[g]) {
            const TileItem &it = x.it;
            const int NT = x.down ? NT2 : NT1;
            if (it.nt < 0 || it.nt >= NT || it.e < 0 || it.e >= E) {
                std::printf("FAIL range\n");
                return 1;
            }
            for (int b = 0; b < (it.rows1 > 0 ? 2 : 1); ++b) {
                const int bx = it.bx + b, off = bx * kItemRows - gpo[it.e];
                int rows = gs[it.e] - off;
                rows = rows < 0 ? 0 : (rows > kItemRows ? kItemRows : rows);
                if (off < 0 || bx >= M || rows <= 0 || rows != (b ? it.rows1 : it.rows0)) {
                    std::printf("FAIL rows bx=%d\n", bx);
                    return 1;
                }
                (x.down ? hit2 : hit1)[(size_t)bx * NT + it.nt] += 1;
            }
        }
    for (int bx = 0; bx < M; ++bx) {
        int e = 0;
        while (e + 1 < E && gpo[e + 1] <= bx * kItemRows) ++e;
        const int live = gs[e] - (bx * kItemRows - gpo[e]) > 0 ? 1 : 0;
        for (int nt = 0; nt < NT1; ++nt)
            if (hit1[(size_t)bx * NT1 + nt] != live) {
                std::printf("FAIL gate/up coverage bx=%d nt=%d\n", bx, nt);
                return 1;
            }
        for (int nt = 0; nt < NT2; ++nt)
            if (hit2[(size_t)bx * NT2 + nt] != live) {
                std::printf("FAIL down coverage bx=%d nt=%d\n", bx, nt);
                return 1;
            }
    }

    // ---- LOCAL: partition of the entries, and gate/up before down per entry
    if (mode == 1) {
        int P = 0;
        for (int e = 0; e < E; ++e) P += entries_of(gs.data(), e);
        int next = 0;
        for (int g = 0; g < kGroups; ++g) {
            const FusedSeq fq = fused_seq(gs.data(), E, NT1, NT2, g, kGroups);
            if (fq.J > 0 && fq.lo != next) {
                std::printf("FAIL partition g=%d lo=%d want %d\n", g, fq.lo, next);
                return 1;
            }
            next += fq.J;
            std::vector<int> last_gu(fq.J, -1), first_dn(fq.J, 1 << 30);
            std::vector<int> seen((size_t)fq.NU * RMOE_FUSED_UNIT * (NT1 + NT2), 0);
            for (int t = 0; t < fq.n; ++t) {
                const FusedTicket k = fused_ticket(fq, t);
                const int NT = k.down ? NT2 : NT1;
                if (k.j < 0 || k.j >= fq.NU * RMOE_FUSED_UNIT || k.nt < 0 || k.nt >= NT) {
                    std::printf("FAIL ticket range g=%d t=%d\n", g, t);
                    return 1;
                }
                // every (stage, entry, slice) of the padded units exactly once
                seen[(size_t)(k.down ? fq.NU * RMOE_FUSED_UNIT * NT1 + k.j * NT2 : k.j * NT1) + k.nt] += 1;
                if (k.j >= fq.J) continue;
                if (k.down)
                    first_dn[k.j] = first_dn[k.j] < t ? first_dn[k.j] : t;
                else
                    last_gu[k.j] = t;
            }
            for (size_t i = 0; i < seen.size(); ++i)
                if (seen[i] != 1) {
                    std::printf("FAIL ticket map g=%d slot %zu seen %d times\n", g, i, seen[i]);
                    return 1;
                }
            for (int j = 0; j < fq.J; ++j)
                if (!(last_gu[j] < first_dn[j])) {
                    std::printf("FAIL order g=%d entry %d: gate/up ticket %d after down ticket %d\n", g, j,
                                last_gu[j], first_dn[j]);
                    return 1;
                }
        }
        if (next != P) {
            std::printf("FAIL partition covers %d of %d entries\n", next, P);
            return 1;
        }
    }

    // ---- progress: discrete-event run of the queues
    std::mt19937 rng(seed);
    std::uniform_int_distribution<int> dur(1, 100);
    std::vector<int> done(M, 0);
    // where each pair's gate/up tickets live (queue ids), for the reachability check
    std::vector<std::vector<int>> gu_queues(M);
    for (int g = 0; g < kGroups; ++g)
        for (const Tk &x : Q[g])
            if (!x.down) gu_queues[x.it.bx].push_back(g);
    struct W {
        int g;
        int state;  // 0 idle, 1 busy, 2 waiting, 3 exited
        long until;
        Tk cur;
    };
    std::vector<W> ws;
    for (int g = 0; g < kGroups; ++g)
        for (int i = 0; i < resident[g]; ++i) ws.push_back({g, 0, 0, Tk{}});
    std::vector<size_t> head(kGroups, 0);
    long now = 0, finished = 0;
    int max_waiting = 0;
    bool drained_fallback = false;
    for (;;) {
        // idle workgroups take their next ticket
        for (W &w : ws) {
            while (w.state == 0) {
                if (head[w.g] >= Q[w.g].size()) {
                    w.state = 3;
                    break;
                }
                w.cur = Q[w.g][head[w.g]++];
                if (w.cur.down) {
                    // every gate/up ticket of its pair must be reachable: in
                    // a queue with a resident, not-yet-exited workgroup, or
                    // already handed out
                    for (int qg : gu_queues[w.cur.it.bx]) {
                        bool served = false;
                        for (const W &o : ws)
                            if (o.g == qg && o.state != 3) served = true;
                        bool handed = true;
                        for (size_t t = head[qg]; t < Q[qg].size(); ++t)
                            if (!Q[qg][t].down && Q[qg][t].it.bx == w.cur.it.bx) handed = false;
                        if (!served && !handed) {
                            std::printf("UNREACHABLE pair bx=%d needs queue %d (no resident workgroup)\n",
                                        w.cur.it.bx, qg);
                            return 3;
                        }
                    }
                    w.state = done[w.cur.it.bx] >= NT1 ? 1 : 2;
                } else {
                    w.state = 1;
                }
                if (w.state == 1) w.until = now + dur(rng);
            }
        }
        int busy = 0, waiting = 0, alive = 0;
        long next_t = -1;
        for (const W &w : ws) {
            if (w.state == 1) {
                ++busy;
                next_t = next_t < 0 || w.until < next_t ? w.until : next_t;
            }
            waiting += w.state == 2;
            alive += w.state != 3;
        }
        max_waiting = waiting > max_waiting ? waiting : max_waiting;
        if (alive == 0) {
            // the last workgroup out serves the queues nobody served (LOCAL)
            bool left = false;
            for (int g = 0; g < kGroups; ++g) left |= head[g] < Q[g].size();
            if (!left) break;
            if (mode != 1) {
                std::printf("FAIL tickets left with no workgroup\n");
                return 1;
            }
            for (int g = 0; g < kGroups; ++g)
                if (head[g] < Q[g].size()) {
                    ws.push_back({g, 0, 0, Tk{}});
                    drained_fallback = true;
                    break;
                }
            continue;
        }
        if (busy == 0) {
            std::printf("FAIL deadlock: %d workgroups waiting, none running\n", waiting);
            return 1;
        }
        now = next_t;
        for (W &w : ws)
            if (w.state == 1 && w.until == now) {
                if (!w.cur.down) done[w.cur.it.bx] += 1;
                ++finished;
                w.state = 0;
            }
        for (W &w : ws)
            if (w.state == 2 && done[w.cur.it.bx] >= NT1) {
                w.state = 1;
                w.until = now + dur(rng);
            }
    }
    if (finished != tickets) {
        std::printf("FAIL finished %ld of %ld tickets\n", finished, tickets);
        return 1;
    }
    std::printf("ok %ld %d%s\n", tickets, max_waiting, drained_fallback ? " fallback" : "");
    return 0;
}
