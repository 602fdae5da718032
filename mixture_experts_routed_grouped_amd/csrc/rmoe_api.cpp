// C-ABI entry points of the routed fused-MoE library: host-side dispatch
// contract, its validator, argument checking and kernel dispatch.  Nothing
// here allocates device memory, synchronises, or reads device tables.
#include "../../include/routed_moe.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "rmoe_internal.h"

namespace {

constexpr int64_t B = RMOE_BLOCK_M;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
constexpr int32_t kMaxDeviceExperts = 8192;  // the device contract keeps per-expert tables in LDS
// default bound on how long a fused down tile waits for its pair's hidden
// rows (the longest real wait is one gate/up stage: milliseconds)
constexpr int64_t kFusedWaitUs = 2000000;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Shape checks shared by the forward and the two stage entry points.
int check_dims(int64_t hidden, int64_t intermediate, int32_t num_experts,
               int64_t total_padded_tokens, int32_t num_blocks_m) {
    if (hidden <= 0 || intermediate <= 0 || num_experts < 1 || num_blocks_m < 0 ||
        total_padded_tokens < 0)
        return RMOE_ERR_INVALID_ARGUMENT;
    if (hidden % 128 != 0 || intermediate % 128 != 0) return RMOE_ERR_UNSUPPORTED_SHAPE;
    if ((int64_t)num_blocks_m * B > total_padded_tokens) return RMOE_ERR_INVALID_ARGUMENT;
    if (num_blocks_m > 65535) return RMOE_ERR_UNSUPPORTED_SHAPE;  // grid y limit
    if (hidden > (int64_t)1 << 20 || intermediate > (int64_t)1 << 20)
        return RMOE_ERR_UNSUPPORTED_SHAPE;
    return RMOE_OK;
}

// Kernel family: the weight-streaming family when experts hold few rows on
// average (then a weight byte serves a handful of tokens and the stage is
// HBM-bound), the LDS-tiled family otherwise.  A streaming block takes the
// narrowest pass of 32, 64 or 96 tokens that holds its rows (96 then 32 for
// 97-128 rows), so blocks of up to 96 rows read their weights once; a group
// of g rows reads its expert's weights about g/64 times beyond that.
//
// Average threshold by expert count, from forward times of both families
// (one MI355X, uniform and Zipf routing, 16-112 rows per expert):
//   E <= 4: 96 rows -- the tiled family has very few work items (E=4,
//     H=4096: 64 down-stage items for 256 CUs); E=4 (4096, 14336) streams
//     14-42% faster at 48-96, tiles 13-14% faster at 112;
//   E <= 8: 56 -- at 56, E=8 (4096, 14336) streams 15% faster (uniform) and
//     1-4% (Zipf 1.2), (6144, 16384) 1-4%; at 64 the Zipf batch tiles 9%
//     faster;
//   E < 32: 32 -- E=16 (4096, 14336) tiles up to 5% faster at 40-48
//     uniform, 7% from 40 under Zipf;
//   E >= 32: 36 -- E=64 (2048, 1408) streams 2-4% faster at 36 and tiles
//     2% faster at 42; E=128 (7168, 2048) tiles 4-6% faster at 40 (E=32
//     (4096, 2048) streams faster up to 64 rows, 18% at 40).
// When the caller knows the largest group (max_group_rows >= 0, from host
// tables):
//   * with fewer than 32 experts streaming also needs every group to fit
//     one 128-row block: the few experts' extra weight reads then weigh on
//     the whole batch (E=16 Zipf 1.2, 40 rows per expert, largest group 197:
//     tiling 7% faster).  With 32 or more experts the extra reads of the
//     large groups are a small share (E=128 Zipf 1.2 at 8-32 rows, largest
//     group 120-485: streaming 2-18% faster; E=64 Zipf 1.1 at 24-36,
//     largest 219-330: 4-9%);
//   * batches of at most 32 experts whose every group fits one pass stream
//     whatever their average while the largest group is at most 64 rows,
//     and up to 96 rows at an average of at most 80 (E <= 8) or 48 rows:
//     each weight byte is then read once, while the tiled family has too
//     few work items (E=8 (4096, 14336) at 64-80 rows, largest 75-94:
//     streaming 5-15% faster, (2048, 5632) 41-52%, (6144, 16384) between
//     2% faster and 8% slower; E=32 (4096, 2048) at 40-48, largest 57-72:
//     14-18% faster; E=16 (4096, 14336) at 40-48, largest 51-62: within 5%
//     either way).
constexpr int64_t kStreamMaxGroupRows = B;
constexpr int32_t kManyExperts = 32;
int64_t stream_max_avg_rows(int32_t num_experts) {
    return num_experts <= 4 ? 96 : num_experts <= 8 ? 56 : num_experts < kManyExperts ? 32 : 36;
}
int pick_variant(int32_t variant, int64_t pairs, int32_t num_experts, int64_t max_group_rows = -1) {
    if (variant == RMOE_VARIANT_STREAM || variant == RMOE_VARIANT_TILE) return variant;
    const int32_t E = num_experts;
    const bool few = pairs <= stream_max_avg_rows(E) * (int64_t)E;
    const bool fits = max_group_rows < 0 || max_group_rows <= kStreamMaxGroupRows || E >= kManyExperts;
    const bool one_pass =
        max_group_rows >= 0 && E <= kManyExperts &&
        (max_group_rows <= 64 || (max_group_rows <= 96 && pairs <= (E <= 8 ? 80 : 48) * (int64_t)E));
    return (few && fits) || one_pass ? RMOE_VARIANT_STREAM : RMOE_VARIANT_TILE;
}
int to_status(hipError_t e) { return e == hipSuccess ? RMOE_OK : RMOE_ERR_LAUNCH; }

// Hand-over of the single launch.  AUTO hands hidden rows across XCDs: the
// XCD-local hand-over is correct on every shape but measured slower on all
// workloads (large 14.0 against 10.9 ms, fine 1.28-1.36 against 0.92 ms):
// a write-back L2 still writes every hidden row out, and running each
// entry's slices on one XCD raises the operand traffic beyond L2 by ~20%.
int pick_handover(int32_t handover) {
    return handover == RMOE_FUSED_LOCAL ? RMOE_FUSED_LOCAL : RMOE_FUSED_GLOBAL;
}
int gate_up_impl(const void *x, const void *gate_w, const void *up_w, const int32_t *gs,
                 const int32_t *gpo, const int32_t *gidx, void *workspace, int64_t hidden,
                 int64_t intermediate, int32_t E, int64_t Tp, int32_t M, int64_t pairs,
                 int32_t variant, void *stream) {
    rmoe::StageArgs a{};
    a.x = static_cast<const _Float16 *>(x);
    a.w0 = static_cast<const _Float16 *>(gate_w);
    a.w1 = static_cast<const _Float16 *>(up_w);
    a.gs = gs;
    a.gpo = gpo;
    a.gidx = gidx;
    a.y = static_cast<_Float16 *>(workspace);
    a.K = hidden;
    a.N = intermediate;
    a.E = E;
    a.M = M;
    a.pairs = pairs;
    (void)Tp;
    if (M == 0) return RMOE_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (pick_variant(variant, pairs, E) == RMOE_VARIANT_STREAM)
        return to_status(rmoe::launch_stream_gate_up(a, s));
    return to_status(rmoe::launch_tile_gate_up(a, s));
}

int down_impl(const void *workspace, const void *down_w, const float *rw, const int32_t *gs,
              const int32_t *go, const int32_t *gpo, const int32_t *gidx, void *out,
              int64_t hidden, int64_t intermediate, int32_t E, int64_t Tp, int32_t M,
              int64_t pairs, int32_t variant, void *stream) {
    rmoe::StageArgs a{};
    a.x = static_cast<const _Float16 *>(workspace);
    a.w0 = static_cast<const _Float16 *>(down_w);
    a.rw = rw;
    a.gs = gs;
    a.go = go;
    a.gpo = gpo;
    a.gidx = gidx;
    a.y = static_cast<_Float16 *>(out);
    a.K = intermediate;
    a.N = hidden;
    a.E = E;
    a.M = M;
    a.pairs = pairs;
    (void)Tp;
    if (M == 0) return RMOE_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (pick_variant(variant, pairs, E) == RMOE_VARIANT_STREAM)
        return to_status(rmoe::launch_stream_down(a, s));
    return to_status(rmoe::launch_tile_down(a, s));
}

bool bad_variant(int32_t v) {
    return v != RMOE_VARIANT_AUTO && v != RMOE_VARIANT_STREAM && v != RMOE_VARIANT_TILE;
}

}  // namespace

extern "C" {

const char *rmoe_status_str(int status) {
    switch (status) {
        case RMOE_OK: return "ok";
        case RMOE_ERR_INVALID_ARGUMENT: return "invalid argument";
        case RMOE_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
        case RMOE_ERR_MISALIGNED: return "misaligned pointer";
        case RMOE_ERR_LAUNCH: return "kernel launch failed";
        case RMOE_ERR_CONTRACT: return "tables violate the dispatch contract";
        case RMOE_ERR_CAPACITY: return "output table too small";
        case RMOE_ERR_SCRATCH: return "batch exceeds the library's static scratch";
        default: return "unknown status";
    }
}

const char *rmoe_version(void) { return "routed_moe 0.1 gfx950"; }

int rmoe_build_contract(const int32_t *topk_ids, int64_t num_tokens, int32_t top_k,
                        int32_t num_experts, int32_t *group_sizes, int32_t *group_offsets,
                        int32_t *group_padded_offsets, int32_t *group_idx_for_bx,
                        int64_t capacity_blocks, int32_t *num_blocks_m, int32_t *order,
                        int32_t *padded_row_of_pair, int32_t *compact_pos_of_pair) {
    if (num_tokens < 0 || top_k < 0 || num_experts < 1 || !group_sizes || !group_offsets ||
        !group_padded_offsets || !num_blocks_m || (num_tokens > 0 && top_k > 0 && !topk_ids))
        return RMOE_ERR_INVALID_ARGUMENT;
    const int64_t pairs = num_tokens * top_k;
    if (pairs > INT32_MAX / 2) return RMOE_ERR_INVALID_ARGUMENT;
    const int32_t E = num_experts;
    // every padded row index (up to 128*M) must fit the int32 tables
    const int64_t M = ceil_div(pairs, B) + E;
    if (M * B > INT32_MAX) return RMOE_ERR_INVALID_ARGUMENT;
    if (capacity_blocks < M || (M > 0 && !group_idx_for_bx)) return RMOE_ERR_CAPACITY;
    // counts (and id range check before anything is written)
    std::vector<int64_t> cnt(E, 0);
    for (int64_t p = 0; p < pairs; ++p) {
        const int32_t e = topk_ids[p];
        if (e < 0 || e >= E) return RMOE_ERR_INVALID_ARGUMENT;
        cnt[e]++;
    }
    // compact and padded offsets (E+1 entries each)
    group_offsets[0] = 0;
    group_padded_offsets[0] = 0;
    for (int32_t e = 0; e < E; ++e) {
        group_sizes[e] = (int32_t)cnt[e];
        group_offsets[e + 1] = group_offsets[e] + (int32_t)cnt[e];
        group_padded_offsets[e + 1] = group_padded_offsets[e] + (int32_t)(ceil_div(cnt[e] + 1, B) * B);
    }
    *num_blocks_m = (int32_t)M;
    // block -> last expert whose padded start is <= bx*128 (starts strictly increase)
    int32_t e = 0;
    for (int64_t bx = 0; bx < M; ++bx) {
        while (e + 1 < E && (int64_t)group_padded_offsets[e + 1] <= bx * B) ++e;
        group_idx_for_bx[bx] = e;
    }
    // stable counting sort of the pairs by expert
    std::vector<int32_t> next(group_offsets, group_offsets + E);
    for (int64_t p = 0; p < pairs; ++p) {
        const int32_t ex = topk_ids[p];
        const int32_t c = next[ex]++;
        const int32_t rank = c - group_offsets[ex];
        if (order) order[c] = (int32_t)p;
        if (padded_row_of_pair) padded_row_of_pair[p] = group_padded_offsets[ex] + rank;
        if (compact_pos_of_pair) compact_pos_of_pair[p] = c;
    }
    return RMOE_OK;
}

int rmoe_validate_contract(const int32_t *gs, const int32_t *go, const int32_t *gpo,
                           const int32_t *gidx, int32_t E, int32_t M, int64_t Tp, int64_t pairs) {
    if (!gs || !go || !gpo || E < 1 || M < 0 || (M > 0 && !gidx)) return RMOE_ERR_INVALID_ARGUMENT;
    if (go[0] != 0 || gpo[0] != 0) return RMOE_ERR_CONTRACT;
    for (int32_t e = 0; e < E; ++e) {
        if (gs[e] < 0) return RMOE_ERR_CONTRACT;
        if ((int64_t)go[e + 1] - go[e] != gs[e]) return RMOE_ERR_CONTRACT;
        if ((int64_t)gpo[e + 1] - gpo[e] != ((int64_t)gs[e] / B + 1) * B) return RMOE_ERR_CONTRACT;
    }
    if ((int64_t)go[E] != pairs) return RMOE_ERR_CONTRACT;
    if ((int64_t)M != ceil_div(pairs, B) + E) return RMOE_ERR_CONTRACT;
    if ((int64_t)gpo[E] > (int64_t)M * B || (int64_t)M * B > Tp) return RMOE_ERR_CONTRACT;
    int32_t e = 0;
    for (int64_t bx = 0; bx < M; ++bx) {
        while (e + 1 < E && (int64_t)gpo[e + 1] <= bx * B) ++e;
        if (gidx[bx] != e) return RMOE_ERR_CONTRACT;
    }
    return RMOE_OK;
}

size_t rmoe_workspace_bytes(int64_t total_padded_tokens, int64_t intermediate) {
    if (total_padded_tokens <= 0 || intermediate <= 0) return 0;
    return (size_t)total_padded_tokens * (size_t)intermediate * 2u;
}

int rmoe_contract_sizes(int64_t num_pairs, int32_t num_experts, int32_t *num_blocks_m,
                        int64_t *total_padded_tokens) {
    if (num_pairs < 0 || num_experts < 1 || num_pairs > INT32_MAX / 2)
        return RMOE_ERR_INVALID_ARGUMENT;
    const int64_t M = ceil_div(num_pairs, B) + num_experts;
    if (M * B > INT32_MAX) return RMOE_ERR_INVALID_ARGUMENT;
    if (num_blocks_m) *num_blocks_m = (int32_t)M;
    if (total_padded_tokens) *total_padded_tokens = M * B;
    return RMOE_OK;
}

int rmoe_pick_variant(int32_t variant, int64_t num_pairs, int32_t num_experts,
                      int64_t max_group_rows) {
    if (bad_variant(variant) || num_pairs < 0 || num_experts < 1 || max_group_rows > num_pairs)
        return RMOE_ERR_INVALID_ARGUMENT;
    return pick_variant(variant, num_pairs, num_experts, max_group_rows);
}

int rmoe_validate_contract_device(const int32_t *gs, const int32_t *go, const int32_t *gpo,
                                  const int32_t *gidx, int32_t num_experts, int32_t num_blocks_m,
                                  int64_t total_padded_tokens, int64_t total_valid_tokens,
                                  int32_t *violations, void *stream) {
    if (!gs || !go || !gpo || !violations || num_experts < 1 || num_blocks_m < 0 ||
        total_valid_tokens < 0 || (num_blocks_m > 0 && !gidx))
        return RMOE_ERR_INVALID_ARGUMENT;
    if (!aligned4(gs) || !aligned4(go) || !aligned4(gpo) || !aligned4(gidx) || !aligned4(violations))
        return RMOE_ERR_MISALIGNED;
    // the size rules need no table: they are checked here, synchronously
    if (total_valid_tokens > INT32_MAX / 2 ||
        (int64_t)num_blocks_m != ceil_div(total_valid_tokens, B) + num_experts ||
        (int64_t)num_blocks_m * B > total_padded_tokens)
        return RMOE_ERR_CONTRACT;
    return to_status(rmoe::launch_validate(gs, go, gpo, gidx, num_experts, num_blocks_m,
                                           total_valid_tokens, violations,
                                           static_cast<hipStream_t>(stream)));
}

int rmoe_gate_up_f16(const void *x, const void *gate_w, const void *up_w, const int32_t *gs,
                     const int32_t *gpo, const int32_t *gidx, void *workspace, int64_t hidden,
                     int64_t intermediate, int32_t num_experts, int64_t total_padded_tokens,
                     int64_t total_valid_tokens, int32_t num_blocks_m, int32_t variant,
                     void *stream) {
    int st = check_dims(hidden, intermediate, num_experts, total_padded_tokens, num_blocks_m);
    if (st != RMOE_OK) return st;
    if (bad_variant(variant) || total_valid_tokens < 0) return RMOE_ERR_INVALID_ARGUMENT;
    if (!x || !gate_w || !up_w || !gs || !gpo || !workspace || (num_blocks_m > 0 && !gidx))
        return RMOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(x) || !aligned16(gate_w) || !aligned16(up_w) || !aligned16(workspace) ||
        !aligned4(gs) || !aligned4(gpo) || !aligned4(gidx))
        return RMOE_ERR_MISALIGNED;
    // the same family choice as rmoe_down_f16 and the forward for this batch
    return gate_up_impl(x, gate_w, up_w, gs, gpo, gidx, workspace, hidden, intermediate,
                        num_experts, total_padded_tokens, num_blocks_m, total_valid_tokens,
                        variant, stream);
}

int rmoe_down_f16(const void *workspace, const void *down_w, const float *rw, const int32_t *gs,
                  const int32_t *go, const int32_t *gpo, const int32_t *gidx, void *out,
                  int64_t hidden, int64_t intermediate, int32_t num_experts,
                  int64_t total_padded_tokens, int64_t total_valid_tokens, int32_t num_blocks_m,
                  int32_t variant, void *stream) {
    int st = check_dims(hidden, intermediate, num_experts, total_padded_tokens, num_blocks_m);
    if (st != RMOE_OK) return st;
    if (bad_variant(variant) || total_valid_tokens < 0) return RMOE_ERR_INVALID_ARGUMENT;
    if (!workspace || !down_w || !gs || !go || !gpo || !out || (num_blocks_m > 0 && !gidx) ||
        (total_valid_tokens > 0 && !rw))
        return RMOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(workspace) || !aligned16(down_w) || !aligned16(out) || !aligned4(rw) ||
        !aligned4(gs) || !aligned4(go) || !aligned4(gpo) || !aligned4(gidx))
        return RMOE_ERR_MISALIGNED;
    return down_impl(workspace, down_w, rw, gs, go, gpo, gidx, out, hidden, intermediate,
                     num_experts, total_padded_tokens, num_blocks_m, total_valid_tokens, variant,
                     stream);
}

int rmoe_forward_f16_variant(const void *x, const void *gate_w, const void *up_w,
                             const void *down_w, const float *rw, const int32_t *gs,
                             const int32_t *go, const int32_t *gpo, const int32_t *gidx,
                             void *workspace, void *out, int64_t hidden, int64_t intermediate,
                             int32_t num_experts, int64_t total_padded_tokens,
                             int64_t total_valid_tokens, int32_t num_blocks_m, int32_t variant,
                             void *stream) {
    int st = check_dims(hidden, intermediate, num_experts, total_padded_tokens, num_blocks_m);
    if (st != RMOE_OK) return st;
    if (bad_variant(variant) || total_valid_tokens < 0) return RMOE_ERR_INVALID_ARGUMENT;
    if (!x || !gate_w || !up_w || !down_w || !gs || !go || !gpo || !workspace || !out ||
        (num_blocks_m > 0 && !gidx) || (total_valid_tokens > 0 && !rw))
        return RMOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(x) || !aligned16(gate_w) || !aligned16(up_w) || !aligned16(down_w) ||
        !aligned16(workspace) || !aligned16(out) || !aligned4(rw) || !aligned4(gs) ||
        !aligned4(go) || !aligned4(gpo) || !aligned4(gidx))
        return RMOE_ERR_MISALIGNED;
    const int v = pick_variant(variant, total_valid_tokens, num_experts);
    st = gate_up_impl(x, gate_w, up_w, gs, gpo, gidx, workspace, hidden, intermediate,
                      num_experts, total_padded_tokens, num_blocks_m, total_valid_tokens, v,
                      stream);
    if (st != RMOE_OK) return st;
    return down_impl(workspace, down_w, rw, gs, go, gpo, gidx, out, hidden, intermediate,
                     num_experts, total_padded_tokens, num_blocks_m, total_valid_tokens, v,
                     stream);
}

int rmoe_forward_f16(const void *x, const void *gate_w, const void *up_w, const void *down_w,
                     const float *rw, const int32_t *gs, const int32_t *go, const int32_t *gpo,
                     const int32_t *gidx, void *workspace, void *out, int64_t hidden,
                     int64_t intermediate, int32_t num_experts, int64_t total_padded_tokens,
                     int64_t total_valid_tokens, int32_t num_blocks_m, void *stream) {
    return rmoe_forward_f16_variant(x, gate_w, up_w, down_w, rw, gs, go, gpo, gidx, workspace,
                                    out, hidden, intermediate, num_experts, total_padded_tokens,
                                    total_valid_tokens, num_blocks_m, RMOE_VARIANT_AUTO, stream);
}

size_t rmoe_fused_sync_words(int32_t num_blocks_m) {
    return num_blocks_m < 0 ? 0 : (size_t)RMOE_FUSED_SYNC_HEAD + (size_t)num_blocks_m;
}

int rmoe_forward_fused_f16(const void *x, const void *gate_w, const void *up_w,
                           const void *down_w, const float *rw, const int32_t *gs,
                           const int32_t *go, const int32_t *gpo, const int32_t *gidx,
                           void *workspace, void *out, int32_t *sync, int64_t hidden,
                           int64_t intermediate, int32_t num_experts, int64_t total_padded_tokens,
                           int64_t total_valid_tokens, int32_t num_blocks_m, int32_t max_wait_us,
                           int32_t handover, void *stream) {
    int st = check_dims(hidden, intermediate, num_experts, total_padded_tokens, num_blocks_m);
    if (st != RMOE_OK) return st;
    if (total_valid_tokens < 0 || handover < RMOE_FUSED_AUTO || handover > RMOE_FUSED_GLOBAL)
        return RMOE_ERR_INVALID_ARGUMENT;
    if (!x || !gate_w || !up_w || !down_w || !gs || !go || !gpo || !workspace || !out || !sync ||
        (num_blocks_m > 0 && !gidx) || (total_valid_tokens > 0 && !rw))
        return RMOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(x) || !aligned16(gate_w) || !aligned16(up_w) || !aligned16(down_w) ||
        !aligned16(workspace) || !aligned16(out) || !aligned4(rw) || !aligned4(gs) ||
        !aligned4(go) || !aligned4(gpo) || !aligned4(gidx) || !aligned4(sync))
        return RMOE_ERR_MISALIGNED;
    if (num_blocks_m == 0) return RMOE_OK;
    rmoe::StageArgs gu{}, dn{};
    gu.x = static_cast<const _Float16 *>(x);
    gu.w0 = static_cast<const _Float16 *>(gate_w);
    gu.w1 = static_cast<const _Float16 *>(up_w);
    gu.y = static_cast<_Float16 *>(workspace);
    gu.K = hidden;
    gu.N = intermediate;
    dn.x = static_cast<const _Float16 *>(workspace);
    dn.w0 = static_cast<const _Float16 *>(down_w);
    dn.rw = rw;
    dn.y = static_cast<_Float16 *>(out);
    dn.K = intermediate;
    dn.N = hidden;
    for (rmoe::StageArgs *a : {&gu, &dn}) {
        a->gs = gs;
        a->go = go;
        a->gpo = gpo;
        a->gidx = gidx;
        a->E = num_experts;
        a->M = num_blocks_m;
        a->pairs = total_valid_tokens;
    }
    const int64_t wait_us = max_wait_us > 0 ? max_wait_us : kFusedWaitUs;
    const bool local = pick_handover(handover) == RMOE_FUSED_LOCAL;
    return to_status(
        rmoe::launch_fused(gu, dn, sync, wait_us, local, static_cast<hipStream_t>(stream)));
}

int rmoe_pack_f16(const void *x, const float *topk_weights, const int32_t *prow,
                  const int32_t *cpos, int64_t num_tokens, int32_t top_k, int64_t hidden,
                  void *stacked, float *w_compact, int64_t total_padded_tokens, void *stream) {
    if (num_tokens < 0 || top_k < 0 || hidden <= 0 || total_padded_tokens < 0)
        return RMOE_ERR_INVALID_ARGUMENT;
    if (hidden % 8 != 0 || hidden / 8 > ((int64_t)1 << 30)) return RMOE_ERR_UNSUPPORTED_SHAPE;
    const int64_t pairs = num_tokens * top_k;
    if (pairs == 0) return RMOE_OK;
    if (!x || !topk_weights || !prow || !cpos || !stacked || !w_compact)
        return RMOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(x) || !aligned16(stacked) || !aligned4(topk_weights) || !aligned4(prow) ||
        !aligned4(cpos) || !aligned4(w_compact))
        return RMOE_ERR_MISALIGNED;
    return to_status(rmoe::launch_pack(static_cast<const _Float16 *>(x), topk_weights, prow, cpos,
                                       pairs, top_k, hidden, total_padded_tokens,
                                       static_cast<_Float16 *>(stacked), w_compact,
                                       static_cast<hipStream_t>(stream)));
}

int rmoe_combine_f16(const void *out, const int32_t *prow, int64_t num_tokens, int32_t top_k,
                     int64_t hidden, void *y, int64_t total_padded_tokens, void *stream) {
    if (num_tokens < 0 || top_k < 0 || hidden <= 0 || total_padded_tokens < 0)
        return RMOE_ERR_INVALID_ARGUMENT;
    if (hidden % 8 != 0 || hidden / 8 > ((int64_t)1 << 30)) return RMOE_ERR_UNSUPPORTED_SHAPE;
    if (num_tokens == 0) return RMOE_OK;
    if (!y || (top_k > 0 && (!out || !prow))) return RMOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(y) || !aligned16(out) || !aligned4(prow)) return RMOE_ERR_MISALIGNED;
    return to_status(rmoe::launch_combine(static_cast<const _Float16 *>(out), prow, num_tokens,
                                          top_k, hidden, total_padded_tokens,
                                          static_cast<_Float16 *>(y), static_cast<hipStream_t>(stream)));
}

// ---- device-side contract ------------------------------------------------

size_t rmoe_contract_workspace_bytes(int64_t num_pairs, int32_t num_experts) {
    if (num_pairs < 0 || num_experts < 1 || num_experts > kMaxDeviceExperts) return 0;
    const int64_t nch = rmoe::contract_chunks(num_pairs);
    const size_t n = (size_t)(nch * ((int64_t)num_experts + 1));
    return n > 0 ? n * sizeof(int32_t) : 4;
}

}  // extern "C"

namespace {

// Argument checks of the device contract build (both entry points), before
// any HIP call; on success *M holds the block count.  The scratch is
// checked by the caller.
int check_contract_device(const int32_t *topk_ids, int64_t num_tokens, int32_t top_k,
                          int32_t num_experts, const int32_t *group_sizes,
                          const int32_t *group_offsets, const int32_t *group_padded_offsets,
                          const int32_t *group_idx_for_bx, int64_t capacity_blocks,
                          const int32_t *num_blocks_m, const int32_t *order,
                          const int32_t *padded_row_of_pair, const int32_t *compact_pos_of_pair,
                          const int32_t *bad_ids, int64_t *M) {
    if (num_tokens < 0 || top_k < 0 || num_experts < 1 || !num_blocks_m) return RMOE_ERR_INVALID_ARGUMENT;
    if (num_experts > kMaxDeviceExperts) return RMOE_ERR_UNSUPPORTED_SHAPE;
    const int64_t pairs = num_tokens * top_k;
    if (pairs > INT32_MAX / 2) return RMOE_ERR_INVALID_ARGUMENT;
    *M = ceil_div(pairs, B) + num_experts;
    if (*M * B > INT32_MAX) return RMOE_ERR_INVALID_ARGUMENT;
    if (!group_sizes || !group_offsets || !group_padded_offsets || !group_idx_for_bx || !bad_ids)
        return RMOE_ERR_INVALID_ARGUMENT;
    if (pairs > 0 && (!topk_ids || !order || !padded_row_of_pair || !compact_pos_of_pair))
        return RMOE_ERR_INVALID_ARGUMENT;
    if (capacity_blocks < *M) return RMOE_ERR_CAPACITY;
    if (!aligned4(topk_ids) || !aligned4(group_sizes) || !aligned4(group_offsets) ||
        !aligned4(group_padded_offsets) || !aligned4(group_idx_for_bx) || !aligned4(order) ||
        !aligned4(padded_row_of_pair) || !aligned4(compact_pos_of_pair) || !aligned4(bad_ids))
        return RMOE_ERR_MISALIGNED;
    return RMOE_OK;
}

}  // namespace

extern "C" {

int rmoe_build_contract_device(const int32_t *topk_ids, int64_t num_tokens, int32_t top_k,
                               int32_t num_experts, int32_t *group_sizes, int32_t *group_offsets,
                               int32_t *group_padded_offsets, int32_t *group_idx_for_bx,
                               int64_t capacity_blocks, int32_t *num_blocks_m, int32_t *order,
                               int32_t *padded_row_of_pair, int32_t *compact_pos_of_pair,
                               int32_t *bad_ids, void *workspace, size_t workspace_bytes,
                               void *stream) {
    int64_t M = 0;
    int st = check_contract_device(topk_ids, num_tokens, top_k, num_experts, group_sizes,
                                   group_offsets, group_padded_offsets, group_idx_for_bx,
                                   capacity_blocks, num_blocks_m, order, padded_row_of_pair,
                                   compact_pos_of_pair, bad_ids, &M);
    if (st != RMOE_OK) return st;
    const int64_t pairs = num_tokens * top_k;
    if (!workspace) return RMOE_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < rmoe_contract_workspace_bytes(pairs, num_experts)) return RMOE_ERR_CAPACITY;
    if (!aligned4(workspace)) return RMOE_ERR_MISALIGNED;
    *num_blocks_m = (int32_t)M;
    return to_status(rmoe::launch_contract(topk_ids, pairs, num_experts, (int32_t)M, group_sizes,
                                           group_offsets, group_padded_offsets, group_idx_for_bx,
                                           order, padded_row_of_pair, compact_pos_of_pair, bad_ids,
                                           static_cast<int32_t *>(workspace),
                                           static_cast<hipStream_t>(stream)));
}

size_t rmoe_contract_noalloc_max_words(void) { return (size_t)rmoe::kNoAllocScratchWords; }

int rmoe_build_contract_device_noalloc(const int32_t *topk_ids, int64_t num_tokens, int32_t top_k,
                                       int32_t num_experts, int32_t *group_sizes,
                                       int32_t *group_offsets, int32_t *group_padded_offsets,
                                       int32_t *group_idx_for_bx, int64_t capacity_blocks,
                                       int32_t *num_blocks_m, int32_t *order,
                                       int32_t *padded_row_of_pair, int32_t *compact_pos_of_pair,
                                       int32_t *bad_ids, void *stream) {
    int64_t M = 0;
    int st = check_contract_device(topk_ids, num_tokens, top_k, num_experts, group_sizes,
                                   group_offsets, group_padded_offsets, group_idx_for_bx,
                                   capacity_blocks, num_blocks_m, order, padded_row_of_pair,
                                   compact_pos_of_pair, bad_ids, &M);
    if (st != RMOE_OK) return st;
    const int64_t pairs = num_tokens * top_k;
    // the scratch this batch needs, against the static array (nothing is allocated)
    const size_t cap = (size_t)rmoe::kNoAllocScratchWords * sizeof(int32_t);
    if (rmoe_contract_workspace_bytes(pairs, num_experts) > cap) return RMOE_ERR_SCRATCH;
    int32_t *ws = nullptr;  // this device's copy of the static scratch
    if (rmoe::noalloc_scratch(&ws) != hipSuccess) return RMOE_ERR_LAUNCH;
    *num_blocks_m = (int32_t)M;
    return to_status(rmoe::launch_contract(topk_ids, pairs, num_experts, (int32_t)M, group_sizes,
                                           group_offsets, group_padded_offsets, group_idx_for_bx,
                                           order, padded_row_of_pair, compact_pos_of_pair, bad_ids,
                                           ws, static_cast<hipStream_t>(stream)));
}

// ---- router ----------------------------------------------------------------

int rmoe_router_f16(const void *x, const void *router_w, int64_t num_tokens, int64_t hidden,
                    int32_t num_experts, int32_t top_k, int32_t *topk_ids, float *topk_weights,
                    void *stream) {
    if (num_tokens < 0 || hidden <= 0 || num_experts < 1 || top_k < 0 || top_k > num_experts)
        return RMOE_ERR_INVALID_ARGUMENT;
    if (num_experts > 256 || top_k > 32 || hidden % 64 != 0) return RMOE_ERR_UNSUPPORTED_SHAPE;
    if (num_tokens == 0 || top_k == 0) return RMOE_OK;
    if (!x || !router_w || !topk_ids || !topk_weights) return RMOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(x) || !aligned16(router_w) || !aligned4(topk_ids) || !aligned4(topk_weights))
        return RMOE_ERR_MISALIGNED;
    return to_status(rmoe::launch_router(static_cast<const _Float16 *>(x),
                                         static_cast<const _Float16 *>(router_w), num_tokens, hidden,
                                         num_experts, top_k, topk_ids, topk_weights,
                                         static_cast<hipStream_t>(stream)));
}

}  // extern "C"
