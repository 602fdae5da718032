/*
 * routed_moe.h -- C ABI of the MI355X (gfx950) routed fused-MoE expert FFN.
 *
 * What the library computes, for every expert-sorted token row r of a
 * 128-row block bx whose expert is e = group_idx_for_bx[bx]
 * ("Fused MoE GEMM 提交说明", sections 算子来源 and 完整算子代码):
 *
 *     gate   = x[r] . gate_w[e]^T              fp16 x fp16, fp32 accumulation
 *     up     = x[r] . up_w[e]^T
 *     hidden = fp16( silu(gate) * up )         written to the fp16 workspace
 *     out[r] = fp16( (hidden . down_w[e]^T) * routed_expert_weights[c] )
 *
 * with token_offset = bx*128 - group_padded_offsets[e],
 * actual_rows = max(0, min(128, group_sizes[e] - token_offset)),
 * row r = bx*128 + i for i < actual_rows, and the COMPACT index
 * c = group_offsets[e] + token_offset + i (section 实现要点: tokens, the
 * workspace and out use padded rows, routed weights use compact rows).
 * Rows i >= actual_rows (padding) are neither computed nor written, in out
 * and in the workspace alike.  A block is computed only if its table entry
 * e lies in [0, E) and names the expert whose padded interval
 * [group_padded_offsets[e], group_padded_offsets[e+1]) holds row bx*128 --
 * always so for tables that satisfy the contract; a corrupted entry leaves
 * that block's rows unwritten in both kernel families alike
 * (rmoe_validate_contract_device reports it).
 *
 * Conventions for every entry point:
 *   - Return 0 (RMOE_OK) on success, a negative rmoe_status otherwise; no
 *     exception crosses the ABI.  On an error nothing is launched.
 *   - Tensors are row-major and contiguous.  "device" pointers are HIP
 *     device memory owned by the caller; "host" pointers are host memory
 *     owned by the caller.  The library keeps no pointer after returning.
 *   - Device work is enqueued asynchronously on `stream` (a hipStream_t
 *     passed as void*; NULL is the default stream).  Nothing synchronises,
 *     nothing allocates, and no table is read back to the host: the tables'
 *     contents are a precondition (check them with rmoe_validate_contract).
 *     A device fault shows at the caller's next synchronisation.
 *   - fp16 is IEEE binary16 (passed as void*), fp32 is float, tables int32.
 */
#ifndef ROUTED_MOE_H
#define ROUTED_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RMOE_API __attribute__((visibility("default")))

/* Rows per block: the kernel's block_token and the contract's padding_M. */
#define RMOE_BLOCK_M 128

typedef enum rmoe_status {
    RMOE_OK = 0,
    RMOE_ERR_INVALID_ARGUMENT = -1, /* null pointer, negative size, bad count */
    RMOE_ERR_UNSUPPORTED_SHAPE = -2, /* hidden/intermediate not a multiple of 128, ... */
    RMOE_ERR_MISALIGNED = -3,        /* a tensor pointer not 16-byte aligned */
    RMOE_ERR_LAUNCH = -4,            /* the HIP runtime refused a launch */
    RMOE_ERR_CONTRACT = -5,          /* tables violate the dispatch contract */
    RMOE_ERR_CAPACITY = -6,          /* an output table is too small */
    RMOE_ERR_SCRATCH = -7            /* a batch beyond the library's static scratch */
} rmoe_status;

/* Kernel family for the forward (RMOE_VARIANT_AUTO picks by shape). */
#define RMOE_VARIANT_AUTO 0
#define RMOE_VARIANT_STREAM 1 /* few rows per block: weight streaming, split K */
#define RMOE_VARIANT_TILE 2   /* many rows per block: LDS-tiled MFMA GEMM */

/* Human-readable name of a status code (static storage). */
RMOE_API const char *rmoe_status_str(int status);

/* Library version string (static storage). */
RMOE_API const char *rmoe_version(void);

/*
 * Host-side dispatch contract (tutorial page "moe_dispatch_contract.py",
 * build_contract steps 1-4; padding rule ceil((count+1)/128)*128).
 *   topk_ids [num_tokens, top_k] host int32, each in [0, num_experts).
 *   Pair p = t*top_k + j.  Pairs are sorted by expert, stably (ties keep
 *   ascending p).
 * Outputs (host, caller-allocated):
 *   group_sizes [E]; group_offsets [E+1] (exclusive scan, last = pairs);
 *   group_padded_offsets [E+1] (scan of padded spans, multiples of 128);
 *   group_idx_for_bx [capacity_blocks] filled for bx < *num_blocks_m, where
 *   *num_blocks_m = ceil(pairs/128) + E and block bx belongs to the last
 *   expert whose padded start is <= bx*128;
 *   order [pairs] (the sorted pair ids); padded_row_of_pair [pairs]
 *   (the token row in the padded layout); compact_pos_of_pair [pairs]
 *   (the routed-weight index).  order/padded/compact may be NULL.
 * Errors: RMOE_ERR_INVALID_ARGUMENT for an id out of range or a bad size
 * (including 128 * num_blocks_m beyond INT32_MAX, which the int32 padded
 * offsets cannot hold), RMOE_ERR_CAPACITY when capacity_blocks <
 * ceil(pairs/128) + E.  Nothing is written on error.
 */
RMOE_API int rmoe_build_contract(const int32_t *topk_ids, int64_t num_tokens, int32_t top_k,
                                 int32_t num_experts, int32_t *group_sizes,
                                 int32_t *group_offsets, int32_t *group_padded_offsets,
                                 int32_t *group_idx_for_bx, int64_t capacity_blocks,
                                 int32_t *num_blocks_m, int32_t *order,
                                 int32_t *padded_row_of_pair, int32_t *compact_pos_of_pair);

/*
 * Check host copies of the tables against the contract (the tutorial's three
 * self-checks in their strict form): offsets start at 0 and step by the
 * sizes, padded spans are (size/128 + 1)*128, group_idx_for_bx is the block
 * -> expert map, every padded interval fits in num_blocks_m*128 <=
 * total_padded_tokens, and group_offsets[E] == total_valid_tokens.
 * Returns RMOE_OK or RMOE_ERR_CONTRACT.
 */
RMOE_API int rmoe_validate_contract(const int32_t *group_sizes, const int32_t *group_offsets,
                                    const int32_t *group_padded_offsets,
                                    const int32_t *group_idx_for_bx, int32_t num_experts,
                                    int32_t num_blocks_m, int64_t total_padded_tokens,
                                    int64_t total_valid_tokens);

/*
 * The same rules checked on DEVICE copies of the tables, asynchronously on
 * `stream` (one small launch, no host read-back): *violations (one int32,
 * device, caller-owned) receives the number of violated rule instances --
 * 0 for valid tables.  Rules on sizes alone (num_blocks_m = ceil(pairs/128)
 * + E, num_blocks_m*128 <= total_padded_tokens) are checked synchronously
 * and return RMOE_ERR_CONTRACT.  The forward kernels themselves compute a
 * block only when group_idx_for_bx maps it to the expert whose padded
 * interval holds it, so a corrupted table leaves rows unwritten instead of
 * reading out of bounds; this call is how to find out.
 * Errors: RMOE_ERR_INVALID_ARGUMENT, RMOE_ERR_MISALIGNED (4-byte),
 * RMOE_ERR_CONTRACT, RMOE_ERR_LAUNCH.
 */
RMOE_API int rmoe_validate_contract_device(const int32_t *group_sizes,
                                           const int32_t *group_offsets,
                                           const int32_t *group_padded_offsets,
                                           const int32_t *group_idx_for_bx, int32_t num_experts,
                                           int32_t num_blocks_m, int64_t total_padded_tokens,
                                           int64_t total_valid_tokens, int32_t *violations,
                                           void *stream);

/*
 * Bytes of the fp16 hidden workspace: total_padded_tokens * intermediate * 2.
 * It is the kernel's global intermediate up_logits of shape
 * [total_padded_tokens, intermediate] in fp16 ("Fused MoE GEMM 提交说明",
 * 完整算子代码: the Step-1 grid writes it, the Step-2 grid reads it).
 * Returns 0 for non-positive sizes.
 */
RMOE_API size_t rmoe_workspace_bytes(int64_t total_padded_tokens, int64_t intermediate);

/*
 * Sizes of the contract for num_pairs (token, expert) pairs over
 * num_experts experts ("moe_dispatch_contract.py", build_contract step 4):
 *   *num_blocks_m = ceil(num_pairs / 128) + num_experts, the number of
 *   128-row blocks the grid covers (each expert owns at most one partly
 *   filled block plus its slack, so the padded intervals always fit);
 *   *total_padded_tokens = 128 * *num_blocks_m, the row count of the padded
 *   token, workspace and out matrices (a caller may use more rows).
 * Either output may be NULL.  Host only, no GPU work.
 * Errors: RMOE_ERR_INVALID_ARGUMENT for negative pairs, num_experts < 1, or
 * sizes whose padded row count would not fit int32.
 */
RMOE_API int rmoe_contract_sizes(int64_t num_pairs, int32_t num_experts, int32_t *num_blocks_m,
                                 int64_t *total_padded_tokens);

/*
 * The kernel family for a batch: `variant` itself if it is
 * RMOE_VARIANT_STREAM or _TILE; for RMOE_VARIANT_AUTO, streaming while the
 * batch averages few routed rows per expert -- there an expert's GEMM is
 * bound by reading its weights, as the contract tutorial's closing note
 * says of small M: at most 96 rows with at most 4 experts, 56 with at most
 * 8 (the tiled family then has few work items), 32 below 32 experts and 36
 * from 32 experts -- and tiling otherwise.  When max_group_rows >= 0 (the
 * largest group size, known to a caller that holds host tables): with fewer
 * than 32 experts streaming also needs every expert to fit one 128-row
 * block (under skewed routing a larger group's blocks read its weights once
 * per block, which weighs on a batch of few experts); and batches of at
 * most 32 experts stream whatever their average while every group fits one
 * streaming pass -- the largest group at most 64 rows, or at most 96 at an
 * average of at most 80 rows (at most 8 experts) or 48 (each weight byte is
 * then read once, while the tiled family has too few work items).
 * max_group_rows < 0 means unknown: the
 * forward, rmoe_gate_up_f16 and rmoe_down_f16 never read device tables,
 * so their AUTO is this function with max_group_rows = -1 (the two stages
 * of one batch therefore always agree); pass the family this returns as
 * their `variant` to use the largest group.
 * Returns RMOE_VARIANT_STREAM or RMOE_VARIANT_TILE, or
 * RMOE_ERR_INVALID_ARGUMENT (unknown variant, negative pairs, E < 1,
 * max_group_rows > num_pairs).
 */
RMOE_API int rmoe_pick_variant(int32_t variant, int64_t num_pairs, int32_t num_experts,
                               int64_t max_group_rows);

/*
 * The fused expert FFN forward (the submission's run_kernel, with the
 * workspace passed in as the runtime-level call does).
 *   stacked_expert_tokens [Tp, H] fp16 device, expert-sorted, 128-padded;
 *   gate_w, up_w [E, I, H] fp16 device; down_w [E, H, I] fp16 device;
 *   routed_expert_weights [pairs] fp32 device, compact order;
 *   group_sizes [E], group_offsets [E+1], group_padded_offsets [E+1],
 *   group_idx_for_bx [num_blocks_m]: int32 device;
 *   workspace [Tp, I] fp16 device (rmoe_workspace_bytes); out [Tp, H] fp16
 *   device.  Only valid rows of workspace and out are written.
 *   H = hidden, I = intermediate (multiples of 128), E = num_experts >= 1,
 *   Tp = total_padded_tokens >= num_blocks_m*128, pairs = total_valid_tokens.
 * Two kernels are enqueued on `stream`: gate/up into the workspace, then
 * down into out.
 */
RMOE_API int rmoe_forward_f16(const void *stacked_expert_tokens, const void *gate_w,
                              const void *up_w, const void *down_w,
                              const float *routed_expert_weights, const int32_t *group_sizes,
                              const int32_t *group_offsets, const int32_t *group_padded_offsets,
                              const int32_t *group_idx_for_bx, void *workspace, void *out,
                              int64_t hidden, int64_t intermediate, int32_t num_experts,
                              int64_t total_padded_tokens, int64_t total_valid_tokens,
                              int32_t num_blocks_m, void *stream);

/* rmoe_forward_f16 with an explicit kernel family (RMOE_VARIANT_*). */
RMOE_API int rmoe_forward_f16_variant(const void *stacked_expert_tokens, const void *gate_w,
                                      const void *up_w, const void *down_w,
                                      const float *routed_expert_weights,
                                      const int32_t *group_sizes, const int32_t *group_offsets,
                                      const int32_t *group_padded_offsets,
                                      const int32_t *group_idx_for_bx, void *workspace,
                                      void *out, int64_t hidden, int64_t intermediate,
                                      int32_t num_experts, int64_t total_padded_tokens,
                                      int64_t total_valid_tokens, int32_t num_blocks_m,
                                      int32_t variant, void *stream);

/*
 * Both stages in ONE launch ("MetaX-TileLang工具链", section 1.12.4: the
 * hidden intermediate's global write and re-read, and kernel fusion as the
 * way to cut it).  Same arguments, layouts and results as
 * rmoe_forward_f16_variant with RMOE_VARIANT_TILE, on any shape; meant for
 * prefill-shaped batches.  One persistent kernel runs every gate/up tile and
 * every down tile; a down tile starts as soon as all gate/up tiles of its own
 * pair of blocks have published their hidden rows, so the two stages overlap
 * (the workspace is still written: it is the hand-over buffer, not a second
 * output).  Results are bit-identical to the two-launch tiled forward.
 *   handover: RMOE_FUSED_LOCAL runs each pair of blocks' gate/up and down
 *         tiles on one XCD (the one whose queue a workgroup reads from the
 *         XCC_ID register), so its hidden rows are handed over inside that
 *         XCD's L2 and leave it only when evicted; RMOE_FUSED_GLOBAL spreads
 *         a pair's tiles over all XCDs and hands the rows over through memory
 *         (write-through stores, device-scope acquire); RMOE_FUSED_AUTO takes
 *         GLOBAL, measured the faster on every workload: the L2 is write-back,
 *         so LOCAL still writes every hidden row out on eviction, and running
 *         each pair's slices on one XCD raises operand reads beyond L2.
 *   sync: int32 device scratch of rmoe_fused_sync_words(num_blocks_m) words,
 *         caller-owned.  It must be all zero before its first use; every
 *         call that runs to completion leaves it zero again, except
 *         sync[RMOE_FUSED_SYNC_ERROR], a sticky count of tiles skipped
 *         because a wait for hidden rows timed out (then every later wait
 *         of that launch gives up at once, so the call still ends).  It is
 *         0 in normal operation; non-zero means out is incomplete.  Calls
 *         that share one sync buffer must not overlap in time (use one
 *         stream, or one buffer each).
 *   max_wait_us: how long a down tile may wait for its pair's hidden rows;
 *         <= 0 selects the default, 2 s (real waits last at most one
 *         gate/up stage, i.e. milliseconds).
 * Returns as rmoe_forward_f16 (RMOE_ERR_INVALID_ARGUMENT for an unknown
 * handover); the launch is asynchronous, nothing is read back.
 */
#define RMOE_FUSED_SYNC_TICKETS 0 /* [8] one work queue per locality group */
#define RMOE_FUSED_SYNC_EXIT 8    /* workgroups done */
#define RMOE_FUSED_SYNC_ERROR 9   /* sticky: skipped tiles */
#define RMOE_FUSED_SYNC_ABORT 10  /* this launch gave up waiting (reset on exit) */
#define RMOE_FUSED_SYNC_HEAD 16   /* then [num_blocks_m]: gate/up tiles done per pair */
#define RMOE_FUSED_AUTO 0
#define RMOE_FUSED_LOCAL 1
#define RMOE_FUSED_GLOBAL 2
RMOE_API size_t rmoe_fused_sync_words(int32_t num_blocks_m);
RMOE_API int rmoe_forward_fused_f16(const void *stacked_expert_tokens, const void *gate_w,
                                    const void *up_w, const void *down_w,
                                    const float *routed_expert_weights,
                                    const int32_t *group_sizes, const int32_t *group_offsets,
                                    const int32_t *group_padded_offsets,
                                    const int32_t *group_idx_for_bx, void *workspace, void *out,
                                    int32_t *sync, int64_t hidden, int64_t intermediate,
                                    int32_t num_experts, int64_t total_padded_tokens,
                                    int64_t total_valid_tokens, int32_t num_blocks_m,
                                    int32_t max_wait_us, int32_t handover, void *stream);

/*
 * Stage 1 alone (the Step-1 grid of section 完整算子代码): workspace rows =
 * fp16(silu(x.Wg^T) * (x.Wu^T)) for valid rows.  Arguments as above;
 * total_valid_tokens (the pair count, group_offsets[E]) only feeds the
 * family choice, which is rmoe_pick_variant's and so the same as
 * rmoe_down_f16's for the same batch.
 */
RMOE_API int rmoe_gate_up_f16(const void *stacked_expert_tokens, const void *gate_w,
                              const void *up_w, const int32_t *group_sizes,
                              const int32_t *group_padded_offsets,
                              const int32_t *group_idx_for_bx, void *workspace, int64_t hidden,
                              int64_t intermediate, int32_t num_experts,
                              int64_t total_padded_tokens, int64_t total_valid_tokens,
                              int32_t num_blocks_m, int32_t variant, void *stream);

/*
 * Stage 2 alone (the Step-2 grid): out rows = fp16((hidden.Wd^T) * w[c])
 * for valid rows, reading the workspace written by stage 1.
 */
RMOE_API int rmoe_down_f16(const void *workspace, const void *down_w,
                           const float *routed_expert_weights, const int32_t *group_sizes,
                           const int32_t *group_offsets, const int32_t *group_padded_offsets,
                           const int32_t *group_idx_for_bx, void *out, int64_t hidden,
                           int64_t intermediate, int32_t num_experts,
                           int64_t total_padded_tokens, int64_t total_valid_tokens,
                           int32_t num_blocks_m, int32_t variant, void *stream);

/*
 * Token packing (the benchmark write-up "MetaX-TileLang工具链", section
 * 1.12.1/2.7: grouping tokens by expert before the routed kernel):
 *   stacked[padded_row_of_pair[p]] = x[p / top_k]            (fp16 rows of H)
 *   w_compact[compact_pos_of_pair[p]] = topk_weights[p]      (fp32)
 * for p < num_tokens*top_k.  x [num_tokens, H] fp16 device, topk_weights
 * [num_tokens*top_k] fp32 device, maps int32 device, stacked [Tp, H] fp16
 * device, w_compact [pairs] fp32 device.  Other rows of stacked are not
 * written.  H must be a multiple of 8, at most 2^33 (RMOE_ERR_UNSUPPORTED_
 * SHAPE otherwise).  Each token row is read once and written to its top_k
 * packed rows.  A pair whose padded row lies outside
 * [0, total_padded_tokens) or whose compact position lies outside [0, pairs)
 * (the device contract marks pairs with invalid expert ids with -1) moves
 * nothing.
 */
RMOE_API int rmoe_pack_f16(const void *x, const float *topk_weights,
                           const int32_t *padded_row_of_pair, const int32_t *compact_pos_of_pair,
                           int64_t num_tokens, int32_t top_k, int64_t hidden, void *stacked,
                           float *w_compact, int64_t total_padded_tokens, void *stream);

/*
 * Combine (same write-up, section 2.7 item 7: the scatter-reduce of the k
 * expert outputs of each token): y[t] = fp16( sum_j out[padded_row_of_pair
 * [t*top_k + j]] ) with the sum in fp32 in slot order j = 0..top_k-1.
 * out [Tp, H] fp16 device, y [num_tokens, H] fp16 device.  H a multiple of
 * 8, at most 2^33 (RMOE_ERR_UNSUPPORTED_SHAPE otherwise).  Slots whose padded
 * row lies outside [0, total_padded_tokens) add nothing.
 */
RMOE_API int rmoe_combine_f16(const void *out, const int32_t *padded_row_of_pair,
                              int64_t num_tokens, int32_t top_k, int64_t hidden, void *y,
                              int64_t total_padded_tokens, void *stream);

/*
 * Device-side dispatch contract (same tables as rmoe_build_contract, the
 * tutorial page "moe_dispatch_contract.py", build_contract; computed on the
 * GPU so that the routing never goes through the host -- the write-up's
 * host-overhead list, section 2.7, names the bincount().cpu() sync and the
 * metadata upload).
 *   topk_ids [num_tokens, top_k] int32 on the device.  Pair p = t*top_k + j;
 *   pairs are sorted by expert, stably (ties keep ascending p), so the tables
 *   are identical to the host builder's.
 * Outputs (device, caller-allocated): group_sizes [E], group_offsets [E+1],
 *   group_padded_offsets [E+1], group_idx_for_bx [capacity_blocks] (filled
 *   for bx < *num_blocks_m), order [pairs], padded_row_of_pair [pairs],
 *   compact_pos_of_pair [pairs], *bad_ids (one int32).  *num_blocks_m (host)
 *   = ceil(pairs/128) + E is returned at once, before the work runs.
 * Ids outside [0, E) are not an error the call can report synchronously:
 *   such pairs are left out of every table (entries of order past the valid
 *   pairs are not written), get -1 in padded_row_of_pair and
 *   compact_pos_of_pair (rmoe_pack_f16 / rmoe_combine_f16 skip them), and
 *   their count lands in *bad_ids.
 * workspace: device scratch of rmoe_contract_workspace_bytes(pairs, E)
 *   bytes, caller-owned, contents irrelevant on entry.
 * Asynchronous on `stream` (4 small launches); allocates nothing.  Errors
 *   (returned before any launch): RMOE_ERR_INVALID_ARGUMENT (negative sizes,
 *   NULL pointers, pairs or padded rows beyond int32), RMOE_ERR_UNSUPPORTED_
 *   SHAPE (E > 8192), RMOE_ERR_CAPACITY (capacity_blocks or workspace too
 *   small), RMOE_ERR_MISALIGNED (pointers not 4-byte aligned).
 */
RMOE_API size_t rmoe_contract_workspace_bytes(int64_t num_pairs, int32_t num_experts);
RMOE_API int rmoe_build_contract_device(const int32_t *topk_ids, int64_t num_tokens, int32_t top_k,
                                        int32_t num_experts, int32_t *group_sizes,
                                        int32_t *group_offsets, int32_t *group_padded_offsets,
                                        int32_t *group_idx_for_bx, int64_t capacity_blocks,
                                        int32_t *num_blocks_m, int32_t *order,
                                        int32_t *padded_row_of_pair, int32_t *compact_pos_of_pair,
                                        int32_t *bad_ids, void *workspace, size_t workspace_bytes,
                                        void *stream);

/*
 * rmoe_build_contract_device without the workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same tables, same
 * arguments otherwise, same asynchronous launches on `stream`; the scratch
 * (contract_chunks * (E + 1) per-chunk counts, as rmoe_contract_workspace_
 * bytes counts them) lives in a static device array of the library,
 * rmoe_contract_noalloc_max_words() int32 words (1 MiB) per GPU, held by each
 * GPU the library runs on until the process ends; nothing in it needs to
 * start at zero, and the call never allocates or frees.  Every call on one
 * GPU uses that GPU's one array: calls that overlap in time on one GPU (on
 * different streams, or from different threads) race and corrupt each
 * other's tables; serialise them.  A batch whose scratch exceeds the array
 * (e.g. E = 128 with more than about 4.1 M pairs) returns RMOE_ERR_SCRATCH
 * before anything is launched; other errors as rmoe_build_contract_device.
 */
RMOE_API size_t rmoe_contract_noalloc_max_words(void);
RMOE_API int rmoe_build_contract_device_noalloc(const int32_t *topk_ids, int64_t num_tokens,
                                                int32_t top_k, int32_t num_experts,
                                                int32_t *group_sizes, int32_t *group_offsets,
                                                int32_t *group_padded_offsets,
                                                int32_t *group_idx_for_bx,
                                                int64_t capacity_blocks, int32_t *num_blocks_m,
                                                int32_t *order, int32_t *padded_row_of_pair,
                                                int32_t *compact_pos_of_pair, int32_t *bad_ids,
                                                void *stream);

/*
 * Router (write-up "MetaX-TileLang工具链", section 2.4: the reference router
 * is a linear gate, a softmax, a top-k):
 *   logits[t, e] = sum_h x[t, h] * router_w[e, h]   (fp32 accumulation)
 *   p[t, :] = softmax(logits[t, :]) over the E experts (fp32)
 *   topk_ids[t, j], topk_weights[t, j], j < top_k: the top_k largest p[t, e]
 *   in decreasing order, equal scores by ascending expert index; the
 *   weights are the probabilities themselves (no renormalisation is stated).
 * x [num_tokens, hidden] fp16 device, router_w [E, hidden] fp16 device,
 * topk_ids [num_tokens, top_k] int32 device, topk_weights [num_tokens,
 * top_k] fp32 device; all caller-owned, contiguous.  The outputs feed
 * rmoe_build_contract_device and rmoe_pack_f16 directly.
 * Shapes: hidden % 64 == 0, 1 <= E <= 256, 0 <= top_k <= min(E, 32).
 * Asynchronous on `stream`, one launch, allocates nothing.  Errors:
 * RMOE_ERR_INVALID_ARGUMENT, RMOE_ERR_UNSUPPORTED_SHAPE, RMOE_ERR_MISALIGNED
 * (fp16 tensors 16-byte, outputs 4-byte aligned), RMOE_ERR_LAUNCH.
 */
RMOE_API int rmoe_router_f16(const void *x, const void *router_w, int64_t num_tokens,
                             int64_t hidden, int32_t num_experts, int32_t top_k,
                             int32_t *topk_ids, float *topk_weights, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ROUTED_MOE_H */
