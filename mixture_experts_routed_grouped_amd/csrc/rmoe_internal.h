// Internal interface between the C-ABI host code (rmoe_api.cpp) and the
// gfx950 kernel launchers (*.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace rmoe {

// Opt a kernel into `bytes` of dynamic LDS, once per device: the attribute
// stays set for the process, so later launches skip the runtime call.
// `done` is the kernel's own per-device flag word (bit d: device d).
inline hipError_t lds_opt_in_once(const void *fn, int bytes, std::atomic<uint64_t> &done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
    return e;
}

// One stage of the routed expert FFN as the kernels see it: a grouped GEMM
// Y[r, n] = epilogue( sum_k X[r, k] * W[e(r), n, k] ) over the valid rows r
// of every 128-row block.  For the gate/up stage W0 = gate_w, W1 = up_w and
// the epilogue is fp16(silu(g) * u); for the down stage W0 = down_w and the
// epilogue is fp16(acc * routed_weight[compact row]).
struct StageArgs {
    const _Float16 *x;      // [Tp, K]
    const _Float16 *w0;     // [E, N, K]
    const _Float16 *w1;     // [E, N, K] (gate/up only)
    const float *rw;        // [pairs] compact order (down only)
    const int32_t *gs;      // group_sizes [E]
    const int32_t *go;      // group_offsets [E+1] (down only)
    const int32_t *gpo;     // group_padded_offsets [E+1]
    const int32_t *gidx;    // group_idx_for_bx [M]
    _Float16 *y;            // [Tp, N]
    int64_t K, N;
    int32_t E, M;
    int64_t pairs;
};

// Kernel-family launchers; return hipSuccess or the launch error.
hipError_t launch_stream_gate_up(const StageArgs &a, hipStream_t s);
hipError_t launch_stream_down(const StageArgs &a, hipStream_t s);
hipError_t launch_tile_gate_up(const StageArgs &a, hipStream_t s);
hipError_t launch_tile_down(const StageArgs &a, hipStream_t s);
// Both tiled stages in one persistent launch (gu.y = dn.x = the hidden
// workspace); sync as described for rmoe_forward_fused_f16; a down tile
// waits at most wait_us for its pair's hidden rows.  local: each XCD runs
// whole entries and the hidden rows stay in its L2 (the kernel's LOCAL
// mode); otherwise entries are spread over all XCDs with write-through
// hand-over.
hipError_t launch_fused(const StageArgs &gu, const StageArgs &dn, int32_t *sync, int64_t wait_us,
                        bool local, hipStream_t s);

hipError_t launch_pack(const _Float16 *x, const float *topk_w, const int32_t *prow,
                       const int32_t *cpos, int64_t pairs, int32_t top_k, int64_t H, int64_t Tp,
                       _Float16 *stacked, float *w_compact, hipStream_t s);
hipError_t launch_combine(const _Float16 *out, const int32_t *prow, int64_t T, int32_t top_k,
                          int64_t H, int64_t Tp, _Float16 *y, hipStream_t s);

// Router: top-k ids and softmax scores of x W^T (E <= 256).
hipError_t launch_router(const _Float16 *x, const _Float16 *w, int64_t T, int64_t H, int32_t E,
                         int32_t k, int32_t *ids, float *vals, hipStream_t s);

// Device-side check of the contract tables: writes the number of violated
// rules to *violations (one workgroup, no memset needed).
hipError_t launch_validate(const int32_t *gs, const int32_t *go, const int32_t *gpo,
                           const int32_t *gidx, int32_t E, int32_t M, int64_t pairs,
                           int32_t *violations, hipStream_t s);

// Words of the static scratch the allocation-free contract build uses
// (1 MiB per GPU): contract_chunks(pairs) * (E + 1) must not exceed it.
constexpr int64_t kNoAllocScratchWords = (int64_t)1 << 18;
// Device address of that scratch on the current device (looked up once per
// device, cached).
hipError_t noalloc_scratch(int32_t **ptr);

// Device-side contract build.  ws holds contract_chunks(pairs) * (E + 1)
// int32 of scratch.
int64_t contract_chunks(int64_t pairs);
hipError_t launch_contract(const int32_t *ids, int64_t pairs, int32_t E, int32_t M, int32_t *gs,
                           int32_t *go, int32_t *gpo, int32_t *gidx, int32_t *order, int32_t *prow,
                           int32_t *cpos, int32_t *bad, int32_t *ws, hipStream_t s);

}  // namespace rmoe
