// Token packing and combine around the routed kernel: pure data movement,
// bound by HBM.  Each thread moves 16-byte chunks (8 fp16), consecutive
// threads take consecutive chunks of one row, so every row is read and
// written with full coalesced lines.
#include "rmoe_device.h"
#include "rmoe_internal.h"

namespace rmoe {
namespace {

// Pack is token-major: a workgroup takes tokens round robin, lanes split a
// token's row into 16-byte chunks (rows of fewer than 256 chunks put several
// tokens in one workgroup), and every index is fixed per thread -- no
// division per chunk.  It read each token row once where a chunk-major pack
// (consecutive workgroups on the k copies of a row, spread over the XCDs)
// read it once per XCD: 544 -> 367 us on the large workload.
struct RowLanes {
    int tpb;  // tokens per workgroup pass
    int lt;   // this thread's token within the pass (>= tpb: idle)
    int c0;   // its first chunk
    int cs;   // chunk stride
};
__device__ __forceinline__ RowLanes row_lanes(int cpr) {
    RowLanes l;
    if (cpr >= (int)blockDim.x) {
        l.tpb = 1;
        l.lt = 0;
        l.c0 = threadIdx.x;
        l.cs = blockDim.x;
    } else {
        l.tpb = blockDim.x / cpr;
        l.lt = threadIdx.x / cpr;
        l.c0 = threadIdx.x - l.lt * cpr;
        l.cs = cpr;
    }
    return l;
}
constexpr int kChunkBatch = 4;  // chunks a thread loads before storing them

// stacked[prow[t*k + j]] = x[t] for every slot j; w_compact[cpos[p]] =
// topk_w[p].  The token row is read once and written k times.  A pair whose
// table entry lies outside [0, Tp) or [0, pairs) (a pair the device contract
// left out for an out-of-range expert id) moves nothing.  NT: store the rows
// with the non-temporal hint -- chosen when they are too large to stay in
// the 256 MB Infinity Cache for the next kernel anyway (the large workload's
// 1.9 GB); smaller batches keep them cacheable.
template <bool NT>
__global__ __launch_bounds__(256) void pack_kernel(const _Float16 *__restrict__ x,
                                                   const float *__restrict__ topk_w,
                                                   const int32_t *__restrict__ prow,
                                                   const int32_t *__restrict__ cpos, int64_t T,
                                                   int32_t k, int32_t cpr, int64_t Tp,
                                                   _Float16 *__restrict__ stacked,
                                                   float *__restrict__ w_compact) {
    const RowLanes l = row_lanes(cpr);
    const int64_t H = (int64_t)cpr * 8, pairs = T * k;
    for (int64_t tb = (int64_t)blockIdx.x * l.tpb; tb < T; tb += (int64_t)gridDim.x * l.tpb) {
        const int64_t t = tb + l.lt;
        if (l.lt >= l.tpb || t >= T) continue;
        for (int j = l.c0; j < k; j += l.cs) {  // the token's routed weights
            const int64_t p = t * k + j, q = cpos[p];
            if (q >= 0 && q < pairs) w_compact[q] = topk_w[p];
        }
        const _Float16 *src = x + t * H;
        for (int cb = l.c0; cb < cpr; cb += kChunkBatch * l.cs) {
            h8 v[kChunkBatch];
#pragma unroll
            for (int u = 0; u < kChunkBatch; ++u)
                if (cb + u * l.cs < cpr) v[u] = *(const h8 *)(src + 8 * (int64_t)(cb + u * l.cs));
            for (int j = 0; j < k; ++j) {
                const int64_t r = prow[t * k + j];
                if (r < 0 || r >= Tp) continue;
                _Float16 *dst = stacked + r * H;
#pragma unroll
                for (int u = 0; u < kChunkBatch; ++u) {
                    if (cb + u * l.cs >= cpr) break;
                    if constexpr (NT)
                        __builtin_nontemporal_store(v[u], (h8 *)(dst + 8 * (int64_t)(cb + u * l.cs)));
                    else
                        *(h8 *)(dst + 8 * (int64_t)(cb + u * l.cs)) = v[u];
                }
            }
        }
    }
}

// y[t] = fp16(sum_j out[prow[t*k + j]]), fp32 sum in slot order; slots whose
// padded row lies outside [0, Tp) contribute nothing
__global__ __launch_bounds__(256) void combine_kernel(const _Float16 *__restrict__ out,
                                                      const int32_t *__restrict__ prow, int64_t T,
                                                      int32_t k, int64_t chunks_per_row, int64_t Tp,
                                                      _Float16 *__restrict__ y) {
    const int64_t total = T * chunks_per_row;
    const int64_t H = chunks_per_row * 8;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = i / chunks_per_row, c = i - t * chunks_per_row;
        float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < k; ++j) {
            const int64_t r = prow[t * k + j];
            if (r < 0 || r >= Tp) continue;
            const h8 v = *(const h8 *)(out + r * H + 8 * c);
#pragma unroll
            for (int q = 0; q < 8; ++q) s[q] += (float)v[q];
        }
        h8 r;
#pragma unroll
        for (int q = 0; q < 8; ++q) r[q] = (_Float16)s[q];
        *(h8 *)(y + t * H + 8 * c) = r;
    }
}

// packed-row bytes above which pack stores non-temporally: twice the
// Infinity Cache, so the rows could not stay cached for the next kernel
constexpr int64_t kPackNtBytes = (int64_t)512 << 20;

unsigned grid_for(int64_t total) {
    int64_t g = (total + 255) / 256;
    if (g > 256 * 64) g = 256 * 64;  // grid-stride beyond 64 workgroups per CU
    return (unsigned)(g < 1 ? 1 : g);
}

// workgroups for T token rows of cpr chunks: one pass of tokens per
// workgroup, at most 64 workgroups per CU (the kernel strides beyond)
unsigned grid_for_rows(int64_t T, int64_t cpr) {
    const int64_t tpb = cpr >= 256 ? 1 : 256 / cpr;
    int64_t g = (T + tpb - 1) / tpb;
    if (g > 256 * 64) g = 256 * 64;
    return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_pack(const _Float16 *x, const float *topk_w, const int32_t *prow,
                       const int32_t *cpos, int64_t pairs, int32_t top_k, int64_t H, int64_t Tp,
                       _Float16 *stacked, float *w_compact, hipStream_t s) {
    if (pairs == 0) return hipSuccess;
    const int64_t cpr = H / 8, T = pairs / top_k;
    const bool nt = pairs * H * 2 > kPackNtBytes;
    if (nt)
        hipLaunchKernelGGL(pack_kernel<true>, dim3(grid_for_rows(T, cpr)), dim3(256), 0, s, x, topk_w, prow,
                           cpos, T, top_k, (int32_t)cpr, Tp, stacked, w_compact);
    else
        hipLaunchKernelGGL(pack_kernel<false>, dim3(grid_for_rows(T, cpr)), dim3(256), 0, s, x, topk_w, prow,
                           cpos, T, top_k, (int32_t)cpr, Tp, stacked, w_compact);
    return hipGetLastError();
}

hipError_t launch_combine(const _Float16 *out, const int32_t *prow, int64_t T, int32_t top_k,
                          int64_t H, int64_t Tp, _Float16 *y, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int64_t cpr = H / 8;
    hipLaunchKernelGGL(combine_kernel, dim3(grid_for(T * cpr)), dim3(256), 0, s, out, prow, T,
                       top_k, cpr, Tp, y);
    return hipGetLastError();
}

}  // namespace rmoe
