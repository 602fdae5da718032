// Token packing and combine around the routed kernel: pure data movement,
// bound by HBM.  Each thread moves 16-byte chunks (8 fp16), consecutive
// threads take consecutive chunks of one row, so every row is read and
// written with full coalesced lines.
#include "rmoe_device.h"
#include "rmoe_internal.h"

namespace rmoe {
namespace {

// stacked[prow[p]] = x[p / k]; w_compact[cpos[p]] = topk_w[p].  A pair whose
// table entry lies outside [0, Tp) or [0, pairs) (a pair the device contract
// left out for an out-of-range expert id) moves nothing.  NT: store the rows
// with the non-temporal hint -- chosen when they are too large to stay in
// the 256 MB Infinity Cache for the next kernel anyway (the large workload's
// 1.9 GB: 672 -> 524 us); smaller batches keep them cacheable.
template <bool NT>
__global__ __launch_bounds__(256) void pack_kernel(const _Float16 *__restrict__ x,
                                                   const float *__restrict__ topk_w,
                                                   const int32_t *__restrict__ prow,
                                                   const int32_t *__restrict__ cpos, int64_t pairs,
                                                   int32_t k, int64_t chunks_per_row, int64_t Tp,
                                                   _Float16 *__restrict__ stacked,
                                                   float *__restrict__ w_compact) {
    const int64_t total = pairs * chunks_per_row;
    const int64_t H = chunks_per_row * 8;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t p = i / chunks_per_row, c = i - p * chunks_per_row;
        const int64_t t = p / k;
        const int64_t r = prow[p];
        if (r >= 0 && r < Tp) {
            const h8 v = *(const h8 *)(x + t * H + 8 * c);
            if constexpr (NT)
                __builtin_nontemporal_store(v, (h8 *)(stacked + r * H + 8 * c));
            else
                *(h8 *)(stacked + r * H + 8 * c) = v;
        }
        if (c == 0) {
            const int64_t q = cpos[p];
            if (q >= 0 && q < pairs) w_compact[q] = topk_w[p];
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

}  // namespace

hipError_t launch_pack(const _Float16 *x, const float *topk_w, const int32_t *prow,
                       const int32_t *cpos, int64_t pairs, int32_t top_k, int64_t H, int64_t Tp,
                       _Float16 *stacked, float *w_compact, hipStream_t s) {
    if (pairs == 0) return hipSuccess;
    const int64_t cpr = H / 8;
    const bool nt = pairs * H * 2 > kPackNtBytes;
    if (nt)
        hipLaunchKernelGGL(pack_kernel<true>, dim3(grid_for(pairs * cpr)), dim3(256), 0, s, x, topk_w,
                           prow, cpos, pairs, top_k, cpr, Tp, stacked, w_compact);
    else
        hipLaunchKernelGGL(pack_kernel<false>, dim3(grid_for(pairs * cpr)), dim3(256), 0, s, x, topk_w,
                           prow, cpos, pairs, top_k, cpr, Tp, stacked, w_compact);
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
