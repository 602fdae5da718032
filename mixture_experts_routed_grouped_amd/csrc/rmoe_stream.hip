// Weight-streaming grouped GEMM for blocks with few valid rows (decode-
// shaped batches).  Such blocks make the expert FFN bound by reading the
// expert weights from HBM (the contract tutorial notes that with few tokens
// and many experts the padded expert GEMMs turn memory-bound), so this
// family is organised around keeping many weight bytes in flight:
//
//   * one workgroup = one 128-row block x 16 output features, KS waves;
//   * each wave streams its own contiguous K range of the 16 weight rows
//     (split K), straight from HBM into MFMA operand registers -- no LDS
//     staging, each weight byte is read exactly once per pass of 32 rows;
//   * v_mfma_f32_16x16x32_f16 with the WEIGHTS as the A operand (16 feature
//     rows) and the tokens as B (16 token columns), so a lane ends up with 4
//     consecutive features of one token (8-byte fp16 stores);
//   * register double buffering: the loads of chunk c+1 are issued before
//     the MFMAs of chunk c;
//   * the KS partial sums are added in a fixed order through LDS
//     (deterministic, no atomics), then the epilogue of the stage.
//
// Blocks with no valid row exit at once, so the tail blocks and the slack
// block of a full group touch no weight.
#include "rmoe_device.h"
#include "rmoe_internal.h"

namespace rmoe {
namespace {

constexpr int kChunk = 128;  // K elements per lane-group step (4 MFMAs of K=32)
constexpr int kRG = 2;       // 16-row token groups per pass (32 rows)

template <bool DUAL>
struct StreamFrag {
    h8 w0[4];
    h8 w1[DUAL ? 4 : 1];
    h8 x[kRG][4];
};

template <bool DUAL>
__device__ __forceinline__ void stream_load(StreamFrag<DUAL> &f, const _Float16 *w0,
                                            const _Float16 *w1, const _Float16 *x, int64_t K,
                                            int ngroups, int64_t k) {
#pragma unroll
    for (int s = 0; s < 4; ++s) f.w0[s] = *(const h8 *)(w0 + k + 32 * s);
    if constexpr (DUAL) {
#pragma unroll
        for (int s = 0; s < 4; ++s) f.w1[s] = *(const h8 *)(w1 + k + 32 * s);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) f.x[0][s] = *(const h8 *)(x + k + 32 * s);
    if (ngroups > 1) {
#pragma unroll
        for (int s = 0; s < 4; ++s) f.x[1][s] = *(const h8 *)(x + 16 * K + k + 32 * s);
    }
}

template <bool DUAL>
__device__ __forceinline__ void stream_mma(const StreamFrag<DUAL> &f, f4 (&acc)[2][kRG],
                                           int ngroups) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.w0[s], f.x[0][s], acc[0][0], 0, 0, 0);
        if constexpr (DUAL)
            acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.w1[s], f.x[0][s], acc[1][0], 0, 0, 0);
    }
    if (ngroups > 1) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.w0[s], f.x[1][s], acc[0][1], 0, 0, 0);
            if constexpr (DUAL)
                acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.w1[s], f.x[1][s], acc[1][1], 0, 0, 0);
        }
    }
}

// grid: (N / 16, num_blocks_m); block: 64 * KS threads.
template <bool DUAL, int KS>
__global__ __launch_bounds__(64 * KS) void stream_kernel(StageArgs a) {
    const int bx = blockIdx.y;
    const BlockInfo bi = block_info(a.gs, a.gpo, a.gidx, bx);
    if (bi.rows == 0) return;

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int lr = lane & 15;  // A: weight row in the 16-row tile; B: token row
    const int lg = lane >> 4;  // k sub-group: 8 consecutive k of each 32
    const int64_t K = a.K, N = a.N;
    const int n0 = blockIdx.x * 16;

    const int nchunks = (int)(K / kChunk);
    const int c_begin = (nchunks * wave) / KS;
    const int c_end = (nchunks * (wave + 1)) / KS;

    const _Float16 *w0 = a.w0 + ((int64_t)bi.e * N + n0 + lr) * K + 8 * lg;
    const _Float16 *w1 = DUAL ? a.w1 + ((int64_t)bi.e * N + n0 + lr) * K + 8 * lg : nullptr;

    constexpr int NM = DUAL ? 2 : 1;
    __shared__ f4 red[KS > 1 ? KS : 1][NM][kRG][64];

    for (int prow0 = 0; prow0 < bi.rows; prow0 += 16 * kRG) {
        const int left = bi.rows - prow0;
        const int ngroups = left > 16 ? 2 : 1;
        const _Float16 *x = a.x + ((int64_t)bx * kBlockM + prow0 + lr) * K + 8 * lg;

        f4 acc[2][kRG];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int g = 0; g < kRG; ++g) acc[m][g] = f4{0.f, 0.f, 0.f, 0.f};

        StreamFrag<DUAL> fa, fb;
        int c = c_begin;
        if (c < c_end) stream_load<DUAL>(fa, w0, w1, x, K, ngroups, (int64_t)c * kChunk);
        for (; c < c_end; c += 2) {
            if (c + 1 < c_end) stream_load<DUAL>(fb, w0, w1, x, K, ngroups, (int64_t)(c + 1) * kChunk);
            stream_mma<DUAL>(fa, acc, ngroups);
            if (c + 2 < c_end) stream_load<DUAL>(fa, w0, w1, x, K, ngroups, (int64_t)(c + 2) * kChunk);
            if (c + 1 < c_end) stream_mma<DUAL>(fb, acc, ngroups);
        }

        if constexpr (KS > 1) {
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int g = 0; g < kRG; ++g) red[wave][m][g][lane] = acc[m][g];
            __syncthreads();
            if (wave < ngroups) {
                const int g = wave;
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    f4 s = red[0][m][g][lane];
#pragma unroll
                    for (int w = 1; w < KS; ++w) s += red[w][m][g][lane];
                    acc[m][0] = s;  // the reduced group lives in slot 0
                }
            }
        }

        // epilogue: lane holds token (prow0 + 16 g + lr), features n0 + 4 lg + [0, 4)
#pragma unroll
        for (int g = 0; g < kRG; ++g) {
            bool mine;
            int slot;
            if constexpr (KS > 1) {
                mine = (wave == g) && g < ngroups;
                slot = 0;
            } else {
                mine = g < ngroups;
                slot = g;
            }
            const int tok = prow0 + 16 * g + lr;
            if (mine && tok < bi.rows) {
                const int64_t row = (int64_t)bx * kBlockM + tok;
                _Float16 *dst = a.y + row * N + n0 + 4 * lg;
                h4 v;
                if constexpr (DUAL) {
                    const f4 gt = acc[0][slot], up = acc[1][slot];
                    v = to_h4(silu(gt[0]) * up[0], silu(gt[1]) * up[1], silu(gt[2]) * up[2],
                              silu(gt[3]) * up[3]);
                } else {
                    const float w = a.rw[a.go[bi.e] + bi.token_offset + tok];
                    const f4 o = acc[0][slot];
                    v = to_h4(o[0] * w, o[1] * w, o[2] * w, o[3] * w);
                }
                *(h4 *)dst = v;
            }
        }
        if constexpr (KS > 1) __syncthreads();  // red[] is reused by the next pass
    }
}

constexpr int kStreamKS = 4;

}  // namespace

hipError_t launch_stream_gate_up(const StageArgs &a, hipStream_t s) {
    dim3 grid((unsigned)(a.N / 16), (unsigned)a.M);
    hipLaunchKernelGGL((stream_kernel<true, kStreamKS>), grid, dim3(64 * kStreamKS), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_stream_down(const StageArgs &a, hipStream_t s) {
    dim3 grid((unsigned)(a.N / 16), (unsigned)a.M);
    hipLaunchKernelGGL((stream_kernel<false, kStreamKS>), grid, dim3(64 * kStreamKS), 0, s, a);
    return hipGetLastError();
}

}  // namespace rmoe
