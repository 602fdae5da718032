// LDS-tiled MFMA grouped GEMM for blocks with many valid rows (prefill-
// shaped batches), where the expert GEMMs are compute-bound.
//
// One workgroup (4 waves, 256 threads) owns one 128-row contract block and a
// 256-row slice of weight rows:
//   * gate/up: 128 gate rows and the SAME 128 up rows, so the activation
//     tile is staged once in LDS and feeds both GEMMs, and each lane ends up
//     holding gate and up of the same (token, feature) for the fused
//     silu(gate) * up epilogue;
//   * down: 256 consecutive rows of down_w.
// Per K step of 64: the weight tile [256 x 64] and the token tile [128 x 64]
// go global -> registers -> LDS (16-byte rows chunks, XOR-swizzled by row so
// that MFMA operand reads hit distinct banks), double-buffered with a single
// barrier per step: the global loads of step k+1 are in flight while the
// MFMAs of step k run.  Waves are 2 (weight rows) x 2 (tokens); each wave
// computes 128 weight rows x 64 tokens with v_mfma_f32_32x32x16_f16 (A =
// weights, B = tokens), 8 accumulator tiles = 128 fp32 registers.
// Token tiles beyond the block's valid rows skip their MFMAs.
#include "rmoe_device.h"
#include "rmoe_internal.h"

namespace rmoe {
namespace {

constexpr int BK = 64;        // K per step
constexpr int WR = 256;       // weight rows per workgroup
constexpr int TR = kBlockM;   // token rows per workgroup
constexpr int ROW_H = BK;     // halves per LDS row
constexpr int STAGE_H = (WR + TR) * ROW_H;

// LDS element offset of 16-byte chunk `c` (0..7) of tile row `r`.
__device__ __forceinline__ int lds_off(int r, int c) { return r * ROW_H + ((c ^ (r & 7)) << 3); }

// grid: (N / (DUAL ? 128 : 256), num_blocks_m); block: 256 threads.
template <bool DUAL>
__global__ __launch_bounds__(256) void tile_kernel(StageArgs a) {
    __shared__ __attribute__((aligned(16))) _Float16 smem[2 * STAGE_H];

    const int bx = blockIdx.y;
    const BlockInfo bi = block_info(a.gs, a.gpo, a.gidx, bx);
    if (bi.rows == 0) return;

    const int64_t K = a.K, N = a.N;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int ww = wave & 1;   // weight-row half of the wave
    const int wt = wave >> 1;  // token half of the wave

    // ---- global -> LDS assignment: thread copies chunk (tid & 7) of rows
    //      (tid >> 3) + 32 j; weights j = 0..7, tokens j = 0..3.
    const int lrow = tid >> 3, lch = tid & 7;
    const _Float16 *wsrc[2];
    int64_t n0;
    if constexpr (DUAL) {
        n0 = (int64_t)blockIdx.x * 128;
        wsrc[0] = a.w0 + ((int64_t)bi.e * N + n0 + lrow) * K + 8 * lch;  // gate rows
        wsrc[1] = a.w1 + ((int64_t)bi.e * N + n0 + lrow) * K + 8 * lch;  // up rows
    } else {
        n0 = (int64_t)blockIdx.x * 256;
        wsrc[0] = a.w0 + ((int64_t)bi.e * N + n0 + lrow) * K + 8 * lch;
        wsrc[1] = wsrc[0] + 128 * K;
    }
    // down with N % 256 == 128: the last slice has 128 weight rows; the
    // upper half is neither loaded nor multiplied nor stored.
    const bool upper = DUAL || n0 + 256 <= N;
    const _Float16 *xsrc = a.x + ((int64_t)bx * kBlockM + lrow) * K + 8 * lch;
    const int64_t step32 = 32 * K;

    h8 wreg[8], xreg[4];
    auto load_tile = [&](int64_t k0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) wreg[j] = *(const h8 *)(wsrc[0] + j * step32 + k0);
        if (upper) {
#pragma unroll
            for (int j = 4; j < 8; ++j) wreg[j] = *(const h8 *)(wsrc[1] + (j - 4) * step32 + k0);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) xreg[j] = *(const h8 *)(xsrc + j * step32 + k0);
    };
    auto store_tile = [&](int buf) {
        _Float16 *base = smem + buf * STAGE_H;
#pragma unroll
        for (int j = 0; j < 8; ++j) *(h8 *)(base + lds_off(lrow + 32 * j, lch)) = wreg[j];
#pragma unroll
        for (int j = 0; j < 4; ++j) *(h8 *)(base + lds_off(WR + lrow + 32 * j, lch)) = xreg[j];
    };

    // ---- MFMA operand rows for this wave
    int arow[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        if constexpr (DUAL)
            arow[t] = (t < 2 ? 0 : 128) + ww * 64 + 32 * (t & 1);
        else
            arow[t] = ww * 128 + 32 * t;
    }
    const int tok0 = wt * 64;
    int ntt = bi.rows <= tok0 ? 0 : (bi.rows <= tok0 + 32 ? 1 : 2);  // live token tiles
    if (ww == 1 && !upper) ntt = 0;

    f16x acc[4][2];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[t][u][i] = 0.f;

    const int lr = lane & 31, lh = lane >> 5;
    auto compute = [&](int buf) {
        const _Float16 *base = smem + buf * STAGE_H;
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
            const int ch = 2 * s + lh;
            h8 af[4], bf[2];
#pragma unroll
            for (int t = 0; t < 4; ++t) af[t] = *(const h8 *)(base + lds_off(arow[t] + lr, ch));
#pragma unroll
            for (int u = 0; u < 2; ++u)
                bf[u] = *(const h8 *)(base + lds_off(WR + tok0 + 32 * u + lr, ch));
            if (ntt > 0) {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    acc[t][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[t], bf[0], acc[t][0], 0, 0, 0);
            }
            if (ntt > 1) {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    acc[t][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[t], bf[1], acc[t][1], 0, 0, 0);
            }
        }
    };

    const int nk = (int)(K / BK);
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const bool more = kt + 1 < nk;
        if (more) load_tile((int64_t)(kt + 1) * BK);
        compute(kt & 1);
        if (more) store_tile((kt + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue.  32x32 accumulator layout: lane holds token column
    //      (lane & 31) and, for register r, weight row 8 (r / 4) + 4 lh + r % 4.
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int tok = tok0 + 32 * u + lr;
        if (tok >= bi.rows || (ww == 1 && !upper)) continue;
        const int64_t row = (int64_t)bx * kBlockM + tok;
        _Float16 *yrow = a.y + row * N + n0;
        if constexpr (DUAL) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int f = ww * 64 + 32 * t + 8 * q + 4 * lh;
                    const f16x &g = acc[t][u];
                    const f16x &p = acc[t + 2][u];
                    *(h4 *)(yrow + f) = to_h4(silu(g[4 * q + 0]) * p[4 * q + 0],
                                              silu(g[4 * q + 1]) * p[4 * q + 1],
                                              silu(g[4 * q + 2]) * p[4 * q + 2],
                                              silu(g[4 * q + 3]) * p[4 * q + 3]);
                }
            }
        } else {
            const float w = a.rw[a.go[bi.e] + bi.token_offset + tok];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int f = ww * 128 + 32 * t + 8 * q + 4 * lh;
                    const f16x &o = acc[t][u];
                    *(h4 *)(yrow + f) = to_h4(o[4 * q + 0] * w, o[4 * q + 1] * w,
                                              o[4 * q + 2] * w, o[4 * q + 3] * w);
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_tile_gate_up(const StageArgs &a, hipStream_t s) {
    dim3 grid((unsigned)(a.N / 128), (unsigned)a.M);
    hipLaunchKernelGGL(tile_kernel<true>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_tile_down(const StageArgs &a, hipStream_t s) {
    dim3 grid((unsigned)((a.N + 255) / 256), (unsigned)a.M);
    hipLaunchKernelGGL(tile_kernel<false>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace rmoe
