// LDS-tiled MFMA grouped GEMM for blocks with many valid rows (prefill-
// shaped batches), where the expert GEMMs are compute-bound.
//
// What bounds it on MI355X is operand delivery into the CUs: L2-resident
// data streams at ~30 B/clk per CU, data beyond L2 at ~15 B/clk, while the
// MFMAs of one CU consume 4096 flop/clk.  So the workgroup tile is the
// largest the register file allows -- 256 weight rows x 256 tokens, 4 waves
// each holding a 128 x 128 fp32 accumulator block (256 AGPRs) -- which needs
// 32 B/clk of operands at full MFMA rate:
//   * 256 tokens = two consecutive 128-row contract blocks of the same expert
//     (a pair starts at every even block of an expert; a lone last block
//     runs with an empty second half);
//   * 256 weight rows: gate/up takes 128 output features, their 128 gate
//     rows AND the same 128 up rows, so a lane holds gate and up of the same
//     (token, feature) for the fused silu(gate) * up epilogue; down takes
//     256 rows of down_w.
// Operands travel global -> LDS by direct DMA (global_load_lds_dwordx4, no
// register staging, no ds_write), 16-byte chunks XOR-swizzled per row so
// that MFMA operand reads (ds_read_b128) hit distinct banks, through a ring
// of 3 LDS stages of K = 32: the DMA of step k+2 is spread over the MFMAs of
// step k.  The waits are explicit (vmcnt) and the barrier is a bare
// s_barrier, because a fenced barrier would drain the DMA ring every step.
// Waves are 2 (weight rows) x 2 (token halves); MFMA is
// v_mfma_f32_32x32x16_f16 with weights as A (32 feature rows) and tokens as
// B (32 token columns).  Token tiles beyond a block's valid rows are
// skipped (the K loop is specialised on their count, a uniform value).
#include <type_traits>

#include "rmoe_device.h"
#include "rmoe_internal.h"

#ifndef RMOE_TILE_GROUP
#define RMOE_TILE_GROUP 4   // weight slices per locality group (see tile_item)
#endif

namespace rmoe {
namespace {

constexpr int kXcd = 8;        // MI355X: workgroups go round-robin over 8 XCDs
constexpr int BK = 32;         // K per step
constexpr int ROWB = 2 * BK;   // bytes per LDS row (64)
constexpr int WROWS = 256;     // weight rows per workgroup
constexpr int TROWS = 256;     // token rows per workgroup (two blocks)
constexpr int STAGE = (WROWS + TROWS) * ROWB;  // 32 KB
constexpr int NSTAGE = 3;
constexpr int DMA_PER_WAVE = (WROWS + TROWS) / 16 / 4;  // 16-row DMA blocks per wave per step (8)

// Physical 16-byte slot of logical chunk c (0..3) in LDS row r: rows are 64
// bytes, four rows share one 256-byte sweep of the 64 banks, and XOR-ing
// with (r >> 2) & 3 gives the 16 consecutive rows of an operand read 16
// distinct (row mod 4, slot) bank groups.
__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int loff(int r, int c) { return r * ROWB + ((c ^ swz(r)) << 4); }

// One 1 KB global -> LDS DMA: lane i stores its 16 bytes at lds + 16 i.
__device__ __forceinline__ void dma16(const void *g, unsigned lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(N) only (expcnt and lgkmcnt left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ void bar() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Work item of workgroup w in an order that keeps operand sharing inside one
// XCD's L2.  Items (weight slice nt, block bx) are listed group by group:
// a group is RMOE_TILE_GROUP consecutive slices, and within a group blocks
// run in order with the group's slices innermost.  Blocks of one expert are
// consecutive, so the workgroups an XCD runs at the same time cover a few
// slices of the same expert's weights and a few token blocks.  The list is
// cut into 8 contiguous parts, one per XCD (workgroup w runs on XCD w % 8).
// Returns false for padding workgroups.
__device__ __forceinline__ bool tile_item(int w, int NT, int M, int &nt, int &bx) {
    const int total = NT * M;
    const int per = (total + kXcd - 1) / kXcd;
    const int item = (w % kXcd) * per + w / kXcd;
    if (w / kXcd >= per || item >= total) return false;
    const int gsz = RMOE_TILE_GROUP * M;
    const int g = item / gsz, r = item - g * gsz;
    const int width = min(RMOE_TILE_GROUP, NT - g * RMOE_TILE_GROUP);
    bx = r / width;
    nt = g * RMOE_TILE_GROUP + (r - bx * width);
    return true;
}

// grid: ceil(NT * M / 8) * 8 workgroups of 256 threads; NT = N / 128 slices
// for gate/up and ceil(N / 256) for down.  Dynamic LDS: NSTAGE * STAGE.
template <bool DUAL>
__global__ __launch_bounds__(256) void tile_kernel(StageArgs a, int NT) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    int nt, bx;
    if (!tile_item(blockIdx.x, NT, a.M, nt, bx)) return;
    // block pairs: the first block of an expert and every second one after it
    const int e = a.gidx[bx];
    const int first = a.gpo[e] / kBlockM, last = a.gpo[e + 1] / kBlockM;  // [first, last)
    if ((bx - first) & 1) return;
    const BlockInfo b0 = block_info(a.gs, a.gpo, a.gidx, bx);
    const bool has1 = bx + 1 < last && bx + 1 < a.M;
    const int rows0 = b0.rows;
    const int rows1 = has1 ? block_info(a.gs, a.gpo, a.gidx, bx + 1).rows : 0;
    if (rows0 == 0 && rows1 == 0) return;

    const int64_t K = a.K, N = a.N;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
    const int lane = tid & 63;
    const int lr = lane & 31, lh = lane >> 5;
    const int ww = wave & 1, wt = wave >> 1;  // weight half, token half (= block bx + wt)

    // ---- DMA sources.  Wave w moves 16-row blocks j = 0..7 of a step: LDS
    //      rows 128 w + 16 j .. +16 (rows 0..255 weights, 256..511 tokens).
    //      Lane i fills row (i >> 2) of the block, slot i & 3, with logical
    //      chunk (i & 3) ^ swz(row).
    const unsigned sbase = (unsigned)(uintptr_t)smem;
    const int64_t n0 = DUAL ? (int64_t)nt * 128 : (int64_t)nt * 256;  // first output feature
    const _Float16 *src[DMA_PER_WAVE];
#pragma unroll
    for (int j = 0; j < DMA_PER_WAVE; ++j) {
        const int r = 128 * wave + 16 * j + (lane >> 2);  // LDS row
        const int c = (lane & 3) ^ swz(r);
        if (r < WROWS) {
            int64_t row;
            const _Float16 *mat;
            if constexpr (DUAL) {
                mat = r < 128 ? a.w0 : a.w1;  // rows 0..127 gate, 128..255 up
                row = n0 + (r & 127);
            } else {
                mat = a.w0;
                row = n0 + r;
            }
            row = row < N ? row : N - 1;  // a narrow last slice: idle rows read a valid row
            src[j] = mat + ((int64_t)b0.e * N + row) * K + 8 * c;
        } else {
            const int t = r - WROWS;  // token row of the pair
            int64_t row = (int64_t)bx * kBlockM + t;
            if (t >= kBlockM && !has1) row -= kBlockM;  // absent second block: stay in bounds
            src[j] = a.x + row * K + 8 * c;
        }
    }
    auto dma_step = [&](int stage, int kt, int j0, int j1) {
        const unsigned st = sbase + stage * STAGE + (128 * wave) * ROWB;
#pragma unroll
        for (int j = j0; j < j1; ++j) dma16(src[j] + (int64_t)kt * BK, st + 16 * j * ROWB);
    };

    // ---- MFMA operands of this wave: weight tiles t (32 rows each), token
    //      tiles u (32 tokens each) of its half
    int wrow[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        if constexpr (DUAL)
            wrow[t] = (t < 2 ? 0 : 128) + 64 * ww + 32 * (t & 1);  // g, g, u, u
        else
            wrow[t] = 128 * ww + 32 * t;
    }
    const int trow0 = WROWS + 128 * wt;
    const int myrows = wt ? rows1 : rows0;
    const bool wlive = DUAL || n0 + 128 * ww < N;
    const int ntt = wlive ? (myrows + 31) / 32 : 0;  // live token tiles (uniform)

    f16x acc[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[t][u][i] = 0.f;

    const int nk = (int)(K / BK);

    auto kloop = [&](auto ntt_c) {
        constexpr int NTT = decltype(ntt_c)::value;
        h8 af[2][4], bf[2][4];
        auto read_frags = [&](const unsigned char *base, int s, int slot) {
            const int ch = 2 * s + lh;
#pragma unroll
            for (int t = 0; t < 4; ++t) af[slot][t] = *(const h8 *)(base + loff(wrow[t] + lr, ch));
#pragma unroll
            for (int u = 0; u < NTT; ++u)
                bf[slot][u] = *(const h8 *)(base + loff(trow0 + 32 * u + lr, ch));
        };
        // prologue: steps 0 and 1 in flight
        dma_step(0, 0, 0, DMA_PER_WAVE);
        dma_step(1, min(1, nk - 1), 0, DMA_PER_WAVE);
        for (int kt = 0; kt < nk; ++kt) {
            // step kt's DMAs are the oldest outstanding: allow step kt+1's
            wait_vm<DMA_PER_WAVE>();
            bar();  // all waves' DMAs of step kt landed; reads of step kt-1 done
            const unsigned char *base = smem + (kt % NSTAGE) * STAGE;
            const int nstage = (kt + 2) % NSTAGE;
            const int kn = min(kt + 2, nk - 1);  // clamped: the ring keeps a fixed DMA count
            if constexpr (NTT > 0) read_frags(base, 0, 0);
#pragma unroll
            for (int s = 0; s < BK / 16; ++s) {
                if constexpr (NTT > 0) {
                    if (s + 1 < BK / 16) read_frags(base, s + 1, (s + 1) & 1);
                }
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (NTT > 0) {
#pragma unroll
                    for (int u = 0; u < NTT; ++u)
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[s & 1][t], bf[s & 1][u],
                                                                             acc[t][u], 0, 0, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                // half of step kt+2's DMA per MFMA step
                dma_step(nstage, kn, s * (DMA_PER_WAVE / 2), (s + 1) * (DMA_PER_WAVE / 2));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        wait_vm<0>();
    };
    switch (ntt) {
        case 4: kloop(std::integral_constant<int, 4>{}); break;
        case 3: kloop(std::integral_constant<int, 3>{}); break;
        case 2: kloop(std::integral_constant<int, 2>{}); break;
        case 1: kloop(std::integral_constant<int, 1>{}); break;
        default: kloop(std::integral_constant<int, 0>{}); break;
    }
    if (ntt == 0) return;

    // ---- epilogue.  32x32 accumulator layout: lane holds token column
    //      (lane & 31) and, for register r, weight row 8 (r / 4) + 4 lh + r % 4.
    const int bmine = bx + wt;
    const int toff = wt ? block_info(a.gs, a.gpo, a.gidx, bx + 1).token_offset : b0.token_offset;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int tok = 32 * u + lr;
        if (tok >= myrows) continue;
        const int64_t row = (int64_t)bmine * kBlockM + tok;
        _Float16 *yrow = a.y + row * N + n0;
        if constexpr (DUAL) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f16x &g = acc[t][u];
                    const f16x &p = acc[t + 2][u];
                    *(h4 *)(yrow + 64 * ww + 32 * t + 8 * q + 4 * lh) =
                        to_h4(silu(g[4 * q + 0]) * p[4 * q + 0], silu(g[4 * q + 1]) * p[4 * q + 1],
                              silu(g[4 * q + 2]) * p[4 * q + 2], silu(g[4 * q + 3]) * p[4 * q + 3]);
                }
            }
        } else {
            const float w = a.rw[a.go[b0.e] + toff + tok];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f16x &o = acc[t][u];
                    *(h4 *)(yrow + 128 * ww + 32 * t + 8 * q + 4 * lh) =
                        to_h4(o[4 * q + 0] * w, o[4 * q + 1] * w, o[4 * q + 2] * w, o[4 * q + 3] * w);
                }
            }
        }
    }
}

unsigned tile_grid(int NT, int M) {
    const long total = (long)NT * M;
    return (unsigned)(((total + kXcd - 1) / kXcd) * kXcd);
}

template <bool DUAL>
hipError_t launch(const StageArgs &a, int NT, hipStream_t s) {
    const unsigned lds = NSTAGE * STAGE;  // 96 KB: above the 64 KB default, so opt in
    hipError_t e = hipFuncSetAttribute((const void *)tile_kernel<DUAL>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(tile_kernel<DUAL>, dim3(tile_grid(NT, a.M)), dim3(256), lds, s, a, NT);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_tile_gate_up(const StageArgs &a, hipStream_t s) {
    return launch<true>(a, (int)(a.N / 128), s);
}

hipError_t launch_tile_down(const StageArgs &a, hipStream_t s) {
    return launch<false>(a, (int)((a.N + 255) / 256), s);
}

}  // namespace rmoe
