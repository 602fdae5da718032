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
// register staging, no ds_write) in steps of K = 64: each DMA instruction
// reads 8 rows x 128 bytes, a pattern the MI355X L2 serves at ~56 B/clk per
// CU (1 KB-contiguous or 64-byte runs reach ~30).  16-byte chunks are
// XOR-swizzled per row so that MFMA operand reads (ds_read_b128) hit
// distinct banks.  The 160 KB of LDS hold five 32 KB slots -- one K step of
// 256 rows each: three for weights and two for tokens -- so weight DMAs run
// two steps ahead of the MFMAs and token DMAs one step (weights are the
// first-touch stream from HBM; tokens are shared by the concurrently running
// slices of a locality group, so more of them hit L2).  Within a step the memory
// instructions (the next sub-step's operand reads, the DMAs) are issued one
// after each MFMA, so they leave the in-order wave while the matrix core is
// busy.  The waits are explicit (vmcnt) and the barrier is a bare s_barrier,
// because a fenced barrier would drain the DMA ring every step.
// Waves are 2 (weight rows) x 2 (token halves); MFMA is
// v_mfma_f32_32x32x16_f16 with weights as A (32 feature rows) and tokens as
// B (32 token columns).  Token tiles beyond a block's valid rows are
// skipped (the K loop is specialised on their count, a uniform value).
#include <atomic>
#include <type_traits>

#include "../../include/routed_moe.h"
#include "rmoe_device.h"
#include "rmoe_internal.h"
#include "rmoe_sched.h"

namespace rmoe {
namespace {

constexpr int kXcd = 8;     // MI355X: workgroups go round-robin over 8 XCDs
constexpr int BK = 64;      // K per step
constexpr int ROWB = 2 * BK;  // bytes per LDS row: one 128-byte line
constexpr int CPR = ROWB / 16;  // 16-byte chunks per row
constexpr int RPD = 64 / CPR;   // rows per 1 KB DMA instruction (8)
constexpr int SROWS = 256;      // rows per slot: 256 weight rows or 256 tokens
constexpr int SLOT = SROWS * ROWB;  // 32 KB
constexpr int NWS = 3;  // weight slots: weight DMA runs two steps ahead
constexpr int NTS = 2;  // token slots: token DMA runs one step ahead
static_assert((NWS + NTS) * SLOT <= 160 * 1024, "LDS slots exceed 160 KB");
constexpr int LDS_BYTES = (NWS + NTS) * SLOT;
constexpr int DMA_HALF = SROWS / RPD / 4;   // DMAs per wave per slot fill (8)
constexpr int DMA_PER_WAVE = 2 * DMA_HALF;  // per step: token fill, then weight fill
constexpr int SUB = BK / 16;                // MFMA sub-steps per K step
// vmcnt a wave may leave outstanding when it publishes step k+1: the weight
// fill of step k+2, issued after the token fill of step k+1
constexpr int VM_ALLOW = DMA_HALF;
constexpr int kCpolSc1 = 16;  // cache-policy operand of the buffer builtins: sc1 (device scope)
typedef int i32x4 __attribute__((ext_vector_type(4)));
static_assert(kItemRows == kBlockM, "work items are contract blocks");

// One 1 KB global -> LDS DMA addressed as a wave-uniform base plus a 32-bit
// per-lane byte offset (the scalar-base form of global_load_lds_dwordx4):
// a K step moves only the base, in scalar registers, so no 64-bit vector
// address add precedes each DMA (measured 2-3% faster on every workload than
// full per-lane addresses).  Counted by vmcnt like a load.
__device__ __forceinline__ void dma16_sb(const void *base, unsigned off, unsigned lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(off), "s"(base)
                 : "memory", "m0");
}

// ---- Phase timing, compiled only into the diagnostic library
//      (RMOE_PHASE_TIMING=1: librmoe_phase.so).  Each workgroup of a
//      persistent launch sums the shader-clock ticks (s_memtime) that its
//      items spend in their prologue (addresses, the first DMAs until step 0
//      has landed), their K loop and their epilogue (until the last output
//      store is issued), and writes the three sums, its item count and its
//      whole run time to phase_cycles[stage][workgroup] (stage 0 gate/up,
//      1 down); rmoe_phase_cycles copies them to the host.  Wave 0 keeps the
//      record: its token half always holds rows.  The instrumentation adds
//      four clock reads per item and leaves every result unchanged.
#ifndef RMOE_PHASE_TIMING
#define RMOE_PHASE_TIMING 0
#endif
constexpr int kPhaseWg = 1024;  // workgroups recorded per stage
struct PhaseSums {
    unsigned long long pro = 0, loop = 0, epi = 0, items = 0;
};
__device__ __forceinline__ unsigned long long phase_clock() {
#if RMOE_PHASE_TIMING
    return __builtin_amdgcn_s_memtime();
#else
    return 0;
#endif
}
#if RMOE_PHASE_TIMING
__device__ unsigned long long phase_cycles[2][kPhaseWg][5];
#endif

// One tile: blocks bx (b0: its expert, offset in the group, valid rows) and
// bx+1 (rows1 valid rows; has1: it belongs to the same expert) against the
// weight slice nt.  Called with the workgroup's LDS; leaves no DMA in flight.
// WT: store the output tile write-through at device scope (sc1), so that a
// store that has completed (vmcnt) is visible to every XCD without an L2
// write-back; the single-launch path hands the hidden rows over this way.
template <bool DUAL, bool WT = false>
__device__ __forceinline__ void run_tile(const StageArgs &a, unsigned char *smem, int nt, int bx,
                                         const BlockInfo &b0, bool has1, int rows1,
                                         PhaseSums *ps = nullptr) {
    const unsigned long long t0 = phase_clock();
    unsigned long long t1 = t0, t2 = t0;
    const int rows0 = b0.rows;
    const int64_t K = a.K, N = a.N;
    // opaque per tile: keeps the compiler from hoisting per-lane address
    // arithmetic out of a loop over tiles, where it would stay live (and
    // spill) through the K loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
    const int lane = tid & 63;
    const int lr = lane & 31, lh = lane >> 5;
    const int ww = wave & 1, wt = wave >> 1;  // weight half, token half (= block bx + wt)

    // ---- DMA sources.  Wave w fills rows 64 w .. 64 w + 63 of every slot,
    //      RPD rows per instruction j: lane i takes row 64 w + RPD j + i / 8,
    //      physical chunk i % 8, i.e. logical chunk (i % 8) ^ swz(row).
    //      Addresses are a wave-uniform base (the wave's first weight row in
    //      its matrix, the pair's first token row) plus per-lane byte offsets
    //      (under 256 rows x K x 2 bytes with K <= 2^20: they fit 32 bits).
    const unsigned sbase = (unsigned)(uintptr_t)smem;
    const int64_t n0 = DUAL ? (int64_t)nt * 128 : (int64_t)nt * 256;  // first output feature
    const _Float16 *wmat = a.w0;
    int64_t wrow0 = n0 + 64 * wave;
    if constexpr (DUAL) {
        wmat = wave < 2 ? a.w0 : a.w1;  // weight rows 0..127 gate, 128..255 up
        wrow0 = n0 + ((64 * wave) & 127);
    }
    wrow0 = wrow0 < N ? wrow0 : N - 1;
    const _Float16 *wbase = wmat + ((int64_t)b0.e * N + wrow0) * K;
    const _Float16 *tbase = a.x + (int64_t)bx * kBlockM * K;
    unsigned woff[DMA_HALF], tkoff[DMA_HALF];
#pragma unroll
    for (int j = 0; j < DMA_HALF; ++j) {
        const int r = 64 * wave + RPD * j + lane / CPR;  // row within the slot
        const int c = (lane % CPR) ^ lds_swz(r);
        int64_t row = DUAL ? n0 + (r & 127) : n0 + r;
        row = row < N ? row : N - 1;  // a narrow last slice: idle rows read a valid row
        woff[j] = (unsigned)(((row - wrow0) * K + 8 * c) * 2);
        int tr = r;                                 // token row r of the pair
        if (r >= kBlockM && !has1) tr -= kBlockM;  // absent second block: stay in bounds
        tkoff[j] = (unsigned)(((int64_t)tr * K + 8 * c) * 2);
    }
    const unsigned dwave = sbase + 64 * wave * ROWB;
    // DMA d of a step: d < DMA_HALF fills the token slot, the rest the weight slot
    auto dma_one = [&](int d, int kt_t, int kt_w, int slot_t, int slot_w) {
        if (d < DMA_HALF)
            dma16_sb(tbase + (int64_t)kt_t * BK, tkoff[d], dwave + (NWS + slot_t) * SLOT + RPD * d * ROWB);
        else
            dma16_sb(wbase + (int64_t)kt_w * BK, woff[d - DMA_HALF],
                     dwave + slot_w * SLOT + RPD * (d - DMA_HALF) * ROWB);
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
    const int trow0 = 128 * wt;
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

    // The pipeline is rotated by one sub-step: the wait and barrier that
    // publish step k+1 sit before the last sub-step of step k, so the LDS
    // reads of step k+1's first sub-step overlap that sub-step's MFMAs
    // instead of stalling every step start.  Group g(j) = the DMAs that
    // refill step j's slots once every wave is done with them (tokens of
    // step j+NTS, weights of step j+NWS), DPS per sub-step over the SUB
    // sub-steps that follow the barrier retiring step j's reads.
    auto kloop = [&](auto ntt_c) {
        constexpr int NTT = decltype(ntt_c)::value;
        constexpr int NMF = 4 * NTT;  // MFMAs per sub-step
        constexpr int NRD = 4 + NTT;  // operand reads per sub-step
        constexpr int DPS = DMA_PER_WAVE / SUB;
        static_assert(DMA_PER_WAVE % SUB == 0, "DMA groups split evenly over the sub-steps");
        h8 af[2][4], bf[2][4];
        auto read_one = [&](const unsigned char *wb, const unsigned char *tb, int s, int buf, int i) {
            const int ch = 2 * s + lh;
            if (i < 4)
                af[buf][i] = *(const h8 *)(wb + lds_off(wrow[i] + lr, ch));
            else
                bf[buf][i - 4] = *(const h8 *)(tb + lds_off(trow0 + 32 * (i - 4) + lr, ch));
        };
        // DMA d of group g(j); indices past the last step are clamped (the
        // repeats land in slots no later step reads)
        auto dma_g = [&](int j, int d) {
            dma_one(d, min(j + NTS, nk - 1), min(j + NWS, nk - 1), (j + NTS) % NTS, (j + NWS) % NWS);
        };
        // one sub-step: MFMAs of sub-step sm (buffer sm & 1), interleaved with
        // the reads of sub-step sr of (rw, rt) into buffer sr & 1 and DMAs
        // dlo .. dlo + DPS - 1 of group gj
        auto substep = [&](int sm, bool rd, const unsigned char *rw, const unsigned char *rt, int sr,
                           bool dm, int gj, int dlo) {
            const int nrd = (NTT > 0 && rd) ? NRD : 0;
            const int ndma = dm ? DPS : 0;
            const int nmem = nrd + ndma;
            const int nslot = NMF > nmem ? NMF : nmem;
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < nslot; ++i) {
                if (i < NMF) {
                    const int u = i / 4, t = i % 4;
                    acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[sm & 1][t], bf[sm & 1][u],
                                                                     acc[t][u], 0, 0, 0);
                }
                int r = -1, d = -1;  // memory slot i: reads on even slots, DMAs between
                if (nrd > 0 && ndma > 0) {
                    const int m = min(nrd, ndma);
                    if (i < 2 * m) {
                        if (i & 1) d = i / 2; else r = i / 2;
                    } else if (i - m < nrd && nrd > ndma) {
                        r = i - m;
                    } else if (i - m < ndma && ndma > nrd) {
                        d = i - m;
                    }
                } else if (i < nrd) {
                    r = i;
                } else if (i < ndma) {
                    d = i;
                }
                if (r >= 0) read_one(rw, rt, sr, sr & 1, r);
                if (d >= 0) dma_g(gj, dlo + d);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // prologue: groups g(-3) (weights of step 0), g(-2) (tokens of step
        // 0, weights of step 1) and the first part of g(-1) (tokens of step 1)
#pragma unroll
        for (int d = DMA_HALF; d < DMA_PER_WAVE; ++d) dma_g(-3, d);
#pragma unroll
        for (int d = 0; d < DMA_PER_WAVE; ++d) dma_g(-2, d);
#pragma unroll
        for (int d = 0; d < DPS; ++d) dma_g(-1, d);
        wait_vm<DMA_HALF + DPS>();  // step 0 landed: only weights 1 and that part may be in flight
        bar();
        if constexpr (RMOE_PHASE_TIMING) t1 = phase_clock();
        if constexpr (NTT > 0) {
#pragma unroll
            for (int i = 0; i < NRD; ++i) read_one(smem, smem + NWS * SLOT, 0, 0, i);
        }
        for (int k = 0; k < nk; ++k) {
            const unsigned char *wb = smem + (k % NWS) * SLOT;
            const unsigned char *tb = smem + (NWS + k % NTS) * SLOT;
            if (k > 0) substep(SUB - 1, true, wb, tb, 0, true, k - 1, 0);  // end of step k-1
#pragma unroll
            for (int s = 0; s + 1 < SUB; ++s) substep(s, true, wb, tb, s + 1, true, k - 1, DPS * (s + 1));
            // publish step k+1 (tokens came with g(k-1); only the weights of
            // step k+2 may still be in flight) and retire this wave's reads of
            // step k, whose slots the next group refills
            wait_vm<VM_ALLOW>();
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
            bar();
        }
        substep(SUB - 1, false, nullptr, nullptr, 0, false, 0, 0);  // end of step nk-1
        wait_vm<0>();
    };
    switch (ntt) {
        case 4: kloop(std::integral_constant<int, 4>{}); break;
        case 3: kloop(std::integral_constant<int, 3>{}); break;
        case 2: kloop(std::integral_constant<int, 2>{}); break;
        case 1: kloop(std::integral_constant<int, 1>{}); break;
        default: kloop(std::integral_constant<int, 0>{}); break;
    }
    if constexpr (RMOE_PHASE_TIMING) t2 = phase_clock();
    auto phase_end = [&]() {
        if constexpr (RMOE_PHASE_TIMING) {
            if (ps) {
                const unsigned long long t3 = phase_clock();
                ps->pro += t1 - t0;
                ps->loop += t2 - t1;
                ps->epi += t3 - t2;
                ps->items += 1;
            }
        }
    };
    // ---- epilogue, staged through LDS so that the global stores are whole
    //      128-byte lines (the MFMA layout gives a lane one token and 4
    //      consecutive features: 8 bytes in each of 32 rows per store).  No
    //      barrier: a wave stages only into its own 8 KB piece of the slots,
    //      which only its own DMAs (all landed: it waited for them) fill, and
    //      no wave reads the ring after the last K-step barrier.
    if (ntt == 0) {
        phase_end();
        return;
    }
    const int bmine = bx + wt;
    const int toff = b0.token_offset + kBlockM * wt;
    // staged tile of this wave: 128 token rows x OB bytes (gate/up: 64
    // features, down: 128), 16-byte chunks XOR-swizzled by row; RPP rows in
    // each of the wave's 8 KB pieces (slot j: bytes j*SLOT + wave*8 KB ..)
    constexpr int OB = DUAL ? 128 : 256;
    constexpr int OC = OB / 16;  // chunks per row
    constexpr int RPP = 8192 / OB;
    static_assert(128 / RPP <= NWS + NTS, "staging fits in the wave's pieces");
    auto stage_row = [&](int row) {
        return smem + (row / RPP) * SLOT + wave * 8192 + (row % RPP) * OB;
    };
    // down: the routed weights of this lane's tokens, all requested before
    // any is used, so the epilogue waits for one memory round trip (read
    // inside the tile loop, the compiler reloaded go[e] and waited for each
    // dependent load in turn: 8 round trips)
    [[maybe_unused]] float wtok[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (!DUAL) {
        const float *rwe = a.rw + a.go[b0.e] + toff;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (u < ntt && 32 * u + lr < myrows) wtok[u] = rwe[32 * u + lr];
    }
    // 32x32 accumulator layout: lane holds token column (lane & 31) and,
    // for register 4q + r, weight row 8q + 4lh + r of its 32-row tile t
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if (u >= ntt) continue;
        const int row = 32 * u + lr;
        unsigned char *srow = stage_row(row);
        if constexpr (DUAL) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f16x &g = acc[t][u];
                    const f16x &p = acc[t + 2][u];
                    const int c = (4 * t + q) ^ (row & (OC - 1));  // features 32t + 8q .. +7
                    *(h4 *)(srow + (c << 4) + 8 * lh) =
                        to_h4(silu(g[4 * q + 0]) * p[4 * q + 0], silu(g[4 * q + 1]) * p[4 * q + 1],
                              silu(g[4 * q + 2]) * p[4 * q + 2], silu(g[4 * q + 3]) * p[4 * q + 3]);
                }
            }
        } else {
            const float w = wtok[u];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f16x &o = acc[t][u];
                    const int c = (4 * t + q) ^ (row & (OC - 1));
                    *(h4 *)(srow + (c << 4) + 8 * lh) =
                        to_h4(o[4 * q + 0] * w, o[4 * q + 1] * w, o[4 * q + 2] * w, o[4 * q + 3] * w);
                }
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes are done
    // row-contiguous read-back: OC lanes per row, 64 / OC rows per instruction
    _Float16 *ybase = a.y + (int64_t)bmine * kBlockM * N + n0 + (DUAL ? 64 : 128) * ww;
    const int c = lane % OC;
    // buffer view of this wave's output tile (128 rows of N, < 2^31 bytes)
    [[maybe_unused]] const __amdgpu_buffer_rsrc_t yres =
        __builtin_amdgcn_make_buffer_rsrc(ybase, 0, 0x7fffffff, 0x00020000);
#pragma unroll 4
    for (int r0 = 0; r0 < 32 * ntt; r0 += 64 / OC) {
        const int row = r0 + lane / OC;
        if (row < myrows) {
            const h8 v = *(const h8 *)(stage_row(row) + ((c ^ (row & (OC - 1))) << 4));
            if constexpr (WT)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), yres,
                                                       (int)(((int64_t)row * N + 8 * c) * 2), 0,
                                                       kCpolSc1);
            else
                *(h8 *)(ybase + (int64_t)row * N + 8 * c) = v;
        }
    }
    phase_end();
}

// Runs work item it (rmoe_sched.h) with the workgroup's LDS.  The item list
// comes from the group sizes and padded offsets; each of its blocks is
// computed only if group_idx_for_bx maps it to the item's expert (the rule
// the streaming family applies per block, in block_info), so both families
// act on the same table and skip the same blocks of a corrupted one.
template <bool DUAL, bool WT = false>
__device__ __forceinline__ void run_item(const StageArgs &a, unsigned char *smem, const TileItem &it,
                                         PhaseSums *ps = nullptr) {
    BlockInfo b0;
    b0.e = it.e;
    b0.token_offset = it.off;
    b0.rows = a.gidx[it.bx] == it.e ? it.rows0 : 0;
    const int rows1 = (it.rows1 > 0 && a.gidx[it.bx + 1] == it.e) ? it.rows1 : 0;
    if (b0.rows == 0 && rows1 == 0) return;
    run_tile<DUAL, WT>(a, smem, it.nt, it.bx, b0, rows1 > 0, rows1, ps);
}

// Persistent kernel: one workgroup per CU (a multiple of 8 of them, LDS_BYTES
// of dynamic LDS each), looping over work items, all live: a pair of blocks
// of one expert that holds valid rows, times a weight slice (NT = N / 128
// slices for gate/up, ceil(N / 256) for down).  The item list (rmoe_sched.h)
// is cut into 8 contiguous parts, one per XCD (workgroup w runs on XCD
// w % 8), so the 32 workgroups of an XCD run a rectangle of 4 consecutive
// pairs x 8 slices at a time -- operands they share in that XCD's L2.
template <bool DUAL>
__global__ __launch_bounds__(256) void tile_kernel(StageArgs a, int NT) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const TileSeq seq = tile_seq(a.gs, a.E, NT, blockIdx.x % kXcd, kXcd);
    const int nl = gridDim.x / kXcd;
    TileCursor cur;
    PhaseSums ps;
    [[maybe_unused]] const unsigned long long ts = phase_clock();
    for (int i = blockIdx.x / kXcd; i < seq.n; i += nl)
        run_item<DUAL>(a, smem, tile_item(a.gs, a.gpo, seq, i, cur), &ps);
#if RMOE_PHASE_TIMING
    const unsigned long long te = phase_clock();
    if (threadIdx.x == 0 && blockIdx.x < kPhaseWg) {
        unsigned long long *g = phase_cycles[DUAL ? 0 : 1][blockIdx.x];
        g[0] = ps.pro;
        g[1] = ps.loop;
        g[2] = ps.epi;
        g[3] = ps.items;
        g[4] = te - ts;
    }
#endif
}

// ---- Both stages in one launch.
//
// The same tiles as the two persistent launches, taken from one queue per
// locality group.  A down item of the pair at block bx needs every gate/up
// slice of that pair in the hidden workspace, so gate/up items count
// themselves into done[bx] once their stores are out, and a down item waits
// until done[bx] reaches the slice count.  Two ways to keep the hand-over
// coherent, the XCDs' L2 caches not being coherent with each other:
//
// LOCAL (hidden kept in one XCD's L2): a workgroup serves the queue of the
//   XCD it runs on (read from the XCC_ID hardware register, so the
//   placement is known, not assumed); each entry's gate/up and down slices
//   all belong to that one queue (fused_seq / fused_ticket in rmoe_sched.h),
//   so producer and consumer of a hidden row share the XCD's L2: gate/up
//   stores are ordinary write-back stores, counted once they have completed
//   into L2, and a down tile only drops its CU's L1 (buffer_inv sc0) after
//   its wait.  Hidden rows then move beyond L2 only when the L2 evicts them.
//   Progress: every gate/up ticket of an entry precedes its down tickets in
//   the same queue, so a waiting workgroup waits only for tickets already
//   handed to running workgroups of its own XCD, whatever else is resident.
//   A queue that no workgroup served (an XCD with no workgroup of this
//   launch) is drained by the last workgroup out, which then runs those
//   entries' gate/up slices before their down slices itself.
// global (hidden handed across XCDs; used when a pair's hidden rows would
//   not fit an L2 or there are too few entries to balance 8 queues):
//   workgroup w serves group w % 8; a group's queue holds its gate/up items,
//   then its down items, in the orders of the two persistent launches.  The
//   gate/up tiles store their hidden rows with device-scope (sc1)
//   write-through stores and wait for them to complete before counting --
//   the effect of an agent-scope release without writing back the whole L2,
//   which measured ~2-5% of the launch -- and a down tile drops its CU's and
//   XCD's stale copies (agent-scope acquire) before reading them.  Progress:
//   a workgroup waits only while holding a down ticket, i.e. after every
//   gate/up ticket of its own queue was handed to a running workgroup, and
//   gate/up items never wait; so every wait ends once one workgroup of each
//   queue runs (dispatch in workgroup order gives every queue one of the
//   first eight workgroups).
// Each wait is bounded all the same, by wait_ticks of the constant-rate
// real-time counter: a wait that gives up skips its item, adds 1 to the
// sticky error word and raises the launch's abort flag, after which every
// wait gives up at once, so the kernel always exits within about one
// deadline.  The last workgroup out returns the tickets, the counters, the
// abort flag and the exit count to zero, ready for the next launch.
__device__ __forceinline__ int xcc_id() {
    return (int)__builtin_amdgcn_s_getreg((3 << 11) | 20);  // hwreg(HW_REG_XCC_ID, 0, 4)
}

template <bool LOCAL>
__device__ void serve_queue(const StageArgs &gu, const StageArgs &dn, int32_t *sync,
                            uint64_t wait_ticks, int grp, unsigned char *smem) {
    int *bcast = reinterpret_cast<int *>(smem);  // LDS is idle between items
    int32_t *tickets = sync + RMOE_FUSED_SYNC_TICKETS;
    int32_t *done = sync + RMOE_FUSED_SYNC_HEAD;
    const int NT1 = (int)(gu.N / 128), NT2 = (int)((dn.N + 255) / 256);
    FusedSeq fq{};
    TileSeq seq1{}, seq2{};
    int n_all;
    if constexpr (LOCAL) {
        fq = fused_seq(gu.gs, gu.E, NT1, NT2, grp, kXcd);
        n_all = fq.n;
    } else {
        seq1 = tile_seq(gu.gs, gu.E, NT1, grp, kXcd);
        seq2 = tile_seq(dn.gs, dn.E, NT2, grp, kXcd);
        n_all = seq1.n + seq2.n;
    }
    TileCursor cur, cur_dn;
    for (;;) {
        __syncthreads();  // every wave is done with the LDS of the last item
        if (threadIdx.x == 0)
            bcast[0] = __hip_atomic_fetch_add(tickets + grp, 1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const int t = bcast[0];
        if (t >= n_all) break;
        bool down;
        TileItem it;
        if constexpr (LOCAL) {
            const FusedTicket k = fused_ticket(fq, t);
            if (k.j >= fq.J) continue;  // void ticket of the padded last unit
            down = k.down;
            if (down)
                it = entry_item(gu.gs, gu.gpo, fq.lo + k.j, k.nt, cur_dn);
            else
                it = entry_item(gu.gs, gu.gpo, fq.lo + k.j, k.nt, cur);
        } else {
            down = t >= seq1.n;
            it = down ? tile_item(dn.gs, dn.gpo, seq2, t - seq1.n, cur)
                      : tile_item(gu.gs, gu.gpo, seq1, t, cur);
        }
        if (!down) {
            __syncthreads();  // the ticket is read before the DMAs reuse its LDS word
            // LOCAL: write-back stores into this XCD's L2; global: write-through
            // at device scope, visible to every XCD once completed
            run_item<true, !LOCAL>(gu, smem, it);
            wait_vm<0>();  // this wave's hidden stores have completed
            __syncthreads();
            if (threadIdx.x == 0)
                __hip_atomic_fetch_add(done + it.bx, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            if (threadIdx.x == 0) {
                const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
                bool ready;
                for (;;) {
                    ready = __hip_atomic_load(done + it.bx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= NT1;
                    if (ready) break;
                    // give up past the deadline, or at once once any wait of this launch has
                    if (__hip_atomic_load(sync + RMOE_FUSED_SYNC_ABORT, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) != 0 ||
                        __builtin_amdgcn_s_memrealtime() - t0 > wait_ticks)
                        break;
                    __builtin_amdgcn_s_sleep(8);
                }
                // acquire before any wave reads (the barrier below orders
                // their loads after it): LOCAL drops this CU's L1 only (the
                // rows sit in this XCD's L2); global also drops the XCD's
                // stale L2 copies
                if constexpr (LOCAL)
                    asm volatile("buffer_inv sc0\n\ts_waitcnt vmcnt(0)" ::: "memory");
                else
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                if (!ready) {
                    __hip_atomic_fetch_add(sync + RMOE_FUSED_SYNC_ERROR, 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(sync + RMOE_FUSED_SYNC_ABORT, 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
                bcast[1] = ready;
            }
            __syncthreads();
            const bool ready = bcast[1] != 0;
            __syncthreads();  // the flag is read before the DMAs reuse its LDS word
            if (!ready) continue;
            run_item<false>(dn, smem, it);
        }
    }
}

template <bool LOCAL>
__global__ __launch_bounds__(256) void fused_kernel(StageArgs gu, StageArgs dn, int32_t *sync,
                                                    uint64_t wait_ticks) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    int *bcast = reinterpret_cast<int *>(smem);
    int32_t *tickets = sync + RMOE_FUSED_SYNC_TICKETS;
    int32_t *done = sync + RMOE_FUSED_SYNC_HEAD;
    // first the queue of this workgroup's group; then, in the last workgroup
    // out only (every other one has finished), LOCAL runs every queue no
    // workgroup served (none ran on that XCD) -- a served queue is already
    // drained, its ticket past its end.  One call site keeps one inlined copy.
    int g = LOCAL ? __builtin_amdgcn_readfirstlane(xcc_id()) % kXcd : (int)(blockIdx.x % kXcd);
    bool last = false;
    for (;;) {
        serve_queue<LOCAL>(gu, dn, sync, wait_ticks, g, smem);
        if (!last) {
            __syncthreads();  // every wave has read the final ticket
            if (threadIdx.x == 0)
                bcast[0] = __hip_atomic_fetch_add(sync + RMOE_FUSED_SYNC_EXIT, 1, __ATOMIC_ACQ_REL,
                                                  __HIP_MEMORY_SCOPE_AGENT) == (int)gridDim.x - 1;
            __syncthreads();
            if (!bcast[0]) return;
            last = true;
            if (!LOCAL) break;
            g = 0;
        } else if (++g == kXcd) {
            break;
        }
    }
    // reset the queue state (the error word stays)
    __syncthreads();
    for (int i = threadIdx.x; i < kXcd; i += blockDim.x) tickets[i] = 0;
    for (int i = threadIdx.x; i < gu.M; i += blockDim.x) done[i] = 0;
    if (threadIdx.x == 0) {
        sync[RMOE_FUSED_SYNC_ABORT] = 0;
        sync[RMOE_FUSED_SYNC_EXIT] = 0;
    }
}

// Workgroup slots of the persistent kernel on the current device: its CU
// count rounded down to a multiple of 8 (cached per device).
hipError_t persistent_grid(unsigned &grid) {
    static std::atomic<int> cached[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int n = dev < 64 ? cached[dev].load(std::memory_order_relaxed) : 0;
    if (n == 0) {
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        n = n / kXcd * kXcd;
        if (n < kXcd) n = kXcd;
        if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
    }
    grid = (unsigned)n;
    return hipSuccess;
}

// Rate of the real-time counter (s_memrealtime) on the current device, in
// kHz (cached per device; 100 MHz where the runtime reports none).
hipError_t wall_clock_khz(int &khz) {
    static std::atomic<int> cached[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int v = dev < 64 ? cached[dev].load(std::memory_order_relaxed) : 0;
    if (v == 0) {
        e = hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, dev);
        if (e != hipSuccess) return e;
        if (v <= 0) v = 100000;
        if (dev < 64) cached[dev].store(v, std::memory_order_relaxed);
    }
    khz = v;
    return hipSuccess;
}

template <bool DUAL>
hipError_t launch(const StageArgs &a, int NT, hipStream_t s) {
    unsigned grid = 0;
    hipError_t e = persistent_grid(grid);
    if (e != hipSuccess) return e;
    const unsigned lds = LDS_BYTES;  // above the 64 KB default, so opt in
    static std::atomic<uint64_t> lds_set{0};
    e = lds_opt_in_once((const void *)tile_kernel<DUAL>, (int)lds, lds_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(tile_kernel<DUAL>, dim3(grid), dim3(256), lds, s, a, NT);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_tile_gate_up(const StageArgs &a, hipStream_t s) {
    return launch<true>(a, (int)(a.N / 128), s);
}

hipError_t launch_tile_down(const StageArgs &a, hipStream_t s) {
    return launch<false>(a, (int)((a.N + 255) / 256), s);
}

hipError_t launch_fused(const StageArgs &gu, const StageArgs &dn, int32_t *sync, int64_t wait_us,
                        bool local, hipStream_t s) {
    unsigned grid = 0;
    hipError_t e = persistent_grid(grid);
    if (e != hipSuccess) return e;
    int khz = 0;
    e = wall_clock_khz(khz);
    if (e != hipSuccess) return e;
    const unsigned lds = LDS_BYTES;
    const uint64_t ticks = (uint64_t)khz * (uint64_t)wait_us / 1000u;
    if (local) {
        static std::atomic<uint64_t> lds_set{0};
        e = lds_opt_in_once((const void *)fused_kernel<true>, (int)lds, lds_set);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(fused_kernel<true>, dim3(grid), dim3(256), lds, s, gu, dn, sync, ticks);
    } else {
        static std::atomic<uint64_t> lds_set{0};
        e = lds_opt_in_once((const void *)fused_kernel<false>, (int)lds, lds_set);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(fused_kernel<false>, dim3(grid), dim3(256), lds, s, gu, dn, sync, ticks);
    }
    return hipGetLastError();
}

}  // namespace rmoe

#if RMOE_PHASE_TIMING
#include "../../include/routed_moe_phase.h"

int rmoe_phase_cycles(uint64_t *cycles, size_t bytes) {
    if (!cycles || bytes < sizeof(rmoe::phase_cycles)) return RMOE_ERR_INVALID_ARGUMENT;
    return hipMemcpyFromSymbol(cycles, HIP_SYMBOL(rmoe::phase_cycles), sizeof(rmoe::phase_cycles), 0,
                               hipMemcpyDeviceToHost) == hipSuccess
               ? RMOE_OK
               : RMOE_ERR_LAUNCH;
}
#endif
