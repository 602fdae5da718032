// Weight-streaming grouped GEMM for blocks with few valid rows (decode-
// shaped batches).  With few tokens per expert the padded expert GEMMs turn
// memory-bound (as the contract tutorial notes): the time is the time to
// read the routed experts' weights from HBM once, so this family is built
// around the access pattern HBM serves fastest.
//
//   * one workgroup = one 128-row block x FT tiles of 32 output features
//     (gate/up: one tile, its gate and up rows; down: two tiles, so each
//     token chunk serves twice the weight bytes -- down 155 -> 147 us on a
//     decode batch, while a second gate/up tile measured 1.5% slower); KS
//     waves split K into contiguous ranges and run independently until the
//     final reduction (no barrier in the K loop);
//   * weights travel HBM -> LDS by direct DMA (global_load_lds_dwordx4) in
//     chunks of K = 64: each instruction reads 8 weight rows x 128 bytes,
//     with the non-temporal hint (weights are read once).  Measured on
//     MI355X, that pattern streams from HBM at ~6.5 TB/s, while loading the
//     MFMA operand layout straight into registers (32 rows x 32 bytes per
//     instruction) reaches ~4 TB/s.  Each wave owns a ring of
//     D chunk slots, refilled D-1 chunks ahead; MFMA operands come back out
//     of LDS with swizzled, conflict-free ds_read_b128;
//   * the pass's tokens (one to three 32-token MFMA tiles: the narrowest
//     pass that holds the block's rows, up to 96) ride in the same slots
//     (tokens are shared by all workgroups of the block and come from L2),
//     so every global read is a DMA and the only waits are the explicit
//     vmcnt ones; a block of 97-128 rows takes a 96-token pass and a
//     32-token one, reading its weights twice;
//   * weights are the MFMA A operand (v_mfma_f32_32x32x16_f16, 32 feature
//     rows), tokens the B operand; a lane ends up with 4 consecutive
//     features of one token, so stores are 8-byte fp16 quads;
//   * the KS partial sums are added in a fixed order through LDS
//     (deterministic, no atomics), the epilogue is split over the waves.
//
// Blocks with no valid row exit at once, so the tail blocks and the slack
// block of a full group touch no weight.
#include "rmoe_device.h"
#include "rmoe_internal.h"

#ifndef RMOE_GU_KS
#define RMOE_GU_KS 4  // waves (K ranges) per workgroup, gate/up
#endif
#ifndef RMOE_GU_D
#define RMOE_GU_D 2   // ring slots per wave, gate/up
#endif
#ifndef RMOE_DN_KS
#define RMOE_DN_KS 4
#endif
#ifndef RMOE_DN_D
#define RMOE_DN_D 2
#endif

namespace rmoe {
namespace {

constexpr int MF = 32;                // output features per workgroup (MFMA rows)
constexpr int CK = 64;                // K per chunk: one 128-byte line per weight row
constexpr int CHUNK_B = MF * CK * 2;  // 4 KB: one matrix's chunk

// TT: 32-token tiles per pass: 1, 2 or 3 (96 tokens, the largest pass the
// 160 KB of LDS holds); a block takes the narrowest pass that holds its rows,
// so it reads its weights once instead of once per 32-token tile.
// FT: 32-feature weight tiles per workgroup, the same for every pass width
// (one grid serves them all): gate/up one (its gate and up rows; the wider
// passes leave no LDS for a second), down two.
template <bool DUAL, int KS, int D, int TT>
struct StreamCfg {
    static constexpr int FT = DUAL ? 1 : 2;
    static constexpr int G = DUAL ? 2 : 1;                  // matrices per feature tile: gate and up, or down
    static constexpr int NM = G * FT;                       // weight tiles: matrix g of feature tile f is g + G f
    static constexpr int SLOT = (NM + TT) * CHUNK_B;        // weights, then 32*TT token rows
    static constexpr int WAVE_LDS = D * SLOT;               // ring of one wave
    static constexpr int RING = KS * WAVE_LDS;
    static constexpr int RED = KS * NM * TT * 16 * 64 * 4;  // partial sums of one pass
    static constexpr int LDS_BYTES = RING > RED ? RING : RED;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    static_assert((D - 1) * 4 * (NM + TT) < 64, "vmcnt range");
};

// One pass: the 32*TT tokens starting at row p0 of block bx against the 32
// features n0.. of the block's expert, over the whole K.  Only the first
// 8*TD token rows of the pass are moved (TD = ceil(valid rows / 8)): LDS rows
// past them keep stale values, which only reach MFMA output columns of
// tokens that are never stored.
template <bool DUAL, int KS, int D, int TT, int TD>
__device__ __forceinline__ void stream_pass(const StageArgs &a, const BlockInfo &bi, int bx, int p0,
                                            int n0, unsigned char *smem, int wave, int lane) {
    using C = StreamCfg<DUAL, KS, D, TT>;
    constexpr int NM = C::NM;
    constexpr int DMA_PER_CHUNK = 4 * NM + TD;
    const int64_t K = a.K, N = a.N;
    const int lr = lane & 31, lh = lane >> 5;

    // contiguous K range of this wave, in chunks
    const int nchunks = (int)(K / CK);
    const int c_begin = (nchunks * wave) / KS;
    const int n = (nchunks * (wave + 1)) / KS - c_begin;

    // DMA sources: instruction j of a weight matrix m moves rows 8j .. 8j+7
    // of its chunk, instruction j of the tokens rows 8j .. 8j+7 of the pass;
    // lane i takes row 8j + i/8 and physical chunk i%8, i.e. logical chunk
    // (i%8) ^ swz(row).  Token rows past the valid ones are read (they lie
    // inside the block) but never stored.
    const _Float16 *wsrc[NM][4], *tsrc[4 * TT];
#pragma unroll
    for (int j = 0; j < 4 * TT; ++j) {
        const int r = 8 * j + (lane >> 3);
        const int c = (lane & 7) ^ lds_swz(r);
        if (j < 4) {
#pragma unroll
            for (int m = 0; m < NM; ++m)
                wsrc[m][j] = (m % C::G ? a.w1 : a.w0) + ((int64_t)bi.e * N + n0 + 32 * (m / C::G) + r) * K +
                             (int64_t)c_begin * CK + 8 * c;
        }
        tsrc[j] = a.x + ((int64_t)bx * kBlockM + p0 + r) * K + (int64_t)c_begin * CK + 8 * c;
    }
    const unsigned wbase = (unsigned)(uintptr_t)smem + wave * C::WAVE_LDS;
    const unsigned char *wring = smem + wave * C::WAVE_LDS;
    auto dma_chunk = [&](int i, int slot) {
        const unsigned sb = wbase + slot * C::SLOT;
        // weight rows are read once: non-temporal; token rows are shared by
        // every slice of the block: cached normally
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) dma16_nt(wsrc[m][j] + (int64_t)i * CK, sb + m * CHUNK_B + 8 * j * 128);
#pragma unroll
        for (int j = 0; j < TD; ++j) dma16(tsrc[j] + (int64_t)i * CK, sb + NM * CHUNK_B + 8 * j * 128);
    };

    f16x acc[NM][TT];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[m][t][i] = 0.f;

    if (n > 0) {
#pragma unroll
        for (int j = 0; j < D - 1; ++j) dma_chunk(min(j, n - 1), j);
        for (int i = 0; i < n; ++i) {
            // refill the slot chunk i-1 used with chunk i+D-1 (clamped: the
            // repeats land in slots no later chunk reads), then wait for
            // chunk i, the oldest in flight
            dma_chunk(min(i + D - 1, n - 1), (i + D - 1) % D);
            wait_vm<(D - 1) * DMA_PER_CHUNK>();
            const unsigned char *slot = wring + (i % D) * C::SLOT;
            h8 af[NM][4], bf[TT][4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int off = lds_off(lr, 2 * s + lh);
#pragma unroll
                for (int m = 0; m < NM; ++m) af[m][s] = *(const h8 *)(slot + m * CHUNK_B + off);
#pragma unroll
                for (int t = 0; t < TT; ++t)
                    bf[t][s] = *(const h8 *)(slot + NM * CHUNK_B + lds_off(32 * t + lr, 2 * s + lh));
            }
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int t = 0; t < TT; ++t)
#pragma unroll
                    for (int m = 0; m < NM; ++m)
                        acc[m][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[m][s], bf[t][s], acc[m][t], 0, 0, 0);
        }
    }
    wait_vm<0>();  // no DMA may land in the ring once it holds partial sums
    __syncthreads();

    // ---- fixed-order reduction of the KS partial sums; output quad q (4
    //      features) of token tile t belongs to wave (4 t + q) % KS
    float *red = reinterpret_cast<float *>(smem);  // [KS][NM][TT][16][64]
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) red[(((wave * NM + m) * TT + t) * 16 + r) * 64 + lane] = acc[m][t][r];
    __syncthreads();
    [[maybe_unused]] const float *rwe = DUAL ? nullptr : a.rw + a.go[bi.e] + bi.token_offset;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        const int tok = p0 + 32 * t + lr;
#pragma unroll
        for (int f = 0; f < C::FT; ++f) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if ((4 * (t * C::FT + f) + q) % KS != wave || tok >= bi.rows) continue;
                // the matrices this output needs: gate and up, or down, of tile f
                float v[C::G][4];
#pragma unroll
                for (int mm = 0; mm < C::G; ++mm) {
                    const int m = mm + C::G * f;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float s = red[(((0 * NM + m) * TT + t) * 16 + 4 * q + r) * 64 + lane];
#pragma unroll
                        for (int w = 1; w < KS; ++w) s += red[(((w * NM + m) * TT + t) * 16 + 4 * q + r) * 64 + lane];
                        v[mm][r] = s;
                    }
                }
                // 32x32 accumulator layout: register 4q + r holds feature 8q + 4lh + r
                const int64_t row = (int64_t)bx * kBlockM + tok;
                _Float16 *dst = a.y + row * N + n0 + 32 * f + 8 * q + 4 * lh;
                h4 o;
                if constexpr (DUAL) {
                    o = to_h4(silu(v[0][0]) * v[1][0], silu(v[0][1]) * v[1][1], silu(v[0][2]) * v[1][2],
                              silu(v[0][3]) * v[1][3]);
                } else {
                    const float w = rwe[tok];
                    o = to_h4(v[0][0] * w, v[0][1] * w, v[0][2] * w, v[0][3] * w);
                }
                *reinterpret_cast<h4 *>(dst) = o;
            }
        }
    }
    __syncthreads();  // the next pass refills the ring that holds red[]
}

// grid: (N / (32 FT), num_blocks_m); block: 64 * KS threads; dynamic LDS: the
// largest pass's.  Each block is run in the fewest passes the LDS allows, so
// that its expert's weights are read once up to 96 rows: one pass of 32, 64
// or 96 tokens, or for 97-128 rows a 96-token pass and a 32-token one.  Token
// rows are moved in groups of 8 (16 for the wider passes, at most 8 rows past
// the valid ones and never past the block).
template <bool DUAL, int KS, int D>
__global__ __launch_bounds__(64 * KS) void stream_kernel(StageArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int bx = blockIdx.y;
    const BlockInfo bi = block_info(a.gs, a.gpo, a.gidx, a.E, bx);
    if (bi.rows == 0) return;
    // wave-uniform by construction; readfirstlane keeps the K range and the
    // loop bounds in scalar registers (uniform branches)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int n0 = blockIdx.x * MF * StreamCfg<DUAL, KS, D, 1>::FT;
    int p0 = 0;
    if (bi.rows > 96) {
        stream_pass<DUAL, KS, D, 3, 12>(a, bi, bx, 0, n0, smem, wave, lane);
        p0 = 96;
    }
    const int rem = bi.rows - p0;
    const int td = (rem + 7) / 8;  // token rows of the last pass, in 8s
    if (rem <= 32) {
        switch (td) {
            case 1: stream_pass<DUAL, KS, D, 1, 1>(a, bi, bx, p0, n0, smem, wave, lane); break;
            case 2: stream_pass<DUAL, KS, D, 1, 2>(a, bi, bx, p0, n0, smem, wave, lane); break;
            case 3: stream_pass<DUAL, KS, D, 1, 3>(a, bi, bx, p0, n0, smem, wave, lane); break;
            default: stream_pass<DUAL, KS, D, 1, 4>(a, bi, bx, p0, n0, smem, wave, lane); break;
        }
    } else if (rem <= 64) {
        if (td <= 6)
            stream_pass<DUAL, KS, D, 2, 6>(a, bi, bx, p0, n0, smem, wave, lane);
        else
            stream_pass<DUAL, KS, D, 2, 8>(a, bi, bx, p0, n0, smem, wave, lane);
    } else {
        if (td <= 10)
            stream_pass<DUAL, KS, D, 3, 10>(a, bi, bx, p0, n0, smem, wave, lane);
        else
            stream_pass<DUAL, KS, D, 3, 12>(a, bi, bx, p0, n0, smem, wave, lane);
    }
}

template <bool DUAL, int KS, int D>
hipError_t launch(const StageArgs &a, hipStream_t s) {
    using C1 = StreamCfg<DUAL, KS, D, 1>;
    using C2 = StreamCfg<DUAL, KS, D, 2>;
    using C3 = StreamCfg<DUAL, KS, D, 3>;
    static_assert(C1::FT == C2::FT && C2::FT == C3::FT, "one grid for every pass width");
    constexpr int lds = C3::LDS_BYTES > C2::LDS_BYTES ? (C3::LDS_BYTES > C1::LDS_BYTES ? C3::LDS_BYTES : C1::LDS_BYTES)
                                                       : (C2::LDS_BYTES > C1::LDS_BYTES ? C2::LDS_BYTES : C1::LDS_BYTES);
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = lds_opt_in_once((const void *)stream_kernel<DUAL, KS, D>, lds, lds_set);
    if (e != hipSuccess) return e;
    dim3 grid((unsigned)(a.N / (MF * C1::FT)), (unsigned)a.M);
    hipLaunchKernelGGL((stream_kernel<DUAL, KS, D>), grid, dim3(64 * KS), lds, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_stream_gate_up(const StageArgs &a, hipStream_t s) {
    return launch<true, RMOE_GU_KS, RMOE_GU_D>(a, s);
}

hipError_t launch_stream_down(const StageArgs &a, hipStream_t s) {
    return launch<false, RMOE_DN_KS, RMOE_DN_D>(a, s);
}

}  // namespace rmoe
