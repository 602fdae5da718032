// Weight-streaming grouped GEMM for blocks with few valid rows (decode-
// shaped batches).  Such blocks make the expert FFN bound by reading the
// expert weights from HBM (with few tokens per expert the padded expert
// GEMMs turn memory-bound, as the contract tutorial notes), so this family
// is organised around keeping many weight bytes in flight:
//
//   * one workgroup = one 128-row block x TF output features (TF = 16 or
//     32), KS waves that split K; each wave streams its contiguous K range
//     of the TF weight rows straight from HBM into MFMA operand registers --
//     no LDS staging, every weight byte is read once per 32-token pass;
//   * weights are the MFMA A operand (feature rows), tokens the B operand,
//     so a lane ends up with 4 consecutive features of one token (8-byte
//     fp16 stores).  TF = 32 uses v_mfma_f32_32x32x16_f16 (one token
//     fragment serves 32 features); TF = 16 uses v_mfma_f32_16x16x32_f16
//     with two 16-token groups;
//   * a ring of D chunk buffers in registers: the loads of chunk c+D-1 are
//     issued before the MFMAs of chunk c; weight loads are non-temporal (each
//     byte is used once), so the token rows stay in L2;
//   * the KS partial sums are added in a fixed order through LDS
//     (deterministic, no atomics), the epilogue is split over the waves.
//
// Blocks with no valid row exit at once, so the tail blocks and the slack
// block of a full group touch no weight.
#include <type_traits>

#include "rmoe_device.h"
#include "rmoe_internal.h"

#ifndef RMOE_GU_MF
#define RMOE_GU_MF 32
#endif
#ifndef RMOE_GU_KS
#define RMOE_GU_KS 4
#endif
#ifndef RMOE_GU_D
#define RMOE_GU_D 2
#endif
#ifndef RMOE_DN_MF
#define RMOE_DN_MF 32
#endif
#ifndef RMOE_DN_KS
#define RMOE_DN_KS 4
#endif
#ifndef RMOE_DN_D
#define RMOE_DN_D 3
#endif
#ifndef RMOE_STREAM_NT
#define RMOE_STREAM_NT 0
#endif
#ifndef RMOE_STREAM_ILV
#define RMOE_STREAM_ILV 1  // K split interleaved chunk by chunk across the waves
#endif

namespace rmoe {
namespace {

template <int MF>
struct Shape {
    static constexpr int KSTEP = MF == 16 ? 32 : 16;  // K of one MFMA
    static constexpr int CK = 4 * KSTEP;              // K per chunk (4 MFMA steps)
    static constexpr int NG = MF == 16 ? 2 : 1;       // token fragments per 32-token pass
    static constexpr int NQ = MF == 16 ? 2 : 4;       // 4-register output quads per matrix
    using Acc = std::conditional_t<MF == 16, f4, f16x>;
};

template <bool DUAL, int MF>
struct Frag {
    static constexpr int NM = DUAL ? 2 : 1;
    h8 w[NM][4];
    h8 x[Shape<MF>::NG][4];
};

template <bool NT>
__device__ __forceinline__ h8 load_w(const _Float16 *p) {
    if constexpr (NT)
        return __builtin_nontemporal_load(reinterpret_cast<const h8 *>(p));
    else
        return *reinterpret_cast<const h8 *>(p);
}

template <bool DUAL, int MF, bool NT>
__device__ __forceinline__ void chunk_load(Frag<DUAL, MF> &f, const _Float16 *w0,
                                           const _Float16 *w1, const _Float16 *x, int64_t K,
                                           int ng, int64_t k) {
    constexpr int KS = Shape<MF>::KSTEP;
#pragma unroll
    for (int s = 0; s < 4; ++s) f.w[0][s] = load_w<NT>(w0 + k + KS * s);
    if constexpr (DUAL) {
#pragma unroll
        for (int s = 0; s < 4; ++s) f.w[1][s] = load_w<NT>(w1 + k + KS * s);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) f.x[0][s] = *reinterpret_cast<const h8 *>(x + k + KS * s);
    if constexpr (MF == 16) {
        if (ng > 1) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
                f.x[1][s] = *reinterpret_cast<const h8 *>(x + 16 * K + k + KS * s);
        }
    }
}

template <bool DUAL, int MF>
__device__ __forceinline__ void chunk_mma(const Frag<DUAL, MF> &f,
                                          typename Shape<MF>::Acc (&acc)[2][2], int ng) {
    constexpr int NM = DUAL ? 2 : 1;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if constexpr (MF == 16) {
                acc[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.w[m][s], f.x[0][s], acc[m][0], 0, 0, 0);
            } else {
                acc[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.w[m][s], f.x[0][s], acc[m][0], 0, 0, 0);
            }
        }
    }
    if constexpr (MF == 16) {
        if (ng > 1) {
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int m = 0; m < NM; ++m)
                    acc[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.w[m][s], f.x[1][s], acc[m][1], 0, 0, 0);
        }
    }
}

// Register r (0..3) of output quad q: its 4 consecutive features and token.
//   TF = 32: token lane & 31, features 8 q + 4 (lane >> 5) + r
//   TF = 16: quad q is token group q: token 16 q + (lane & 15), features 4 (lane >> 4) + r
template <int MF>
__device__ __forceinline__ void quad_pos(int q, int lane, int &tok, int &feat) {
    if constexpr (MF == 32) {
        tok = lane & 31;
        feat = 8 * q + 4 * (lane >> 5);
    } else {
        tok = 16 * q + (lane & 15);
        feat = 4 * (lane >> 4);
    }
}

template <int MF>
__device__ __forceinline__ float acc_get(const typename Shape<MF>::Acc (&acc)[2], int q, int r) {
    if constexpr (MF == 32)
        return acc[0][4 * q + r];
    else
        return acc[q][r];
}

// grid: (N / MF, num_blocks_m); block: 64 * KS threads.
template <bool DUAL, int MF, int KS, int D, bool NT>
__global__ __launch_bounds__(64 * KS) void stream_kernel(StageArgs a) {
    using S = Shape<MF>;
    using Acc = typename S::Acc;
    constexpr int NM = DUAL ? 2 : 1;
    const int bx = blockIdx.y;
    const BlockInfo bi = block_info(a.gs, a.gpo, a.gidx, bx);
    if (bi.rows == 0) return;

    // wave-uniform by construction; readfirstlane lets the compiler keep the
    // K range and every loop bound in scalar registers (uniform branches)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int lrow = MF == 16 ? (lane & 15) : (lane & 31);  // A row / B token of this lane
    const int koff = MF == 16 ? 8 * (lane >> 4) : 8 * (lane >> 5);
    const int64_t K = a.K, N = a.N;
    const int n0 = blockIdx.x * MF;

    // K split.  Interleaved: wave w takes chunks w, w + KS, w + 2 KS, ... so
    // the KS waves of a workgroup read neighbouring chunks of the same weight
    // rows at the same time -- KS * CK * 2 contiguous bytes per row in flight
    // instead of CK * 2 (DRAM pages are opened for longer runs).  Otherwise
    // each wave takes one contiguous quarter of K.
    const int nchunks = (int)(K / S::CK);
#if RMOE_STREAM_ILV
    const int c_begin = wave;
    const int c_step = KS;
    const int n_mine = (nchunks - wave + KS - 1) / KS;
#else
    const int c_begin = (nchunks * wave) / KS;
    const int c_step = 1;
    const int n_mine = (nchunks * (wave + 1)) / KS - c_begin;
#endif

    const _Float16 *w0 = a.w0 + ((int64_t)bi.e * N + n0 + lrow) * K + koff;
    const _Float16 *w1 = DUAL ? a.w1 + ((int64_t)bi.e * N + n0 + lrow) * K + koff : nullptr;

    __shared__ float red[KS > 1 ? KS : 1][NM][16][64];

    for (int prow0 = 0; prow0 < bi.rows; prow0 += 32) {
        const int left = bi.rows - prow0;
        const int ng = (MF == 16 && left > 16) ? 2 : 1;
        const _Float16 *x = a.x + ((int64_t)bx * kBlockM + prow0 + lrow) * K + koff;

        Acc acc[2][2];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int g = 0; g < 2; ++g) acc[m][g] = Acc{};

        // Ring of D chunks.  Prefetches are unconditional -- past the end of
        // the range they re-read the last chunk (an L2 hit) -- so the loop
        // body has no load under a branch and the wait counts stay exact.
        const int n = n_mine;
        if (n > 0) {
            const _Float16 *w0c = w0 + (int64_t)c_begin * S::CK;
            const _Float16 *w1c = DUAL ? w1 + (int64_t)c_begin * S::CK : nullptr;
            const _Float16 *xc = x + (int64_t)c_begin * S::CK;
            Frag<DUAL, MF> ring[D];
#pragma unroll
            for (int j = 0; j < D - 1; ++j)
                chunk_load<DUAL, MF, NT>(ring[j], w0c, w1c, xc, K, ng,
                                         (int64_t)min(j, n - 1) * c_step * S::CK);
            for (int i = 0; i < n; i += D) {
#pragma unroll
                for (int j = 0; j < D; ++j) {
                    const int cc = i + j;
                    chunk_load<DUAL, MF, NT>(ring[(j + D - 1) % D], w0c, w1c, xc, K, ng,
                                             (int64_t)min(cc + D - 1, n - 1) * c_step * S::CK);
                    // keep the prefetch ahead of the MFMAs: without this fence
                    // the scheduler sinks the loads below them to save
                    // registers and the ring degenerates to depth 1
                    __builtin_amdgcn_sched_barrier(0);
                    if (cc < n) chunk_mma<DUAL, MF>(ring[j], acc, ng);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }

        // ---- fixed-order reduction of the KS partial sums; quads split over waves
        if constexpr (KS > 1) {
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int q = 0; q < S::NQ; ++q)
#pragma unroll
                    for (int r = 0; r < 4; ++r) red[wave][m][4 * q + r][lane] = acc_get<MF>(acc[m], q, r);
            __syncthreads();
        }
#pragma unroll
        for (int q = 0; q < S::NQ; ++q) {
            if (KS > 1 && q % KS != wave) continue;  // quad q belongs to wave q % KS
            if (MF == 16 && q >= ng) continue;
            int tok, feat;
            quad_pos<MF>(q, lane, tok, feat);
            tok += prow0;
            if (tok >= bi.rows) continue;
            float v[NM][4];
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if constexpr (KS > 1) {
                        float s = red[0][m][4 * q + r][lane];
#pragma unroll
                        for (int w = 1; w < KS; ++w) s += red[w][m][4 * q + r][lane];
                        v[m][r] = s;
                    } else {
                        v[m][r] = acc_get<MF>(acc[m], q, r);
                    }
                }
            const int64_t row = (int64_t)bx * kBlockM + tok;
            _Float16 *dst = a.y + row * N + n0 + feat;
            h4 o;
            if constexpr (DUAL) {
                o = to_h4(silu(v[0][0]) * v[1][0], silu(v[0][1]) * v[1][1],
                          silu(v[0][2]) * v[1][2], silu(v[0][3]) * v[1][3]);
            } else {
                const float w = a.rw[a.go[bi.e] + bi.token_offset + tok];
                o = to_h4(v[0][0] * w, v[0][1] * w, v[0][2] * w, v[0][3] * w);
            }
            *reinterpret_cast<h4 *>(dst) = o;
        }
        if constexpr (KS > 1) __syncthreads();  // red[] is reused by the next pass
    }
}

}  // namespace

hipError_t launch_stream_gate_up(const StageArgs &a, hipStream_t s) {
    constexpr int MF = RMOE_GU_MF;
    dim3 grid((unsigned)(a.N / MF), (unsigned)a.M);
    hipLaunchKernelGGL((stream_kernel<true, MF, RMOE_GU_KS, RMOE_GU_D, RMOE_STREAM_NT != 0>), grid,
                       dim3(64 * RMOE_GU_KS), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_stream_down(const StageArgs &a, hipStream_t s) {
    constexpr int MF = RMOE_DN_MF;
    dim3 grid((unsigned)(a.N / MF), (unsigned)a.M);
    hipLaunchKernelGGL((stream_kernel<false, MF, RMOE_DN_KS, RMOE_DN_D, RMOE_STREAM_NT != 0>), grid,
                       dim3(64 * RMOE_DN_KS), 0, s, a);
    return hipGetLastError();
}

}  // namespace rmoe
