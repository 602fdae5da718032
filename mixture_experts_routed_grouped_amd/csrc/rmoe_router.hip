// Router: logits = x W^T, softmax over the experts, top-k ids and scores
// ("MetaX-TileLang工具链", section 2.4: the reference router is a linear gate,
// a softmax, a top-k; no renormalisation of the k scores is stated, so the
// scores are the softmax probabilities).
//
// One workgroup = TOK tokens (64 or 32) x every expert (E padded to a
// multiple of 32, at most 256).  Tokens and gate rows travel HBM/L2 -> LDS
// by DMA in K-chunks of 64 (8 rows x 128 bytes per instruction) through a
// 4-stage ring (one barrier per chunk); v_mfma_f32_32x32x16_f16 with gate
// rows as A and a 32-token tile as B, fp32 logits.  TOK = 64: 4 waves = 2
// token halves x 2 interleaved sets of 32-expert tiles; TOK = 32: one token
// tile, 4 interleaved sets of expert tiles -- or, with fewer than four
// expert tiles (E <= 64), the waves also split each chunk's four K-steps
// (E <= 32: one K-step per wave; E <= 64: two), so that every wave has work
// and a chunk costs one or two dependent MFMAs instead of four (64 tokens,
// E = 8, H = 4096: two workgroups of 64 chunks); their partial logits are
// added in a fixed order.  TOK = 32 gives twice the
// workgroups, i.e. more memory streams per CU, for batches that would not
// fill the chip twice over (16384 tokens, H = 7168, E = 128: 197 -> 100 us).
// The logits go through LDS; 4 lanes per token then take the row maximum,
// the exponential sum and k rounds of arg-max (equal scores: lower expert
// index first), combining with lane shuffles.  The gate matrix ([E, H],
// ~1.8 MB at E = 128, H = 7168) stays in L2; x is read once.
#include "rmoe_device.h"
#include "rmoe_internal.h"

namespace rmoe {
namespace {

constexpr int RT_CK = 64;   // K per chunk
constexpr int RT_NST = 4;   // LDS ring stages: DMA runs 3 chunks ahead

template <int EP, int TOK>
struct RouterCfg {
    static constexpr int TROWS = TOK;             // LDS token rows
    static constexpr int ROWS = TROWS + EP;       // LDS rows per chunk: tokens, then gate rows
    static constexpr int STAGE = ROWS * 128;
    static constexpr int NI = ROWS / 8;           // DMA instructions per chunk
    static_assert(NI % 4 == 0, "DMA split over 4 waves");
    static constexpr int NIW = NI / 4;            // per wave
    static constexpr int NT = EP / 32;            // 32-expert tiles
    static constexpr int EW = TOK == 64 ? 2 : 4;  // waves sharing the expert tiles
    static constexpr int TPW = (NT + EW - 1) / EW;  // tiles per wave
    // waves per expert tile that split a chunk's 4 K-steps (TOK = 32 only)
    static constexpr int KSW = TOK == 32 && NT == 1 ? 4 : TOK == 32 && NT == 2 ? 2 : 1;
    static constexpr int LDS_BYTES = RT_NST * STAGE;  // >= the TROWS x EP fp32 logits
    static_assert(TOK == 64 || TOK == 32, "tokens per workgroup: whole 32-token tiles");
    static_assert(LDS_BYTES >= KSW * TROWS * EP * 4, "partial logits fit in the ring");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

__device__ __forceinline__ bool better(float s, int e, float s2, int e2) {
    return s > s2 || (s == s2 && e < e2);
}

template <int EP, int TOK>
__global__ __launch_bounds__(256) void router_kernel(const _Float16 *__restrict__ x,
                                                     const _Float16 *__restrict__ w, int64_t T,
                                                     int64_t H, int32_t E, int32_t k,
                                                     int32_t *__restrict__ ids,
                                                     float *__restrict__ vals) {
    using C = RouterCfg<EP, TOK>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int64_t t0 = (int64_t)blockIdx.x * TOK;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, lr = lane & 31, lh = lane >> 5;
    // token tile of this wave, and its first expert tile (then every EW-th)
    // (with KSW > 1: expert tile wave % NT, K-steps s with s % KSW == ks)
    const int ks = C::KSW > 1 ? wave / C::NT : 0;
    const int th = TOK == 64 ? (wave & 1) : 0;
    const int eh = TOK == 64 ? (wave >> 1) : C::KSW > 1 ? wave % C::NT : wave;

    // DMA sources: instruction j = wave*NIW + i moves rows 8j .. 8j+7 of the
    // chunk (rows < TOK: tokens, clamped to the last token; the rest: gate
    // rows, clamped to the last expert -- padding rows feed outputs nobody reads)
    const _Float16 *src[C::NIW];
#pragma unroll
    for (int i = 0; i < C::NIW; ++i) {
        const int r = 8 * (wave * C::NIW + i) + (lane >> 3);
        const int c = (lane & 7) ^ lds_swz(r);
        if (r < C::TROWS) {
            const int64_t row = t0 + r < T ? t0 + r : T - 1;
            src[i] = x + row * H + 8 * c;
        } else {
            const int e = r - C::TROWS < E ? r - C::TROWS : E - 1;
            src[i] = w + (int64_t)e * H + 8 * c;
        }
    }
    const unsigned sbase = (unsigned)(uintptr_t)smem + wave * C::NIW * 1024;
    // every workgroup reads the same gate rows: each starts its K sweep at a
    // different chunk, so that concurrent workgroups do not ask the L2 for
    // the same lines at the same moment (a token's sum order stays fixed)
    const int nk = (int)(H / RT_CK);
    const int kofs = (int)((blockIdx.x * 7u) % (unsigned)nk);
    auto dma_chunk = [&](int kc, int stage) {
        const int kk = kc + kofs < nk ? kc + kofs : kc + kofs - nk;
#pragma unroll
        for (int i = 0; i < C::NIW; ++i) dma16(src[i] + (int64_t)kk * RT_CK, sbase + stage * C::STAGE + i * 1024);
    };

    f16x acc[C::TPW];
#pragma unroll
    for (int t = 0; t < C::TPW; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;

#pragma unroll
    for (int p = 0; p < RT_NST - 1; ++p) dma_chunk(p < nk ? p : nk - 1, p);
    for (int kc = 0; kc < nk; ++kc) {
        wait_vm<(RT_NST - 2) * C::NIW>();  // chunk kc landed (own DMAs) ...
        bar();  // ... and everyone's; and every wave is done with chunk kc-1's stage
        // refill that stage (clamped at the end: repeats land in stages no
        // later chunk reads)
        dma_chunk(kc + RT_NST - 1 < nk ? kc + RT_NST - 1 : nk - 1, (kc + RT_NST - 1) % RT_NST);
        const unsigned char *base = smem + (kc % RT_NST) * C::STAGE;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s % C::KSW != ks) continue;
            const h8 b = *(const h8 *)(base + lds_off(32 * th + lr, 2 * s + lh));
#pragma unroll
            for (int t = 0; t < C::TPW; ++t) {
                const int et = eh + C::EW * t;
                if (et < C::NT) {
                    const h8 a = *(const h8 *)(base + lds_off(C::TROWS + 32 * et + lr, 2 * s + lh));
                    acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[t], 0, 0, 0);
                }
            }
        }
    }
    wait_vm<0>();
    bar();

    // ---- logits -> LDS [TROWS tokens][EP experts] fp32 (partial logits of
    //      K-split ks at L + ks * TROWS * EP, then added in order of ks).
    //      32x32 accumulator layout: register 4q + r holds expert row
    //      8q + 4lh + r, token lr.
    float *L = reinterpret_cast<float *>(smem);
#pragma unroll
    for (int t = 0; t < C::TPW; ++t) {
        const int et = eh + C::EW * t;
        if (et < C::NT) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    L[ks * C::TROWS * EP + (32 * th + lr) * EP + 32 * et + 8 * q + 4 * lh + r] = acc[t][4 * q + r];
        }
    }
    __syncthreads();
    if constexpr (C::KSW > 1) {
        for (int i = tid; i < C::TROWS * EP; i += 256) {
            float v = L[i];
#pragma unroll
            for (int j = 1; j < C::KSW; ++j) v += L[j * C::TROWS * EP + i];
            L[i] = v;
        }
        __syncthreads();
    }

    // ---- softmax and top-k: 4 consecutive lanes per token, lane `sub` owns
    //      experts sub, sub + 4, ...
    const int tok = tid >> 2, sub = tid & 3;
    float *row = L + tok * EP;
    float m = -__builtin_inff();
    for (int e = sub; e < E; e += 4) m = fmaxf(m, row[e]);
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    float sum = 0.f;
    for (int e = sub; e < E; e += 4) {
        const float p = __builtin_amdgcn_exp2f((row[e] - m) * 1.4426950408889634f);
        row[e] = p;
        sum += p;
    }
    sum += __shfl_xor(sum, 1);
    sum += __shfl_xor(sum, 2);
    const float inv = 1.0f / sum;
    uint64_t taken = 0;  // bit i: expert sub + 4i already chosen
    const bool live = tok < TOK && t0 + tok < T;
    for (int j = 0; j < k; ++j) {
        float bs = -1.f;
        int be = 0x7fffffff;
        for (int e = sub, i = 0; e < E; e += 4, ++i) {
            if ((taken >> i) & 1) continue;
            const float s = row[e] * inv;
            if (better(s, e, bs, be)) {
                bs = s;
                be = e;
            }
        }
#pragma unroll
        for (int d = 1; d <= 2; d <<= 1) {
            const float os = __shfl_xor(bs, d);
            const int oe = __shfl_xor(be, d);
            if (better(os, oe, bs, be)) {
                bs = os;
                be = oe;
            }
        }
        if ((be & 3) == sub) taken |= 1ull << (be >> 2);
        if (live && sub == 0) {
            ids[(t0 + tok) * k + j] = be;
            vals[(t0 + tok) * k + j] = bs;
        }
    }
}

template <int EP, int TOK>
hipError_t launch_ep(const _Float16 *x, const _Float16 *w, int64_t T, int64_t H, int32_t E,
                     int32_t k, int32_t *ids, float *vals, hipStream_t s) {
    using C = RouterCfg<EP, TOK>;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = lds_opt_in_once((const void *)router_kernel<EP, TOK>, C::LDS_BYTES, lds_set);
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)((T + TOK - 1) / TOK);
    hipLaunchKernelGGL((router_kernel<EP, TOK>), dim3(grid), dim3(256), C::LDS_BYTES, s, x, w, T, H,
                       E, k, ids, vals);
    return hipGetLastError();
}

template <int EP>
hipError_t launch_tok(int tok, const _Float16 *x, const _Float16 *w, int64_t T, int64_t H,
                      int32_t E, int32_t k, int32_t *ids, float *vals, hipStream_t s) {
    if (tok == 64) return launch_ep<EP, 64>(x, w, T, H, E, k, ids, vals, s);
    return launch_ep<EP, 32>(x, w, T, H, E, k, ids, vals, s);
}

// Compute units of the current device (cached per device).
hipError_t cu_count(int &n) {
    static std::atomic<int> cached[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    n = dev < 64 ? cached[dev].load(std::memory_order_relaxed) : 0;
    if (n == 0) {
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        if (n < 1) n = 1;
        if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_router(const _Float16 *x, const _Float16 *w, int64_t T, int64_t H, int32_t E,
                         int32_t k, int32_t *ids, float *vals, hipStream_t s) {
    if (T == 0 || k == 0) return hipSuccess;
    // tokens per workgroup: 64 once that still gives two workgroups per CU
    int cus = 0;
    hipError_t e = cu_count(cus);
    if (e != hipSuccess) return e;
    const int tok = T >= (int64_t)64 * 2 * cus ? 64 : 32;
    switch ((E + 31) / 32) {
        case 1: return launch_tok<32>(tok, x, w, T, H, E, k, ids, vals, s);
        case 2: return launch_tok<64>(tok, x, w, T, H, E, k, ids, vals, s);
        case 3: return launch_tok<96>(tok, x, w, T, H, E, k, ids, vals, s);
        case 4: return launch_tok<128>(tok, x, w, T, H, E, k, ids, vals, s);
        case 5: return launch_tok<160>(tok, x, w, T, H, E, k, ids, vals, s);
        case 6: return launch_tok<192>(tok, x, w, T, H, E, k, ids, vals, s);
        case 7: return launch_tok<224>(tok, x, w, T, H, E, k, ids, vals, s);
        case 8: return launch_tok<256>(tok, x, w, T, H, E, k, ids, vals, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace rmoe
