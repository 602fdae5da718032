// Device-side dispatch contract: the tables of the MoE dispatch contract
// ("moe_dispatch_contract.py", build_contract) computed on the GPU from the
// router's top-k ids, so a forward pass needs no host round trip.
//
// Pairs p = t*k + j are cut into chunks of CHUNK consecutive pairs:
//   1. hist: per-chunk expert histogram (LDS atomics on integer counts, so
//      the result is exact and independent of their order);
//   2. scan: one workgroup turns the per-chunk counts into each chunk's
//      exclusive start inside every expert, and the expert totals into
//      group_sizes, group_offsets and group_padded_offsets (padded size of
//      an expert with c pairs: ceil((c+1)/128)*128);
//   3. scatter: every chunk walks its pairs 256 at a time in pair order; a
//      pair's rank among the earlier pairs of its expert in its wave comes
//      from one ballot per bit of the expert id, and the four waves take
//      their positions in pair order, so the sort is stable (ascending pair
//      index inside an expert) and the tables are unique;
//   4. blocks: group_idx_for_bx[bx] = the last expert whose padded start is
//      <= bx*128 (binary search over the strictly increasing starts).
// Pairs whose expert id lies outside [0, E) are left out of every table,
// get -1 as padded row and compact position, and are counted in *bad.
// A batch that fits one chunk (decode-sized) runs all four steps in one
// workgroup and one launch, with the same arithmetic.
#include <atomic>

#include "rmoe_device.h"
#include "rmoe_internal.h"

namespace rmoe {

// Library-owned scratch of the contract build that allocates nothing
// (rmoe_build_contract_device_noalloc): the per-chunk expert counts, kept in
// one static array per GPU for the life of the process.  Host code never
// passes `scratch` itself (on the host that name is only a stand-in): its
// device address is fetched once per device with hipGetSymbolAddress.
static __device__ __align__(256) int32_t scratch[kNoAllocScratchWords];

hipError_t noalloc_scratch(int32_t **ptr) {
    static std::atomic<int32_t *> cached[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    int32_t *p = cached[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        void *addr = nullptr;
        e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        p = static_cast<int32_t *>(addr);
        cached[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

namespace {

constexpr int TPB = 256;
constexpr int CHUNK = 2048;  // pairs per chunk
constexpr int SMALL_E = 1024;  // expert bound of the one-launch path (its LDS)
constexpr int NWAVE = TPB / 64;

// Exclusive scans of two per-thread values over the workgroup, in thread
// order (shuffles within each wave, then the wave totals); also the totals.
// Integer sums: exact, whatever the order.  Every thread must call it.
__device__ __forceinline__ void block_scan2(int32_t c, int32_t p, int32_t &exc_c, int32_t &exc_p,
                                            int32_t &tot_c, int32_t &tot_p, int32_t *wsum_c,
                                            int32_t *wsum_p) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int32_t ic = c, ip = p;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t tc = __shfl_up(ic, d), tp = __shfl_up(ip, d);
        if (lane >= d) {
            ic += tc;
            ip += tp;
        }
    }
    if (lane == 63) {
        wsum_c[wave] = ic;
        wsum_p[wave] = ip;
    }
    __syncthreads();
    exc_c = ic - c;
    exc_p = ip - p;
    tot_c = 0;
    tot_p = 0;
#pragma unroll
    for (int w = 0; w < NWAVE; ++w) {
        if (w < wave) {
            exc_c += wsum_c[w];
            exc_p += wsum_p[w];
        }
        tot_c += wsum_c[w];
        tot_p += wsum_p[w];
    }
    __syncthreads();  // wsum_* may be reused
}

// Stable placement of 256 consecutive pairs (one per thread, in pair order;
// valid = its expert e lies in [0, E)): the lanes of a wave holding the same
// expert are found with one ballot per bit of the expert id (a lane keeps
// the lanes whose bit agrees with its own, bit after bit), which gives the
// pair's rank among the earlier pairs of its expert in its wave; then the
// waves take their positions from next[] in pair order and advance it.
// Returns the compact position, or -1 for an invalid pair.  Every thread
// must call it (nbits: bits of E - 1, uniform).
__device__ __forceinline__ int32_t place_pairs(int32_t e, bool valid, int nbits, int32_t *next) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    uint64_t same = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
        const bool set = (e >> bit) & 1;
        const uint64_t m = __ballot(set);
        same &= set ? m : ~m;
    }
    const int rank = __popcll(same & below), cnt = __popcll(same);
    int32_t pos = -1;
    for (int w = 0; w < NWAVE; ++w) {
        if (wave == w && valid) {
            pos = next[e] + rank;
            if (rank == cnt - 1) next[e] = pos + 1;  // after every lane of the wave read next[e]
        }
        __syncthreads();
    }
    return pos;
}

__global__ __launch_bounds__(TPB) void hist_kernel(const int32_t *__restrict__ ids, int64_t pairs,
                                                   int32_t E, int32_t *__restrict__ cc,
                                                   int32_t *__restrict__ bad_c) {
    extern __shared__ int32_t h[];  // E counts + 1 out-of-range count
    for (int e = threadIdx.x; e <= E; e += TPB) h[e] = 0;
    __syncthreads();
    const int64_t c0 = (int64_t)blockIdx.x * CHUNK;
    for (int i = threadIdx.x; i < CHUNK; i += TPB) {
        const int64_t p = c0 + i;
        if (p >= pairs) break;
        const int32_t e = ids[p];
        atomicAdd(&h[(e >= 0 && e < E) ? e : E], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += TPB) cc[(int64_t)blockIdx.x * E + e] = h[e];
    if (threadIdx.x == 0) bad_c[blockIdx.x] = h[E];
}

// one workgroup; dynamic LDS: E expert totals
__global__ __launch_bounds__(TPB) void scan_kernel(int32_t *__restrict__ cc,
                                                   const int32_t *__restrict__ bad_c, int32_t nch,
                                                   int32_t E, int32_t *__restrict__ gs,
                                                   int32_t *__restrict__ go, int32_t *__restrict__ gpo,
                                                   int32_t *__restrict__ bad) {
    extern __shared__ int32_t cnt[];
    __shared__ int32_t wsum_c[NWAVE], wsum_p[NWAVE];
    // per expert: exclusive scan over the chunks, in place; total -> gs.
    // Counts are read 8 chunks at a time, so the loads of a group overlap.
    for (int e = threadIdx.x; e < E; e += TPB) {
        int32_t run = 0;
        for (int c0 = 0; c0 < nch; c0 += 8) {
            int32_t v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = c0 + j < nch ? cc[(int64_t)(c0 + j) * E + e] : 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (c0 + j < nch) {
                    cc[(int64_t)(c0 + j) * E + e] = run;
                    run += v[j];
                }
            }
        }
        cnt[e] = run;
        gs[e] = run;
    }
    // out-of-range pairs of every chunk
    int32_t nb = 0;
    for (int c = threadIdx.x; c < nch; c += TPB) nb += bad_c[c];
    __syncthreads();
    // exclusive scans over the experts: each thread a contiguous segment
    const int seg = (E + TPB - 1) / TPB;
    const int e0 = min(E, (int)threadIdx.x * seg), e1 = min(E, e0 + seg);
    int32_t sc = 0, sp = 0;
    for (int e = e0; e < e1; ++e) {
        sc += cnt[e];
        sp += (cnt[e] / kBlockM + 1) * kBlockM;  // ceil((c+1)/128)*128
    }
    int32_t rc, rp, tc, tp, xb, xd, tb, td;
    block_scan2(sc, sp, rc, rp, tc, tp, wsum_c, wsum_p);
    block_scan2(nb, 0, xb, xd, tb, td, wsum_c, wsum_p);  // tb: the out-of-range total
    if (threadIdx.x == 0) {
        go[E] = tc;
        gpo[E] = tp;
        *bad = tb;
    }
    for (int e = e0; e < e1; ++e) {
        go[e] = rc;
        gpo[e] = rp;
        rc += cnt[e];
        rp += (cnt[e] / kBlockM + 1) * kBlockM;
    }
}

__global__ __launch_bounds__(TPB) void scatter_kernel(const int32_t *__restrict__ ids, int64_t pairs,
                                                      int32_t E, const int32_t *__restrict__ cc,
                                                      const int32_t *__restrict__ go,
                                                      const int32_t *__restrict__ gpo,
                                                      int32_t *__restrict__ order,
                                                      int32_t *__restrict__ prow,
                                                      int32_t *__restrict__ cpos) {
    extern __shared__ int32_t base[];  // [E] next compact position per expert
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    for (int e = threadIdx.x; e < E; e += TPB) base[e] = go[e] + cc[(int64_t)blockIdx.x * E + e];
    __syncthreads();
    const int64_t c0 = (int64_t)blockIdx.x * CHUNK;
    for (int sub = 0; sub < CHUNK && c0 + sub < pairs; sub += TPB) {  // uniform bound
        const int64_t p = c0 + sub + threadIdx.x;
        const int32_t e = p < pairs ? ids[p] : -1;
        const bool valid = e >= 0 && e < E;
        const int32_t pos = place_pairs(e, valid, nbits, base);
        if (p < pairs) {
            if (valid) {
                order[pos] = (int32_t)p;
                cpos[p] = pos;
                prow[p] = gpo[e] + (pos - go[e]);
            } else {
                cpos[p] = -1;
                prow[p] = -1;
            }
        }
    }
}

__global__ __launch_bounds__(TPB) void blocks_kernel(const int32_t *__restrict__ gpo, int32_t E,
                                                     int32_t M, int32_t *__restrict__ gidx) {
    const int bx = blockIdx.x * TPB + threadIdx.x;
    if (bx >= M) return;
    const int64_t t = (int64_t)bx * kBlockM;
    int lo = 0, hi = E - 1;  // gpo[0] = 0 <= t, starts strictly increase
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if ((int64_t)gpo[mid] <= t)
            lo = mid;
        else
            hi = mid - 1;
    }
    gidx[bx] = lo;
}

// All four steps for a batch of at most CHUNK pairs and at most SMALL_E
// experts: one workgroup, tables kept in LDS between the steps.
__global__ __launch_bounds__(TPB) void small_contract_kernel(const int32_t *__restrict__ ids,
                                                             int32_t pairs, int32_t E, int32_t M,
                                                             int32_t *__restrict__ gs,
                                                             int32_t *__restrict__ go,
                                                             int32_t *__restrict__ gpo,
                                                             int32_t *__restrict__ gidx,
                                                             int32_t *__restrict__ order,
                                                             int32_t *__restrict__ prow,
                                                             int32_t *__restrict__ cpos,
                                                             int32_t *__restrict__ bad) {
    __shared__ int32_t h[SMALL_E + 1];    // counts (+ out-of-range), then next position
    __shared__ int32_t lgo[SMALL_E + 1], lgpo[SMALL_E + 1];
    __shared__ int32_t wsum_c[NWAVE], wsum_p[NWAVE];
    // 1. histogram
    for (int e = threadIdx.x; e <= E; e += TPB) h[e] = 0;
    __syncthreads();
    for (int p = threadIdx.x; p < pairs; p += TPB) {
        const int32_t e = ids[p];
        atomicAdd(&h[(e >= 0 && e < E) ? e : E], 1);
    }
    __syncthreads();
    // 2. totals and the two exclusive scans over the experts: each thread
    //    sums a contiguous run of experts, then a scan across the threads
    const int seg = (E + TPB - 1) / TPB;
    const int e0 = min(E, (int)threadIdx.x * seg), e1 = min(E, e0 + seg);
    int32_t sc = 0, sp = 0;
    for (int e = e0; e < e1; ++e) {
        gs[e] = h[e];
        sc += h[e];
        sp += (h[e] / kBlockM + 1) * kBlockM;  // ceil((c+1)/128)*128
    }
    int32_t rc, rp, tc, tp;
    block_scan2(sc, sp, rc, rp, tc, tp, wsum_c, wsum_p);
    if (threadIdx.x == 0) {
        go[E] = lgo[E] = tc;
        gpo[E] = lgpo[E] = tp;
        *bad = h[E];
    }
    for (int e = e0; e < e1; ++e) {
        go[e] = lgo[e] = rc;
        gpo[e] = lgpo[e] = rp;
        rc += h[e];
        rp += (h[e] / kBlockM + 1) * kBlockM;
    }
    __syncthreads();  // every count was read: h[] becomes the next compact position
    for (int e = threadIdx.x; e < E; e += TPB) h[e] = lgo[e];
    __syncthreads();
    // 3. stable scatter, 256 pairs at a time in pair order
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    for (int sub = 0; sub < pairs; sub += TPB) {
        const int p = sub + threadIdx.x;
        const int32_t e = p < pairs ? ids[p] : -1;
        const bool valid = e >= 0 && e < E;
        const int32_t pos = place_pairs(e, valid, nbits, h);
        if (p < pairs) {
            if (valid) {
                order[pos] = p;
                cpos[p] = pos;
                prow[p] = lgpo[e] + (pos - lgo[e]);
            } else {
                cpos[p] = -1;
                prow[p] = -1;
            }
        }
    }
    // 4. block -> expert: the last expert whose padded start is <= bx*128
    for (int bx = threadIdx.x; bx < M; bx += TPB) {
        const int64_t t = (int64_t)bx * kBlockM;
        int lo = 0, hi = E - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) / 2;
            if ((int64_t)lgpo[mid] <= t)
                lo = mid;
            else
                hi = mid - 1;
        }
        gidx[bx] = lo;
    }
}

// The contract's rules on device tables ("moe_dispatch_contract.py", the
// three self-checks in their strict form), counted: offsets start at 0 and
// step by the group sizes, each padded span is (size/128 + 1)*128, the
// compact total is the pair count, the padded total fits in M blocks, and
// every block maps to the last expert whose padded start is <= bx*128.
// One workgroup; each violated rule instance adds 1.
__global__ __launch_bounds__(TPB) void validate_kernel(const int32_t *__restrict__ gs,
                                                       const int32_t *__restrict__ go,
                                                       const int32_t *__restrict__ gpo,
                                                       const int32_t *__restrict__ gidx, int32_t E,
                                                       int32_t M, int64_t pairs,
                                                       int32_t *__restrict__ violations) {
    __shared__ int32_t bad;
    if (threadIdx.x == 0) bad = 0;
    __syncthreads();
    int32_t mine = 0;
    if (threadIdx.x == 0) {
        mine += go[0] != 0;
        mine += gpo[0] != 0;
        mine += (int64_t)go[E] != pairs;
        mine += (int64_t)gpo[E] > (int64_t)M * kBlockM;
    }
    for (int e = threadIdx.x; e < E; e += TPB) {
        const int64_t c = gs[e];
        mine += c < 0;
        mine += (int64_t)go[e + 1] - go[e] != c;
        mine += (int64_t)gpo[e + 1] - gpo[e] != (c / kBlockM + 1) * kBlockM;
    }
    for (int bx = threadIdx.x; bx < M; bx += TPB) {
        const int64_t t = (int64_t)bx * kBlockM;
        int lo = 0, hi = E - 1;  // stays in [0, E) whatever gpo holds
        while (lo < hi) {
            const int mid = (lo + hi + 1) / 2;
            if ((int64_t)gpo[mid] <= t)
                lo = mid;
            else
                hi = mid - 1;
        }
        mine += gidx[bx] != lo;
    }
    if (mine) atomicAdd(&bad, mine);
    __syncthreads();
    if (threadIdx.x == 0) *violations = bad;
}

}  // namespace

hipError_t launch_validate(const int32_t *gs, const int32_t *go, const int32_t *gpo,
                           const int32_t *gidx, int32_t E, int32_t M, int64_t pairs,
                           int32_t *violations, hipStream_t s) {
    hipLaunchKernelGGL(validate_kernel, dim3(1), dim3(TPB), 0, s, gs, go, gpo, gidx, E, M, pairs,
                       violations);
    return hipGetLastError();
}

int64_t contract_chunks(int64_t pairs) { return (pairs + CHUNK - 1) / CHUNK; }

hipError_t launch_contract(const int32_t *ids, int64_t pairs, int32_t E, int32_t M, int32_t *gs,
                           int32_t *go, int32_t *gpo, int32_t *gidx, int32_t *order, int32_t *prow,
                           int32_t *cpos, int32_t *bad, int32_t *ws, hipStream_t s) {
    const int64_t nch = contract_chunks(pairs);
    if (nch <= 1 && E <= SMALL_E) {
        hipLaunchKernelGGL(small_contract_kernel, dim3(1), dim3(TPB), 0, s, ids, (int32_t)pairs, E, M, gs,
                           go, gpo, gidx, order, prow, cpos, bad);
        return hipGetLastError();
    }
    int32_t *cc = ws;                // [nch][E]
    int32_t *bad_c = ws + nch * E;   // [nch]
    const size_t lds = (size_t)(E + 1) * sizeof(int32_t);
    if (nch > 0) {
        hipLaunchKernelGGL(hist_kernel, dim3((unsigned)nch), dim3(TPB), lds, s, ids, pairs, E, cc, bad_c);
    }
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(TPB), lds, s, cc, bad_c, (int32_t)nch, E, gs, go, gpo, bad);
    if (nch > 0) {
        hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)nch), dim3(TPB), lds, s, ids, pairs, E, cc, go,
                           gpo, order, prow, cpos);
    }
    if (M > 0) {
        hipLaunchKernelGGL(blocks_kernel, dim3((unsigned)((M + TPB - 1) / TPB)), dim3(TPB), 0, s, gpo, E, M,
                           gidx);
    }
    return hipGetLastError();
}

}  // namespace rmoe
