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
//      pair's rank among the earlier pairs of its expert in the same 256 is
//      counted directly, so the sort is stable (ascending pair index inside
//      an expert) and the tables are unique;
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
    __shared__ int32_t part_c[TPB], part_p[TPB];
    // per expert: exclusive scan over the chunks, in place; total -> gs
    for (int e = threadIdx.x; e < E; e += TPB) {
        int32_t run = 0;
        for (int c = 0; c < nch; ++c) {
            const int32_t v = cc[(int64_t)c * E + e];
            cc[(int64_t)c * E + e] = run;
            run += v;
        }
        cnt[e] = run;
        gs[e] = run;
    }
    __syncthreads();
    // exclusive scans over the experts: each thread a contiguous segment
    const int seg = (E + TPB - 1) / TPB;
    const int e0 = min(E, (int)threadIdx.x * seg), e1 = min(E, e0 + seg);
    int32_t sc = 0, sp = 0;
    for (int e = e0; e < e1; ++e) {
        sc += cnt[e];
        sp += (cnt[e] / kBlockM + 1) * kBlockM;  // ceil((c+1)/128)*128
    }
    part_c[threadIdx.x] = sc;
    part_p[threadIdx.x] = sp;
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t rc = 0, rp = 0;
        for (int i = 0; i < TPB; ++i) {
            const int32_t vc = part_c[i], vp = part_p[i];
            part_c[i] = rc;
            part_p[i] = rp;
            rc += vc;
            rp += vp;
        }
        go[E] = rc;
        gpo[E] = rp;
        int32_t nb = 0;
        for (int c = 0; c < nch; ++c) nb += bad_c[c];
        *bad = nb;
    }
    __syncthreads();
    int32_t rc = part_c[threadIdx.x], rp = part_p[threadIdx.x];
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
    __shared__ int32_t eid[TPB];
    for (int e = threadIdx.x; e < E; e += TPB) base[e] = go[e] + cc[(int64_t)blockIdx.x * E + e];
    __syncthreads();
    const int64_t c0 = (int64_t)blockIdx.x * CHUNK;
    for (int sub = 0; sub < CHUNK && c0 + sub < pairs; sub += TPB) {  // uniform bound
        const int64_t p = c0 + sub + threadIdx.x;
        const int32_t e = p < pairs ? ids[p] : -1;
        const bool valid = e >= 0 && e < E;
        eid[threadIdx.x] = valid ? e : -1;
        __syncthreads();
        int32_t rank = 0, tot = 0, pos = -1;
        if (valid) {
            for (int j = 0; j < TPB; ++j) {
                const bool same = eid[j] == e;
                rank += (same && j < (int)threadIdx.x) ? 1 : 0;
                tot += same ? 1 : 0;
            }
            pos = base[e] + rank;
        }
        __syncthreads();  // every pair read base[] before it moves on
        if (valid && rank == tot - 1) base[e] += tot;
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
        __syncthreads();  // eid[] and base[] are reused by the next 256 pairs
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
    __shared__ int32_t part_c[TPB], part_p[TPB], eid[TPB];
    // 1. histogram
    for (int e = threadIdx.x; e <= E; e += TPB) h[e] = 0;
    __syncthreads();
    for (int p = threadIdx.x; p < pairs; p += TPB) {
        const int32_t e = ids[p];
        atomicAdd(&h[(e >= 0 && e < E) ? e : E], 1);
    }
    __syncthreads();
    // 2. totals and the two exclusive scans over the experts
    const int seg = (E + TPB - 1) / TPB;
    const int e0 = min(E, (int)threadIdx.x * seg), e1 = min(E, e0 + seg);
    int32_t sc = 0, sp = 0;
    for (int e = e0; e < e1; ++e) {
        gs[e] = h[e];
        sc += h[e];
        sp += (h[e] / kBlockM + 1) * kBlockM;  // ceil((c+1)/128)*128
    }
    part_c[threadIdx.x] = sc;
    part_p[threadIdx.x] = sp;
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t rc = 0, rp = 0;
        for (int i = 0; i < TPB; ++i) {
            const int32_t vc = part_c[i], vp = part_p[i];
            part_c[i] = rc;
            part_p[i] = rp;
            rc += vc;
            rp += vp;
        }
        go[E] = lgo[E] = rc;
        gpo[E] = lgpo[E] = rp;
        *bad = h[E];
    }
    __syncthreads();
    {
        int32_t rc = part_c[threadIdx.x], rp = part_p[threadIdx.x];
        for (int e = e0; e < e1; ++e) {
            go[e] = lgo[e] = rc;
            gpo[e] = lgpo[e] = rp;
            rc += h[e];
            rp += (h[e] / kBlockM + 1) * kBlockM;
        }
    }
    __syncthreads();  // every count was read: h[] becomes the next compact position
    for (int e = threadIdx.x; e < E; e += TPB) h[e] = lgo[e];
    __syncthreads();
    // 3. stable scatter, 256 pairs at a time in pair order
    for (int sub = 0; sub < pairs; sub += TPB) {
        const int p = sub + threadIdx.x;
        const int32_t e = p < pairs ? ids[p] : -1;
        const bool valid = e >= 0 && e < E;
        eid[threadIdx.x] = valid ? e : -1;
        __syncthreads();
        int32_t rank = 0, tot = 0, pos = -1;
        if (valid) {
            for (int j = 0; j < TPB; ++j) {
                const bool same = eid[j] == e;
                rank += (same && j < (int)threadIdx.x) ? 1 : 0;
                tot += same ? 1 : 0;
            }
            pos = h[e] + rank;
        }
        __syncthreads();  // every pair read h[] before it moves on
        if (valid && rank == tot - 1) h[e] += tot;
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
        __syncthreads();  // eid[] and h[] are reused by the next 256 pairs
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
