// Device-side helpers shared by the gfx950 kernels: vector types, the
// block -> (expert, rows) predicate and the SwiGLU gate.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rmoe {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16x __attribute__((ext_vector_type(16)));

constexpr int kBlockM = 128;  // rows per contract block (block_token)

// Expert and valid-row count of block bx: the row predicate shared by the
// Step-1 and Step-2 grids ("Fused MoE GEMM 提交说明", 完整算子代码):
// actual_rows = max(0, min(128, group_size - (bx*128 - padded_start))).
struct BlockInfo {
    int e;             // expert of the block
    int token_offset;  // bx*128 - group_padded_offsets[e]
    int rows;          // valid rows in [0, 128]
};

// The block is computed only when group_idx_for_bx names the expert whose
// padded interval [gpo[e], gpo[e+1]) holds it; a table entry that names any
// other expert (or none) leaves the block's rows unwritten.  With a valid
// table this changes nothing; with a corrupted one both kernel families
// skip exactly the same blocks (the tiled family checks each block of its
// work items against the table the same way), and no read leaves the
// tables or the expert's rows.
__device__ __forceinline__ BlockInfo block_info(const int32_t *__restrict__ gs,
                                                const int32_t *__restrict__ gpo,
                                                const int32_t *__restrict__ gidx, int E, int bx) {
    BlockInfo b;
    b.e = gidx[bx];
    b.rows = 0;
    b.token_offset = 0;
    if (b.e < 0 || b.e >= E) return b;
    const int start = bx * kBlockM;
    if (start < gpo[b.e] || start >= gpo[b.e + 1]) return b;
    b.token_offset = start - gpo[b.e];
    int r = gs[b.e] - b.token_offset;
    b.rows = r < 0 ? 0 : (r > kBlockM ? kBlockM : r);
    return b;
}

// silu(g) = g * sigmoid(g) = g / (1 + e^-g), with the hardware exp2 and
// reciprocal (each ~1 ulp of fp32; the result is rounded to fp16, whose ulp
// is 2^13 times coarser).  For g -> -inf, e^-g -> inf and the reciprocal
// -> 0, so silu -> -0 as it should.
__device__ __forceinline__ float silu(float g) {
    return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
}

__device__ __forceinline__ h4 to_h4(float a, float b, float c, float d) {
    h4 r;
    r[0] = (_Float16)a;
    r[1] = (_Float16)b;
    r[2] = (_Float16)c;
    r[3] = (_Float16)d;
    return r;
}

// ---- global -> LDS staging shared by the LDS-fed kernels.  An LDS row holds
// 64 K-elements of one matrix row (one 128-byte line) as eight 16-byte chunks.

// Physical 16-byte position of logical chunk c in LDS row r.  A 256-byte
// sweep of the 64 banks holds two rows; XOR-ing the chunk with (r / 2) % 8
// gives the 16 consecutive rows of an operand read (ds_read_b128, 16 lanes
// per LDS cycle) distinct banks.
__device__ __forceinline__ int lds_swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int lds_off(int r, int c) { return r * 128 + ((c ^ lds_swz(r)) << 4); }

// One 1 KB global -> LDS DMA (global_load_lds_dwordx4): lane i stores the
// 16 bytes at g to LDS byte lds + 16 i.  Counted by vmcnt like a load.
__device__ __forceinline__ void dma16(const void *g, unsigned lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g)
                 : "memory", "m0");
}

// The same with the non-temporal hint, for lines read once (streamed weight
// rows): MI355X serves a read stream with that hint ~13% faster (about 7.0
// against 6.2 TB/s in a 4 GiB read probe).
__device__ __forceinline__ void dma16_nt(const void *g, unsigned lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(lds), "v"(g)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(N) only (expcnt and lgkmcnt left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
}

// Bare workgroup barrier: no memory fence, so outstanding DMAs stay in flight.
__device__ __forceinline__ void bar() {
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace rmoe
