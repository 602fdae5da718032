/*
 * Oracle: routed fused-MoE expert FFN, plain C, one padded row at a time.
 * TEST INFRASTRUCTURE ONLY: loaded by tests/, the smoke check and the
 * benchmark's CPU-baseline leg; the product path never links or calls it.
 * It shares no code, header or table with the HIP library.
 *
 * What it computes ("Fused MoE GEMM 提交说明", section 算子来源, the
 * computation semantics; dtypes from section 完整算子代码):
 *     gate   = x . Wg[e]^T          fp16 inputs, fp32 accumulation
 *     up     = x . Wu[e]^T          fp16 inputs, fp32 accumulation
 *     hidden = silu(gate) * up      fp32, then rounded to the fp16 workspace
 *     acc    = hidden . Wd[e]^T     fp16 inputs, fp32 accumulation
 *     out    = acc * w              fp32 routed weight, rounded to fp16
 * Rows and the expert of each 128-row block follow the kernel's row predicate
 * (same section, both grids): only rows i < actual_rows of a block are
 * computed and written; padding rows are left untouched (section 实现要点).
 *
 * Arithmetic choices (the pages fix fp16 storage and fp32 accumulation):
 *   - every dot product is a sequential fp32 sum in ascending index order,
 *     product then add (built with -ffp-contract=off, no fast-math);
 *   - silu(v) = v / (1 + exp(-v)) evaluated in fp32 with expf; the page
 *     writes the same function as v * 1/(1 + 2^(-v*log2 e));
 *   - fp32 -> fp16 is IEEE round-to-nearest-even with subnormals kept,
 *     written out below from the binary16 format definition.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- IEEE binary16 <-> binary32 ------------------------------------------ */

/* Exact widening of a binary16 bit pattern. */
float oracle_f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h >> 15) << 31;
    uint32_t exp = (h >> 10) & 0x1f;
    uint32_t man = h & 0x3ff;
    float mag;
    if (exp == 0x1f) {
        uint32_t bits = sign | 0x7f800000u | (man << 13); /* inf / nan */
        float f;
        memcpy(&f, &bits, 4);
        return f;
    }
    if (exp == 0)
        mag = ldexpf((float)man, -24);                  /* subnormal or zero */
    else
        mag = ldexpf((float)(man | 0x400), (int)exp - 25); /* 1.man * 2^(exp-15) */
    return sign ? -mag : mag;
}

/* Round a binary32 value to the nearest binary16, ties to even. */
uint16_t oracle_f32_to_f16(float f) {
    uint32_t bits;
    memcpy(&bits, &f, 4);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    uint32_t exp = (bits >> 23) & 0xff;
    uint32_t man = bits & 0x7fffff;
    if (exp == 0xff) /* inf stays inf; nan stays a quiet nan */
        return (uint16_t)(sign | 0x7c00u | (man ? 0x200u | (man >> 13) : 0));
    /* value = m * 2^q with an integer significand m (24 bits when normal) */
    int32_t q;
    uint32_t m;
    if (exp == 0) {
        m = man;
        q = -149;
    } else {
        m = man | 0x800000u;
        q = (int32_t)exp - 150;
    }
    if (m == 0)
        return sign;
    /* binary16 quantum at the value's binade: 2^-24 for subnormals and the
     * smallest binade, 2^(E-10) for a value in [2^E, 2^(E+1)). */
    int32_t top = q + 23; /* exponent of the leading bit when normal */
    if (exp == 0) {
        top = q;
        for (uint32_t t = m; t > 1; t >>= 1) top++;
    }
    int32_t quantum = top - 10;
    if (quantum < -24) quantum = -24;
    int32_t shift = quantum - q; /* bits of m below the binary16 quantum */
    uint32_t n;
    if (shift <= 0) {
        n = m << (-shift); /* exact (only when q >= quantum) */
    } else if (shift >= 32) {
        n = 0;             /* far below half of the smallest subnormal */
    } else {
        n = m >> shift;
        uint32_t rem = m & ((1u << shift) - 1u);
        uint32_t half = 1u << (shift - 1);
        if (rem > half || (rem == half && (n & 1u))) n++;
    }
    /* n counts quanta of 2^quantum; rebuild the binary16 fields */
    if (quantum == -24) {
        /* n * 2^-24 with n <= 2048: below 1024 the encoding is the subnormal
         * field n; from 1024 (2^-14) up to 2048 (2^-13) the exponent field 1
         * or 2 plus the fraction spell the same integer n */
        return (uint16_t)(sign | n);
    }
    /* normal: n in [1024, 2048]; 2048 means the rounding carried a binade */
    int32_t e16 = top + 15;
    if (n == 0x800) {
        n = 0x400;
        e16 += 1;
    }
    if (e16 >= 31) return (uint16_t)(sign | 0x7c00u); /* overflow -> inf */
    return (uint16_t)(sign | ((uint32_t)e16 << 10) | (n - 0x400));
}

/* ---- one padded row ------------------------------------------------------ */

static float silu_f32(float v) { return v / (1.0f + expf(-v)); }

/*
 * One token row through expert e.  x_row: [H] fp16; wg_e, wu_e: [I, H] fp16
 * (row n is output feature n, K = H contiguous, nn.Linear layout as in the
 * kernel signature); wd_e: [H, I] fp16.  Writes hid_row [I] and out_row [H]
 * as fp16 bit patterns.  scratch_h: [I] floats of caller-owned scratch.
 */
void oracle_moe_row(const uint16_t *x_row, const uint16_t *wg_e, const uint16_t *wu_e,
                    const uint16_t *wd_e, float routed_weight, int64_t H, int64_t I,
                    uint16_t *hid_row, uint16_t *out_row, float *scratch_h) {
    for (int64_t n = 0; n < I; n++) {
        float gate = 0.0f, up = 0.0f;
        const uint16_t *g = wg_e + n * H;
        const uint16_t *u = wu_e + n * H;
        for (int64_t h = 0; h < H; h++) {
            float xv = oracle_f16_to_f32(x_row[h]);
            gate += xv * oracle_f16_to_f32(g[h]);
            up += xv * oracle_f16_to_f32(u[h]);
        }
        uint16_t hv = oracle_f32_to_f16(silu_f32(gate) * up);
        hid_row[n] = hv;
        scratch_h[n] = oracle_f16_to_f32(hv); /* the down GEMM reads the fp16 workspace */
    }
    for (int64_t m = 0; m < H; m++) {
        float acc = 0.0f;
        const uint16_t *d = wd_e + m * I;
        for (int64_t n = 0; n < I; n++) acc += scratch_h[n] * oracle_f16_to_f32(d[n]);
        out_row[m] = oracle_f32_to_f16(acc * routed_weight);
    }
}

/*
 * Whole forward over the padded layout, block by block, with the kernel's
 * row predicate.  Tables are the contract: group_sizes [E],
 * group_offsets [E+1], group_padded_offsets [E+1], group_idx_for_bx [M].
 * x: [Tp, H]; wg, wu: [E, I, H]; wd: [E, H, I]; w_compact: [pairs] fp32;
 * hid: [Tp, I]; out: [Tp, H].  Rows that no block computes are not touched.
 * scratch: n_threads * I floats.  Returns the number of rows computed.
 */
int64_t oracle_moe_forward(const uint16_t *x, const uint16_t *wg, const uint16_t *wu,
                           const uint16_t *wd, const float *w_compact,
                           const int32_t *group_sizes, const int32_t *group_offsets,
                           const int32_t *group_padded_offsets,
                           const int32_t *group_idx_for_bx, int32_t num_blocks_m,
                           int64_t H, int64_t I, uint16_t *hid, uint16_t *out,
                           float *scratch, int32_t n_threads) {
    const int64_t B = 128;
    int64_t done = 0;
    /* one task per (block, row); rows are independent */
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads) reduction(+ : done)
    for (int64_t task = 0; task < (int64_t)num_blocks_m * B; task++) {
        int64_t bx = task / B, i = task % B;
        int32_t e = group_idx_for_bx[bx];
        int64_t token_offset = bx * B - group_padded_offsets[e];
        int64_t rows = group_sizes[e] - token_offset;
        if (rows > B) rows = B;
        if (rows < 0) rows = 0;
        if (i >= rows) continue;
        int64_t r = bx * B + i;
        float routed = w_compact[group_offsets[e] + token_offset + i];
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        oracle_moe_row(x + r * H, wg + (int64_t)e * I * H, wu + (int64_t)e * I * H,
                       wd + (int64_t)e * H * I, routed, H, I, hid + r * I, out + r * H,
                       scratch + (int64_t)tid * I);
        done += 1;
    }
    return done;
}

/*
 * A list of rows, each with its own expert slices (for sampled checks at
 * sizes where only some experts' weights are on the host).  Row j uses
 * x_rows[j], wg_list[j], wu_list[j], wd_list[j] and weights[j].
 */
void oracle_moe_rows(int64_t n_rows, const uint16_t *const *x_rows,
                     const uint16_t *const *wg_list, const uint16_t *const *wu_list,
                     const uint16_t *const *wd_list, const float *weights, int64_t H,
                     int64_t I, uint16_t *hid, uint16_t *out, float *scratch,
                     int32_t n_threads) {
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads)
    for (int64_t j = 0; j < n_rows; j++) {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        oracle_moe_row(x_rows[j], wg_list[j], wu_list[j], wd_list[j], weights[j], H, I,
                       hid + j * I, out + j * H, scratch + (int64_t)tid * I);
    }
}
