/*
 * A plain C caller of the routed fused-MoE library (include/routed_moe.h):
 * no Python, no torch, only the C ABI and the HIP runtime API for device
 * memory.  It runs one routed layer the way a C host program would:
 *
 *   host contract (rmoe_build_contract, checked by rmoe_validate_contract)
 *   -> device pack of the token rows and routed weights (rmoe_pack_f16)
 *   -> both expert stages (rmoe_forward_f16, the library's kernel choice)
 *   -> k-way combine back to token order (rmoe_combine_f16),
 *
 * on the default stream, then writes the combined output.
 *
 * Usage: c_abi_layer <dir> <tokens> <top_k> <experts> <hidden> <intermediate>
 * Inputs in <dir> (raw little-endian, row-major):
 *   x.bin   [T, H] fp16        ids.bin [T, k] int32      w.bin [T, k] fp32
 *   wg.bin, wu.bin [E, I, H] fp16                        wd.bin [E, H, I] fp16
 * Output: <dir>/y.bin [T, H] fp16.  Exit status 0 on success; on any error
 * it prints the failing call and the library's status string.
 *
 * Test infrastructure: the GPU test that runs it compares y.bin with the
 * oracle's layer on the same inputs.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../include/routed_moe.h"

#define FAIL(...)                     \
    do {                              \
        fprintf(stderr, __VA_ARGS__); \
        fputc('\n', stderr);          \
        exit(1);                      \
    } while (0)

#define HIP_OK(call)                                                     \
    do {                                                                 \
        hipError_t e_ = (call);                                          \
        if (e_ != hipSuccess) FAIL("%s: %s", #call, hipGetErrorString(e_)); \
    } while (0)

#define RMOE_OK_(call)                                                       \
    do {                                                                     \
        int s_ = (call);                                                     \
        if (s_ != RMOE_OK) FAIL("%s: %s (%d)", #call, rmoe_status_str(s_), s_); \
    } while (0)

static void *read_file(const char *dir, const char *name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE *f = fopen(path, "rb");
    if (!f) FAIL("cannot open %s", path);
    void *p = malloc(bytes ? bytes : 1);
    if (!p) FAIL("out of host memory");
    if (bytes && fread(p, 1, bytes, f) != bytes) FAIL("%s: short read", path);
    fclose(f);
    return p;
}

static void *to_device(const void *host, size_t bytes) {
    void *d = NULL;
    HIP_OK(hipMalloc(&d, bytes ? bytes : 16));
    if (bytes) HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

static void *device_buffer(size_t bytes) {
    void *d = NULL;
    HIP_OK(hipMalloc(&d, bytes ? bytes : 16));
    return d;
}

int main(int argc, char **argv) {
    if (argc != 7) FAIL("usage: %s <dir> <tokens> <top_k> <experts> <hidden> <intermediate>", argv[0]);
    const char *dir = argv[1];
    const int64_t T = atoll(argv[2]), H = atoll(argv[5]), I = atoll(argv[6]);
    const int32_t k = atoi(argv[3]), E = atoi(argv[4]);
    const int64_t pairs = T * k;

    /* inputs */
    uint16_t *x = read_file(dir, "x.bin", (size_t)(T * H) * 2);
    int32_t *ids = read_file(dir, "ids.bin", (size_t)pairs * 4);
    float *w = read_file(dir, "w.bin", (size_t)pairs * 4);
    uint16_t *wg = read_file(dir, "wg.bin", (size_t)(E * I * H) * 2);
    uint16_t *wu = read_file(dir, "wu.bin", (size_t)(E * I * H) * 2);
    uint16_t *wd = read_file(dir, "wd.bin", (size_t)(E * H * I) * 2);

    /* host contract: sizes first, then the tables and the pair maps */
    int32_t M = 0;
    int64_t Tp = 0;
    RMOE_OK_(rmoe_contract_sizes(pairs, E, &M, &Tp));
    int32_t *gs = calloc((size_t)E, 4), *go = calloc((size_t)E + 1, 4), *gpo = calloc((size_t)E + 1, 4);
    int32_t *gidx = calloc((size_t)M, 4);
    int32_t *prow = calloc((size_t)pairs + 1, 4), *cpos = calloc((size_t)pairs + 1, 4);
    if (!gs || !go || !gpo || !gidx || !prow || !cpos) FAIL("out of host memory");
    int32_t M_built = 0;
    RMOE_OK_(rmoe_build_contract(ids, T, k, E, gs, go, gpo, gidx, M, &M_built, NULL, prow, cpos));
    if (M_built != M) FAIL("rmoe_build_contract: %d blocks, rmoe_contract_sizes said %d", M_built, M);
    RMOE_OK_(rmoe_validate_contract(gs, go, gpo, gidx, E, M, Tp, pairs));
    int32_t max_rows = 0;
    for (int32_t e = 0; e < E; ++e) max_rows = gs[e] > max_rows ? gs[e] : max_rows;
    const int variant = rmoe_pick_variant(RMOE_VARIANT_AUTO, pairs, E, -1);
    if (variant < 0) FAIL("rmoe_pick_variant: %s (%d)", rmoe_status_str(variant), variant);

    /* device copies of everything the layer reads */
    void *d_x = to_device(x, (size_t)(T * H) * 2);
    void *d_w = to_device(w, (size_t)pairs * 4);
    void *d_wg = to_device(wg, (size_t)(E * I * H) * 2);
    void *d_wu = to_device(wu, (size_t)(E * I * H) * 2);
    void *d_wd = to_device(wd, (size_t)(E * H * I) * 2);
    void *d_gs = to_device(gs, (size_t)E * 4), *d_go = to_device(go, ((size_t)E + 1) * 4);
    void *d_gpo = to_device(gpo, ((size_t)E + 1) * 4), *d_gidx = to_device(gidx, (size_t)M * 4);
    void *d_prow = to_device(prow, (size_t)pairs * 4), *d_cpos = to_device(cpos, (size_t)pairs * 4);
    void *d_stacked = device_buffer((size_t)(Tp * H) * 2);
    void *d_wc = device_buffer((size_t)pairs * 4);
    void *d_hid = device_buffer(rmoe_workspace_bytes(Tp, I));
    void *d_out = device_buffer((size_t)(Tp * H) * 2);
    void *d_y = device_buffer((size_t)(T * H) * 2);

    /* the layer, asynchronous on the default stream */
    RMOE_OK_(rmoe_pack_f16(d_x, d_w, d_prow, d_cpos, T, k, H, d_stacked, d_wc, Tp, NULL));
    RMOE_OK_(rmoe_forward_f16(d_stacked, d_wg, d_wu, d_wd, d_wc, d_gs, d_go, d_gpo, d_gidx, d_hid,
                              d_out, H, I, E, Tp, pairs, M, NULL));
    RMOE_OK_(rmoe_combine_f16(d_out, d_prow, T, k, H, d_y, Tp, NULL));
    HIP_OK(hipDeviceSynchronize());

    uint16_t *y = malloc((size_t)(T * H) * 2 + 2);
    if (!y) FAIL("out of host memory");
    HIP_OK(hipMemcpy(y, d_y, (size_t)(T * H) * 2, hipMemcpyDeviceToHost));
    char path[4096];
    snprintf(path, sizeof path, "%s/y.bin", dir);
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(y, 2, (size_t)(T * H), f) != (size_t)(T * H)) FAIL("cannot write %s", path);
    fclose(f);

    void *dev[] = {d_x, d_w, d_wg, d_wu, d_wd, d_gs, d_go, d_gpo, d_gidx, d_prow, d_cpos,
                   d_stacked, d_wc, d_hid, d_out, d_y};
    for (size_t i = 0; i < sizeof dev / sizeof dev[0]; ++i) HIP_OK(hipFree(dev[i]));
    free(x), free(ids), free(w), free(wg), free(wu), free(wd), free(gs), free(go), free(gpo);
    free(gidx), free(prow), free(cpos), free(y);
    printf("ok %s: %lld pairs, %d blocks, largest group %d, family %s\n", rmoe_version(),
           (long long)pairs, M, max_rows, variant == RMOE_VARIANT_STREAM ? "stream" : "tile");
    return 0;
}
