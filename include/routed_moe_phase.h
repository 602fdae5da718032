/*
 * routed_moe_phase.h -- diagnostic entry point of the phase-timing build of
 * the routed fused-MoE library (librmoe_phase.so, the tiled kernel source
 * compiled with RMOE_PHASE_TIMING=1; the product library librmoe.so does
 * not export it).
 *
 * What it serves: the device-side questions of "MetaX-TileLang工具链"
 * section 1.12.4 -- whether the gate/up GEMM keeps the matrix units busy and
 * whether the down GEMM is the bottleneck -- answered per phase of the tiled
 * kernels' work items instead of per launch.  In this build every persistent
 * tiled launch of the two-launch path (rmoe_gate_up_f16, rmoe_down_f16 and
 * the forwards with the tiled family; the single launch records nothing)
 * records, per workgroup, shader-clock ticks (s_memtime):
 *
 *   cycles[stage][wg][0]  prologue: item start until the first K step's
 *                         operands have landed in LDS
 *   cycles[stage][wg][1]  K loop
 *   cycles[stage][wg][2]  epilogue: until the last output store is issued
 *   cycles[stage][wg][3]  work items the workgroup ran
 *   cycles[stage][wg][4]  the workgroup's whole run, first item to last
 *
 * stage 0 = gate/up, 1 = down; wg < RMOE_PHASE_WG (workgroups beyond it are
 * not recorded).  Each launch overwrites the slots of the workgroups it ran
 * and leaves the others.  Ticks not in [0..2] of [4] are spent between items
 * (walking the item list, reading the tables).  Results are bit-identical to
 * the product library's.
 */
#ifndef ROUTED_MOE_PHASE_H
#define ROUTED_MOE_PHASE_H

#include <stddef.h>
#include <stdint.h>

#include "routed_moe.h"

#ifdef __cplusplus
extern "C" {
#endif

#define RMOE_PHASE_WG 1024

/*
 * Copy the records (uint64 [2][RMOE_PHASE_WG][5], 81920 bytes, host memory
 * owned by the caller) of the last tiled launches.  Synchronous: call after
 * the launches have completed.  Errors: RMOE_ERR_INVALID_ARGUMENT (NULL, or
 * bytes below the record size), RMOE_ERR_LAUNCH (the copy failed).
 */
RMOE_API int rmoe_phase_cycles(uint64_t *cycles, size_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* ROUTED_MOE_PHASE_H */
