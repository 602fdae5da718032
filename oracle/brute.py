"""Brute-force per-(token, expert) reference in float64 numpy.

TEST INFRASTRUCTURE ONLY, for tiny inputs.  It uses no contract table, no
sorting, no padding and no code from ``contract`` or ``moe_ref.c``: each
routed pair (t, j) with expert e = topk_ids[t][j] is pushed through that
expert's FFN on its own, straight from the computation semantics in
"Fused MoE GEMM 提交说明", section 算子来源:

    gate = x_t Wg[e]^T,  up = x_t Wu[e]^T,  hidden = silu(gate) * up,
    y[t, j] = (hidden Wd[e]^T) * w[t, j]

Sums are float64.  ``round_hidden=True`` rounds the hidden vector to fp16
(numpy's IEEE conversion), as the kernel's fp16 workspace does; the output
is returned in float64 so a caller can compare at any precision.
"""
from __future__ import annotations

import numpy as np


def silu64(v):
    return v / (1.0 + np.exp(-v))


def routed_pairs(x, topk_ids, topk_w, wg, wu, wd, round_hidden=True):
    """Returns (hidden [T, k, I], y [T, k, H]) in float64."""
    x = np.asarray(x, dtype=np.float64)
    wg = np.asarray(wg, dtype=np.float64)
    wu = np.asarray(wu, dtype=np.float64)
    wd = np.asarray(wd, dtype=np.float64)
    T, k = np.asarray(topk_ids).shape
    I, H = wg.shape[1], wg.shape[2]
    hid = np.zeros((T, k, I))
    y = np.zeros((T, k, H))
    for t in range(T):
        for j in range(k):
            e = int(topk_ids[t][j])
            gate = wg[e] @ x[t]          # [I]
            up = wu[e] @ x[t]            # [I]
            h = silu64(gate) * up
            if round_hidden:
                h = h.astype(np.float16).astype(np.float64)
            hid[t, j] = h
            y[t, j] = (wd[e] @ h) * float(topk_w[t][j])
    return hid, y
