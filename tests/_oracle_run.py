"""Test helper: run the oracle end to end on a workload's inputs.

Builds the contract with oracle/contract.py, packs the padded token matrix
(padding rows filled with an fp16 NaN) and the compact routed weights, and
runs the C oracle with hid/out pre-filled with a sentinel bit pattern, so a
test can see which rows were written."""
from __future__ import annotations

import numpy as np

from oracle import contract as C
from oracle import ref

SENTINEL = 0x7E5A          # an fp16 quiet-NaN bit pattern no computation produces
PAD_NAN = 0x7E00


def pack(c, x16: np.ndarray, topk_w: np.ndarray):
    """numpy packing from the oracle's pair maps."""
    H = x16.shape[1]
    Tp = c["total_padded_tokens"]
    xs = np.full((Tp, H), PAD_NAN, np.uint16)
    if c["pairs"]:
        prow = np.asarray(c["padded_row_of_pair"])
        tok = np.asarray(c["flat_token"])
        xs[prow] = x16.view(np.uint16)[tok]
    wc = np.zeros(c["pairs"], np.float32)
    if c["pairs"]:
        wc[np.asarray(c["compact_pos_of_pair"])] = np.asarray(topk_w, np.float32).reshape(-1)
    return xs.view(np.float16), wc


def run(inp, n_threads=None):
    """Oracle forward on a workloads.Inputs whose tensors are on the CPU."""
    c = C.build_contract(inp.topk_ids.tolist(), inp.cfg.experts)
    x16 = inp.x.cpu().numpy()
    xs, wc = pack(c, x16, inp.topk_w)
    Tp = c["total_padded_tokens"]
    H, I = inp.cfg.hidden, inp.cfg.intermediate
    hid = np.full((Tp, I), SENTINEL, np.uint16).view(np.float16)
    out = np.full((Tp, H), SENTINEL, np.uint16).view(np.float16)
    n = ref.moe_forward(xs, inp.wg.cpu().numpy(), inp.wu.cpu().numpy(), inp.wd.cpu().numpy(), wc,
                        c["group_sizes"], c["group_offsets"], c["group_padded_offsets"],
                        c["group_idx_for_bx"], hid, out, n_threads=n_threads)
    assert n == c["pairs"]
    return {"c": c, "x_stacked": xs, "w_compact": wc, "hid": hid, "out": out}


def per_pair(c, arr):
    """Rows of a padded [Tp, *] array in pair order p = t*k + j."""
    if c["pairs"] == 0:
        return arr[:0]
    return arr[np.asarray(c["padded_row_of_pair"])]
