"""Test helper: the product path on the GPU, driven through the C-ABI.

Contract from the library's C++ builder, packing with the library's pack
kernel, then the forward.  The padded token rows are NaN-poisoned and the
workspace/out are filled with a sentinel bit pattern before the call, so a
test can check that padding rows are never read into valid rows nor
written.  Nothing here imports the oracle."""
from __future__ import annotations

import numpy as np
import torch

import mixture_experts_routed_grouped_amd as R

SENTINEL = 0x7E5A
PAD_NAN = 0x7E00


def _fill16(shape, bits, device):
    return torch.full(shape, bits, dtype=torch.int16, device=device).view(torch.float16)


def prepare(inp, device="cuda"):
    """Contract + device tensors for a workloads.Inputs; returns a dict."""
    cfg = inp.cfg
    E, H, I = cfg.experts, cfg.hidden, cfg.intermediate
    T, k = inp.topk_ids.shape
    c = R.build_contract(inp.topk_ids, E)
    Tp = c["total_padded_tokens"]
    d = {"c": c, "E": E, "H": H, "I": I, "T": T, "k": k, "Tp": Tp}
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
    d["gs"], d["go"], d["gpo"] = i32(c["group_sizes"]), i32(c["group_offsets"]), i32(c["group_padded_offsets"])
    d["gidx"] = i32(c["group_idx_for_bx"])
    d["prow"], d["cpos"] = i32(c["padded_row_of_pair"]), i32(c["compact_pos_of_pair"])
    x = inp.x.to(device)
    d["x"] = x
    d["wg"], d["wu"], d["wd"] = inp.wg.to(device), inp.wu.to(device), inp.wd.to(device)
    d["topk_w"] = torch.from_numpy(np.ascontiguousarray(inp.topk_w.reshape(-1))).to(device)
    d["stacked"] = _fill16((Tp, H), PAD_NAN, device)
    d["w_compact"] = torch.zeros(max(c["pairs"], 1), dtype=torch.float32, device=device)[:c["pairs"]]
    if c["pairs"]:
        R.pack(x, d["topk_w"], d["prow"], d["cpos"], d["stacked"], d["w_compact"])
    return d


def fresh_outputs(d):
    d["hid"] = _fill16((d["Tp"], d["I"]), SENTINEL, d["x"].device)
    d["out"] = _fill16((d["Tp"], d["H"]), SENTINEL, d["x"].device)
    return d


def forward(d, variant="auto"):
    fresh_outputs(d)
    R.forward(d["stacked"], d["wg"], d["wu"], d["wd"], d["w_compact"], d["gs"], d["go"], d["gpo"],
              d["gidx"], d["hid"], d["out"], variant=variant)
    torch.cuda.synchronize()
    return d


def valid_row_mask(d):
    m = torch.zeros(d["Tp"], dtype=torch.bool, device=d["x"].device)
    if d["c"]["pairs"]:
        m[d["prow"].long()] = True
    return m


def untouched(t, mask_valid):
    """True iff every row outside mask_valid still holds the sentinel."""
    bits = t.view(torch.int16)[~mask_valid]
    return bool((bits == SENTINEL).all().item())
