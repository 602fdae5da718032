"""GPU test of rmoe_build_contract_device_noalloc, the contract build for
callers that cannot allocate device memory: through the C-ABI it must give
the tables rmoe_build_contract_device gives with a caller workspace, bit for
bit, on two calls in a row on the same GPU -- the second on a smaller batch,
so it runs over the scratch the first one left behind."""
import numpy as np
import pytest
import torch

import mixture_experts_routed_grouped_amd as R
import workloads

pytestmark = pytest.mark.gpu

KEYS = ["group_sizes", "group_offsets", "group_padded_offsets", "group_idx_for_bx", "order",
        "padded_row_of_pair", "compact_pos_of_pair", "bad_ids"]


def _both(ids, E):
    want = R.build_contract_device(ids, E)
    got = R.build_contract_device(ids, E)            # fresh tensors of the same shapes
    for key in KEYS:
        got[key].fill_(-7)
    R.build_contract_device_noalloc(ids, E, got)
    torch.cuda.synchronize()
    assert got["num_blocks_m"] == want["num_blocks_m"]
    # entries of order past the valid pairs are left unwritten when ids are
    # out of range (documented); every other table is compared whole
    n_valid = ids.numel() - int(want["bad_ids"].item())
    for key in KEYS:
        g, w = (got[key][:n_valid], want[key][:n_valid]) if key == "order" else (got[key], want[key])
        assert torch.equal(g, w), key
    return got


def test_noalloc_contract_matches_workspace_entry_two_calls():
    big = workloads.CONFIGS["large"]                 # 131072 pairs, E=128: 64 chunks of scratch
    ids = torch.from_numpy(workloads.draw_routing(big)).cuda()
    print(f"[noalloc] call 1: {ids.numel()} pairs, E={big.experts}", flush=True)
    _both(ids, big.experts)
    small = workloads.Config("na", 5000, 64, 6, 128, 128, routing="zipf", zipf_s=1.1, seed=3)
    ids2 = workloads.draw_routing(small)
    ids2[7, 2] = 64                                   # one out-of-range id: counted, left out
    ids2 = torch.from_numpy(ids2).cuda()
    print(f"[noalloc] call 2: {ids2.numel()} pairs, E={small.experts}", flush=True)
    got = _both(ids2, small.experts)
    assert int(got["bad_ids"].item()) == 1
    # and a decode-sized batch (one-workgroup path, no scratch) right after
    ids3 = torch.from_numpy(workloads.draw_routing(workloads.CONFIGS["decode"])).cuda()
    _both(ids3, 8)
