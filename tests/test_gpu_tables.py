"""GPU tests of how the kernels use the contract tables.

* Both kernel families (and the single launch) compute a block only when
  group_idx_for_bx maps it to the expert whose padded interval holds it
  (the row predicate of "Fused MoE GEMM 提交说明", 完整算子代码, applied to the
  block -> expert table of "moe_dispatch_contract.py", build_contract step 4).
  With one entry of that table corrupted, every family leaves exactly the
  corrupted block's rows unwritten, writes every other valid row bit for bit
  as on the valid table, and rmoe_validate_contract_device counts the
  violation; on valid tables it counts none.
* The two stage entry points choose the same kernel family as the forward
  for one batch (rmoe_pick_variant), so gate/up then down under AUTO equals
  the forward of the family the library names, bit for bit.
"""
import numpy as np
import pytest
import torch

import mixture_experts_routed_grouped_amd as R
import workloads
from _gpu_run import SENTINEL, fresh_outputs, prepare, valid_row_mask

pytestmark = pytest.mark.gpu


def _run(d, family, gidx):
    fresh_outputs(d)
    args = (d["stacked"], d["wg"], d["wu"], d["wd"], d["w_compact"], d["gs"], d["go"], d["gpo"],
            gidx, d["hid"], d["out"])
    if family == "fused":
        sync = torch.zeros(R.fused_sync_words(gidx.numel()), dtype=torch.int32, device="cuda")
        R.forward_fused(*args, sync=sync)
        assert R.fused_sync_errors(sync) == 0
    else:
        R.forward(*args, variant=family)
    torch.cuda.synchronize()
    return d["hid"].clone(), d["out"].clone()


def _violations(d, gidx):
    v = R.validate_contract_device(d["gs"], d["go"], d["gpo"], gidx, d["Tp"], d["c"]["pairs"])
    torch.cuda.synchronize()
    return int(v.item())


@pytest.fixture(scope="module")
def batch():
    # multi-block experts, an empty one, a count on a block multiple (slack block)
    counts = [300, 0, 129, 500, 40, 256]
    ids = workloads.routing_from_counts(counts, seed=21)
    cfg = workloads.Config("tables", ids.shape[0], len(counts), 1, 256, 384, seed=21)
    return prepare(workloads.make_inputs(cfg, topk_ids=ids))


def _corruptions(d):
    gpo = d["c"]["group_padded_offsets"]
    E = d["E"]
    b0 = gpo[0] // 128 + 1          # second block of expert 0 (live)
    b3 = gpo[3] // 128              # first block of expert 3 (live)
    b3l = gpo[3] // 128 + 3         # fourth block of expert 3: its last live block
    return [(b0, 2), (b3, 0), (b3l, -1), (b0, E), (b3l, 4)]


@pytest.mark.parametrize("family", ["stream", "tile", "fused"])
def test_corrupted_block_table(batch, family):
    d = batch
    assert _violations(d, d["gidx"]) == 0
    want_hid, want_out = _run(d, family, d["gidx"])
    valid = valid_row_mask(d)
    for bx, e_bad in _corruptions(d):
        gidx = d["gidx"].clone()
        gidx[bx] = e_bad
        print(f"[tables] {family}: block {bx} -> expert {e_bad}", flush=True)
        assert _violations(d, gidx) == 1
        hid, out = _run(d, family, gidx)
        blk = torch.zeros_like(valid)
        blk[bx * 128:(bx + 1) * 128] = True
        for got, want in ((hid, want_hid), (out, want_out)):
            bits, wbits = got.view(torch.int16), want.view(torch.int16)
            assert bool((bits[blk] == SENTINEL).all()), "a corrupted block was written"
            keep = valid & ~blk
            assert torch.equal(bits[keep], wbits[keep]), "other rows changed"
            assert bool((bits[~valid] == SENTINEL).all()), "padding rows written"


def test_validator_on_workload_tables():
    """Valid tables of every workload: no violation; a group size, an offset
    and a padded offset changed one at a time: violations counted."""
    for name, cfg in workloads.CONFIGS.items():
        c = R.build_contract(workloads.draw_routing(cfg), cfg.experts)
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
        t = [i32(c[k]) for k in ("group_sizes", "group_offsets", "group_padded_offsets",
                                 "group_idx_for_bx")]
        v = R.validate_contract_device(*t, c["total_padded_tokens"], c["pairs"])
        torch.cuda.synchronize()
        assert int(v.item()) == 0, name
        for which, idx, delta in ((0, 0, 1), (1, 1, -1), (2, cfg.experts, 128)):
            bad = [x.clone() for x in t]
            bad[which][idx] += delta
            v = R.validate_contract_device(*bad, c["total_padded_tokens"], c["pairs"])
            torch.cuda.synchronize()
            assert int(v.item()) > 0, (name, which)


@pytest.mark.parametrize("T,E", [(75, 5), (128, 8), (192, 8), (193, 8), (144, 9), (145, 9), (600, 8)])
def test_stage_entries_agree_with_forward(T, E):
    """gate_up then down, each under AUTO, equal the forward with the family
    rmoe_pick_variant names, bit for bit (E=5 with 150 pairs is the batch on
    which an estimate from the block count alone picked differently)."""
    cfg = workloads.Config(f"agree{T}", T, E, 2, 256, 512, routing="uniform", seed=31)
    d = prepare(workloads.make_inputs(cfg))
    pairs = d["c"]["pairs"]
    fam = R.pick_variant(pairs, E)
    print(f"[agree] T={T} E={E} pairs={pairs}: {fam}", flush=True)
    fresh_outputs(d)
    R.gate_up(d["stacked"], d["wg"], d["wu"], d["gs"], d["gpo"], d["gidx"], d["hid"], pairs)
    R.down(d["hid"], d["wd"], d["w_compact"], d["gs"], d["go"], d["gpo"], d["gidx"], d["out"])
    torch.cuda.synchronize()
    got_hid, got_out = d["hid"].clone(), d["out"].clone()
    want_hid, want_out = _run(d, fam, d["gidx"])
    assert torch.equal(got_hid.view(torch.int16), want_hid.view(torch.int16))
    assert torch.equal(got_out.view(torch.int16), want_out.view(torch.int16))
