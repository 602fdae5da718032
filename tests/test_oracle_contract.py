"""Pins for the contract oracle (oracle/contract.py) against things other
than itself: hand-worked examples from the page rules, closed forms computed
with numpy library routines, the invariants, and planted mistakes that the
invariants must catch."""
import copy
import json
import os

import numpy as np
import pytest

import workloads
from oracle import contract as C

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _load("contract_handworked.json")["cases"], ids=lambda c: c["name"])
def test_handworked_cases(case):
    ids = workloads.routing_from_counts(case["counts"], seed=3)
    c = C.build_contract(ids.tolist(), case["experts"])
    C.check_all(c)
    for key in ["group_sizes", "group_offsets", "group_padded_offsets", "num_blocks_m",
                "group_idx_for_bx"]:
        assert c[key] == case[key], key
    rows = [C.block_rows(c, bx)[2] for bx in range(c["num_blocks_m"])]
    assert rows == case["actual_rows"]


def test_tutorial_defaults():
    g = _load("contract_tutorial_defaults.json")
    cfg = workloads.CONFIGS["tiny"]
    ids = workloads.draw_routing(cfg)
    assert ids.tolist() == g["expert_of"]          # input generator regression
    c = C.build_contract(g["expert_of"], 4)
    C.check_all(c)
    for key in ["group_sizes", "group_offsets", "group_padded_offsets", "num_blocks_m",
                "group_idx_for_bx", "order"]:
        assert c[key] == g[key], key
    assert [C.block_rows(c, bx)[2] for bx in range(5)] == g["actual_rows"]


def _closed_forms(ids, E):
    """Tables from numpy library routines: bincount, cumsum, stable argsort,
    searchsorted.  Independent of the oracle's loops."""
    flat = np.asarray(ids).reshape(-1)
    counts = np.bincount(flat, minlength=E)
    go = np.concatenate([[0], np.cumsum(counts)])
    spans = (counts // 128 + 1) * 128                  # ceil((c+1)/128)*128
    gpo = np.concatenate([[0], np.cumsum(spans)])
    M = -(-flat.size // 128) + E
    gidx = np.searchsorted(gpo[:E], 128 * np.arange(M), side="right") - 1
    order = np.argsort(flat, kind="stable")
    return counts, go, gpo, M, gidx, order


@pytest.mark.parametrize("seed", range(12))
def test_closed_forms_random(seed):
    rng = np.random.default_rng(100 + seed)
    E = int(rng.integers(1, 20))
    k = int(rng.integers(1, min(E, 4) + 1))
    T = int(rng.integers(0, 700))
    routing = "zipf" if seed % 2 else "uniform"
    cfg = workloads.Config("r", T, E, k, 128, 128, routing=routing, zipf_s=1.3, seed=seed)
    ids = workloads.draw_routing(cfg)
    c = C.build_contract(ids.tolist(), E)
    C.check_all(c)
    counts, go, gpo, M, gidx, order = _closed_forms(ids, E)
    assert c["group_sizes"] == counts.tolist()
    assert c["group_offsets"] == go.tolist()
    assert c["group_padded_offsets"] == gpo.tolist()
    assert c["num_blocks_m"] == M
    assert c["group_idx_for_bx"] == gidx.tolist()
    assert c["order"] == order.tolist()
    # M blocks always hold every padded interval (E + sum floor(c/128) <= ceil(pairs/128) + E)
    assert gpo[E] <= 128 * M


def test_workload_contracts():
    """Contracts of the four big workloads satisfy the invariants and the
    closed forms (the routing draw is cheap; no tensors are built)."""
    for name in ["decode", "prefill", "fine", "large"]:
        cfg = workloads.CONFIGS[name]
        ids = workloads.draw_routing(cfg)
        assert ids.shape == (cfg.tokens, cfg.top_k)
        assert all(len(set(r)) == cfg.top_k for r in ids.tolist()[:500])
        c = C.build_contract(ids.tolist(), cfg.experts)
        C.check_all(c)
        counts, go, gpo, M, gidx, order = _closed_forms(ids, cfg.experts)
        assert c["group_padded_offsets"] == gpo.tolist()
        assert c["group_idx_for_bx"] == gidx.tolist()
        assert c["num_blocks_m"] == cfg.num_blocks_m


def test_zipf_routing_is_skewed():
    ids = workloads.draw_routing(workloads.CONFIGS["large"])
    counts = np.bincount(ids.reshape(-1), minlength=128)
    assert counts[0] == counts.max() and counts[0] > 10 * counts[-1]


# ------------------------------------------------------------ planted mistakes
def _tiny():
    return C.build_contract(_load("contract_tutorial_defaults.json")["expert_of"], 4)


def test_planted_mistakes_are_caught():
    base = _tiny()
    muts = []
    m = copy.deepcopy(base)                      # padding without the +1 slack
    m["group_padded_offsets"] = [0, 128, 256, 384, 512]
    m["group_sizes"] = [128, 4, 3, 3]
    muts.append(m)
    m = copy.deepcopy(base)                      # block mapped to the wrong expert
    m["group_idx_for_bx"] = [0, 2, 2, 3, 3]
    muts.append(m)
    m = copy.deepcopy(base)                      # offsets off by one
    m["group_offsets"] = [0, 9, 12, 15, 18]
    muts.append(m)
    m = copy.deepcopy(base)                      # order not a permutation
    m["order"] = [base["order"][1]] + base["order"][1:]
    muts.append(m)
    m = copy.deepcopy(base)                      # packing map shifted
    m["padded_row_of_pair"] = [r + 1 for r in base["padded_row_of_pair"]]
    muts.append(m)
    for mm in muts:
        with pytest.raises(AssertionError):
            C.check_all(mm)


def test_pack_rows():
    c = _tiny()
    T = 9
    rows = [f"tok{t}" for t in range(T)]
    w = [float(p) for p in range(18)]
    stacked, wc = C.pack_rows(c, rows, w, "pad")
    for p in range(18):
        assert stacked[c["padded_row_of_pair"][p]] == f"tok{p // 2}"
        assert wc[c["compact_pos_of_pair"][p]] == float(p)
    assert sum(1 for s in stacked if s != "pad") == 18
    # compact order = expert-sorted stable order of pairs
    assert wc == [float(p) for p in c["order"]]


def test_bad_expert_id_rejected():
    with pytest.raises(ValueError):
        C.build_contract([[0, 5]], 4)
