"""GPU tests of the device-side dispatch contract (rmoe_build_contract_device).

Bar: integer tables, so bit-exact against the contract oracle (ties broken by
ascending pair index on both sides, which makes every table unique); pairs
with expert ids outside [0, E) are counted, marked -1 and left out, the other
tables equal those of the valid pairs alone; a routed layer whose contract
never leaves the GPU matches the oracle to the stated tolerance."""
import numpy as np
import pytest
import torch

import mixture_experts_routed_grouped_amd as R
import workloads
from _oracle_run import run as oracle_run
from oracle import combine as CB
from oracle import contract as C

pytestmark = pytest.mark.gpu

KEYS = ["group_sizes", "group_offsets", "group_padded_offsets", "group_idx_for_bx", "order",
        "padded_row_of_pair", "compact_pos_of_pair"]


def _device(ids, E):
    t = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()  # [T, k]
    d = R.build_contract_device(t, E)
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def _assert_same(d, oc):
    for key in KEYS:
        assert d[key].tolist() == list(oc[key]), key
    assert d["num_blocks_m"] == oc["num_blocks_m"]
    assert d["total_padded_tokens"] == oc["total_padded_tokens"]
    assert int(d["bad_ids"][0]) == 0


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "fine", "large"])
def test_device_contract_workloads(name):
    cfg = workloads.CONFIGS[name]
    ids = workloads.draw_routing(cfg)
    print(f"device contract: {name} T={cfg.tokens} k={cfg.top_k} E={cfg.experts}", flush=True)
    _assert_same(_device(ids, cfg.experts), C.build_contract(ids.tolist(), cfg.experts))


@pytest.mark.parametrize("T,k,E,seed", [
    (0, 2, 4, 1),          # no pairs: every expert empty, E blocks
    (1, 1, 1, 2),          # one expert, one pair
    (4096, 1, 1, 3),       # one expert takes everything (two chunks)
    (2047, 1, 7, 4),       # just under one 2048-pair chunk
    (2049, 1, 7, 5),       # one pair into a second chunk
    (700, 8, 256, 6),      # many experts, many of them empty
    (5000, 3, 300, 7),     # E above one workgroup of scan threads
    (3, 2, 8192, 8),       # the largest supported E
    (1024, 2, 16, 9),      # exactly one chunk: the one-launch path at its pair limit
    (1000, 2, 1024, 10),   # the one-launch path at its expert limit
    (1000, 2, 1025, 11),   # one chunk, one expert more: the multi-launch path
])
def test_device_contract_random(T, k, E, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32) \
        if T else np.zeros((0, k), np.int32)
    print(f"device contract: random T={T} k={k} E={E}", flush=True)
    _assert_same(_device(ids, E), C.build_contract(ids.tolist(), E))


@pytest.mark.parametrize("counts", [
    [0, 128, 127, 129, 256, 0, 1],   # slack blocks, empty experts, 127/128/129 rows
    [0, 0, 0, 3000],                 # everything in the last expert
    [2048, 2048],                    # chunk-aligned groups
])
def test_device_contract_counts(counts):
    ids = workloads.routing_from_counts(counts, seed=11)
    print(f"device contract: counts {counts}", flush=True)
    _assert_same(_device(ids, len(counts)), C.build_contract(ids.tolist(), len(counts)))


@pytest.mark.parametrize("T,k,E", [(64, 2, 8), (3000, 3, 40)])  # one-launch and chunked paths
def test_device_contract_reuses_out(T, k, E):
    """out=: the same tensors are filled again for new ids, with the new
    tables; a dict of another shape is refused before anything runs."""
    print(f"device contract: out= reuse T={T} k={k} E={E}", flush=True)
    rng = np.random.default_rng(31)
    first, second = (np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
                     for _ in range(2))
    d1 = R.build_contract_device(torch.from_numpy(first).cuda(), E)
    keep = {key: d1[key].data_ptr() for key in KEYS}
    d2 = R.build_contract_device(torch.from_numpy(second).cuda(), E, out=d1)
    torch.cuda.synchronize()
    assert d2 is d1 and all(d2[key].data_ptr() == keep[key] for key in KEYS)
    got = {key: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for key, v in d2.items()}
    _assert_same(got, C.build_contract(second.tolist(), E))
    with pytest.raises(ValueError):
        R.build_contract_device(torch.from_numpy(second[:-1]).cuda(), E, out=d1)


def test_device_contract_out_of_range_ids():
    """Invalid ids: counted, -1 in both pair maps, absent from the tables;
    what remains equals the contract of the valid pairs alone."""
    E, T, k = 9, 1500, 3
    rng = np.random.default_rng(21)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    flat = ids.reshape(-1)
    bad_pos = rng.choice(flat.size, size=37, replace=False)
    flat[bad_pos] = rng.choice([-1, -7, E, E + 5, 2 ** 30], size=bad_pos.size)
    print("device contract: 37 out-of-range ids", flush=True)
    d = _device(ids, E)
    valid = (flat >= 0) & (flat < E)
    assert int(d["bad_ids"][0]) == int((~valid).sum()) == 37
    assert (d["padded_row_of_pair"][~valid] == -1).all()
    assert (d["compact_pos_of_pair"][~valid] == -1).all()
    # the valid pairs alone, through the oracle, with pair ids mapped back
    vp = np.nonzero(valid)[0]
    oc = C.build_contract([[int(e)] for e in flat[vp]], E)
    for key in ["group_sizes", "group_offsets", "group_padded_offsets", "group_idx_for_bx"]:
        if key == "group_idx_for_bx":
            # the block count still covers all pairs (it is fixed before the ids are read)
            M = d["num_blocks_m"]
            assert M == -(-flat.size // 128) + E
            want = [max(e for e in range(E) if oc["group_padded_offsets"][e] <= bx * 128) for bx in range(M)]
            assert d[key].tolist() == want
        else:
            assert d[key].tolist() == list(oc[key]), key
    V = vp.size
    assert d["order"][:V].tolist() == vp[np.asarray(oc["order"])].tolist()
    assert d["padded_row_of_pair"][vp].tolist() == list(oc["padded_row_of_pair"])
    assert d["compact_pos_of_pair"][vp].tolist() == list(oc["compact_pos_of_pair"])


def test_layer_with_device_contract():
    """ids on the GPU -> device contract -> pack -> forward -> combine, with
    no host round trip, against the oracle's forward and combine."""
    cfg = workloads.Config("dc", 333, 7, 3, 256, 128, routing="zipf", zipf_s=1.2, seed=9)
    inp = workloads.make_inputs(cfg)
    print("device contract: routed layer, 333 tokens, E=7, k=3", flush=True)
    dev = torch.device("cuda")
    d = R.build_contract_device(torch.from_numpy(inp.topk_ids).to(dev), cfg.experts)
    Tp, H, I = d["total_padded_tokens"], cfg.hidden, cfg.intermediate
    x = inp.x.to(dev)
    topk_w = torch.from_numpy(np.ascontiguousarray(inp.topk_w.reshape(-1))).to(dev)
    stacked = torch.zeros((Tp, H), dtype=torch.float16, device=dev)
    w_compact = torch.zeros(d["pairs"], dtype=torch.float32, device=dev)
    R.pack(x, topk_w, d["padded_row_of_pair"], d["compact_pos_of_pair"], stacked, w_compact)
    hid = torch.zeros((Tp, I), dtype=torch.float16, device=dev)
    out = torch.zeros((Tp, H), dtype=torch.float16, device=dev)
    R.forward(stacked, inp.wg.to(dev), inp.wu.to(dev), inp.wd.to(dev), w_compact,
              d["group_sizes"], d["group_offsets"], d["group_padded_offsets"], d["group_idx_for_bx"],
              hid, out)
    y = torch.empty((cfg.tokens, H), dtype=torch.float16, device=dev)
    R.combine(out, d["padded_row_of_pair"], cfg.top_k, y)
    torch.cuda.synchronize()
    o = oracle_run(inp)
    want = CB.combine(o["out"], np.asarray(o["c"]["padded_row_of_pair"]), cfg.tokens, cfg.top_k)
    got = y.cpu().numpy().astype(np.float64)
    ref_y = want.astype(np.float64)
    err = np.abs(got - ref_y)
    assert np.isfinite(got).all()
    assert (err <= 2e-2 + 2e-2 * np.abs(ref_y)).all(), float(err.max())
