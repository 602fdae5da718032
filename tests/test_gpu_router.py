"""GPU parity of the router (rmoe_router_f16) against the router oracle.

Scores: |gpu - oracle| <= 1e-6 + 1e-4 * oracle (fp32 logits of K = H terms
and the hardware exp2 against float64).  Ids are a decision taken from
floating point: where the oracle's scores around a rank are separated by
more than that tolerance the ids must be identical; inside a near-tie either
order is correct, so there the test checks that the GPU's choice is a valid
top-k (its experts' oracle scores equal the oracle's top-k scores within the
tolerance).  A routed layer driven end to end from the GPU router (router ->
device contract -> pack -> expert FFN -> combine) matches the oracle fed
with the same routing."""
import numpy as np
import pytest
import torch

import mixture_experts_routed_grouped_amd as R
import workloads
from _oracle_run import run as oracle_run
from oracle import combine as CB
from oracle import contract as C
from oracle import router as RT

pytestmark = pytest.mark.gpu

ATOL, RTOL = 1e-6, 1e-4


def _check_router(ids, vals, x16, w16, k):
    o_ids, o_vals, p = RT.route(x16, w16, k)
    T, E = p.shape
    tol = ATOL + RTOL * o_vals
    assert ids.shape == (T, k) and vals.shape == (T, k)
    assert ((ids >= 0) & (ids < E)).all()
    exact = 0
    for t in range(T):
        assert len(set(ids[t].tolist())) == k
        got_scores = p[t, ids[t]]
        assert np.all(np.abs(vals[t] - got_scores) <= ATOL + RTOL * got_scores), t
        assert np.all(np.abs(np.sort(got_scores)[::-1] - o_vals[t]) <= tol[t]), t
        s = np.sort(p[t])[::-1]
        gaps = np.abs(np.diff(s[:k + 1])) if k < E else np.abs(np.diff(s[:k]))
        if np.all(gaps > 2 * (ATOL + RTOL * s[:len(gaps)])):
            assert ids[t].tolist() == o_ids[t].tolist(), t
            exact += 1
    return exact


@pytest.mark.parametrize("T,E,k,H,seed", [
    (9, 4, 2, 256, 1),
    (64, 8, 2, 4096, 2),        # decode-shaped
    (1000, 64, 6, 2048, 3),     # fine-shaped
    (300, 128, 8, 7168, 4),     # large-shaped
    (77, 7, 3, 512, 5),         # E not a multiple of 32, ragged token tile
    (130, 256, 16, 1024, 6),    # the largest E, k = 16
    (5, 1, 1, 128, 7),          # a single expert
    (65, 32, 32, 64, 8),        # k = E, one K chunk
    (65, 33, 32, 64, 9),        # k at its maximum, E one past a tile
    (40001, 16, 2, 128, 10),    # enough tokens for 64-token workgroups (two per CU), ragged
])
def test_router_parity(T, E, k, H, seed):
    cfg = workloads.Config("rt", T, E, k, H, 128, seed=seed)
    x = workloads._normal_f16((T, H), 1.0, seed, 1, "cpu")
    w = workloads.make_router_weight(cfg)
    print(f"router: T={T} E={E} k={k} H={H}", flush=True)
    ids, vals = R.router(x.cuda(), w.cuda(), k)
    torch.cuda.synchronize()
    exact = _check_router(ids.cpu().numpy(), vals.cpu().numpy(), x.numpy(), w.numpy(), k)
    assert exact >= 0.5 * T  # the exact-id path is exercised: near-ties are a minority


def test_router_ties_take_lower_index():
    """A zero gate makes every score 1/E: ids must be 0..k-1 in order."""
    T, E, k, H = 70, 12, 5, 128
    x = workloads._normal_f16((T, H), 1.0, 3, 1, "cuda")
    w = torch.zeros((E, H), dtype=torch.float16, device="cuda")
    print("router: zero gate", flush=True)
    ids, vals = R.router(x, w, k)
    torch.cuda.synchronize()
    assert (ids.cpu().numpy() == np.arange(k)[None, :]).all()
    assert np.allclose(vals.cpu().numpy(), 1.0 / E, rtol=1e-6, atol=0)


def test_layer_from_gpu_router():
    """Router -> device contract -> pack -> forward -> combine on the GPU,
    against the oracle forward and combine fed with the GPU's routing."""
    cfg = workloads.Config("rl", 200, 16, 4, 256, 128, seed=12)
    x = workloads._normal_f16((cfg.tokens, cfg.hidden), 1.0, cfg.seed, 1, "cpu")
    wr = workloads.make_router_weight(cfg)
    print("router: routed layer 200 tokens, E=16, k=4", flush=True)
    dev = torch.device("cuda")
    ids, vals = R.router(x.to(dev), wr.to(dev), cfg.top_k)
    d = R.build_contract_device(ids, cfg.experts)
    inp = workloads.make_inputs(cfg, topk_ids=ids.cpu().numpy())
    inp.topk_w = vals.cpu().numpy()
    inp.x = x
    Tp, H, I = d["total_padded_tokens"], cfg.hidden, cfg.intermediate
    stacked = torch.zeros((Tp, H), dtype=torch.float16, device=dev)
    w_compact = torch.zeros(d["pairs"], dtype=torch.float32, device=dev)
    R.pack(x.to(dev), vals.reshape(-1), d["padded_row_of_pair"], d["compact_pos_of_pair"], stacked,
           w_compact)
    hid = torch.zeros((Tp, I), dtype=torch.float16, device=dev)
    out = torch.zeros((Tp, H), dtype=torch.float16, device=dev)
    R.forward(stacked, inp.wg.to(dev), inp.wu.to(dev), inp.wd.to(dev), w_compact, d["group_sizes"],
              d["group_offsets"], d["group_padded_offsets"], d["group_idx_for_bx"], hid, out)
    y = torch.empty((cfg.tokens, H), dtype=torch.float16, device=dev)
    R.combine(out, d["padded_row_of_pair"], cfg.top_k, y)
    torch.cuda.synchronize()
    o = oracle_run(inp)
    want = CB.combine(o["out"], np.asarray(o["c"]["padded_row_of_pair"]), cfg.tokens, cfg.top_k)
    got = y.cpu().numpy().astype(np.float64)
    ref_y = want.astype(np.float64)
    assert np.isfinite(got).all()
    assert (np.abs(got - ref_y) <= 2e-2 + 2e-2 * np.abs(ref_y)).all()


def test_layer_sweep():
    """16 seeded random layers (1-256 experts, top-k up to 8, 1-600 tokens,
    H 128-512, I 128-256): the GPU router's top-k is a valid top-k of the
    router oracle, the device contract built from it equals the contract
    oracle's tables bit for bit, and router -> device contract -> pack ->
    forward -> combine matches the oracle layer fed with the same routing."""
    rng = np.random.default_rng(77)
    dev = torch.device("cuda")
    for i in range(16):
        E = int(rng.integers(1, 257))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.integers(1, 601))
        H = 128 * int(rng.integers(1, 5))
        I = 128 * int(rng.integers(1, 3))
        cfg = workloads.Config(f"ls{i}", T, E, k, H, I, seed=200 + i)
        print(f"router: layer sweep {i}: T={T} E={E} k={k} H={H} I={I}", flush=True)
        x = workloads._normal_f16((T, H), 1.0, cfg.seed, 1, "cpu")
        wr = workloads.make_router_weight(cfg)
        ids, vals = R.router(x.to(dev), wr.to(dev), k)
        d = R.build_contract_device(ids, E)
        torch.cuda.synchronize()
        ids_h = ids.cpu().numpy()
        _check_router(ids_h, vals.cpu().numpy(), x.numpy(), wr.numpy(), k)
        oc = C.build_contract(ids_h.tolist(), E)
        for key in ["group_sizes", "group_offsets", "group_padded_offsets", "group_idx_for_bx",
                    "padded_row_of_pair", "compact_pos_of_pair"]:
            assert d[key].cpu().numpy().tolist() == list(oc[key]), key
        inp = workloads.make_inputs(cfg, topk_ids=ids_h)
        inp.topk_w = vals.cpu().numpy()
        inp.x = x
        Tp = d["total_padded_tokens"]
        stacked = torch.zeros((Tp, H), dtype=torch.float16, device=dev)
        w_compact = torch.zeros(max(d["pairs"], 1), dtype=torch.float32, device=dev)
        R.pack(x.to(dev), vals.reshape(-1), d["padded_row_of_pair"], d["compact_pos_of_pair"],
               stacked, w_compact)
        hid = torch.zeros((Tp, I), dtype=torch.float16, device=dev)
        out = torch.zeros((Tp, H), dtype=torch.float16, device=dev)
        R.forward(stacked, inp.wg.to(dev), inp.wu.to(dev), inp.wd.to(dev), w_compact[:d["pairs"]],
                  d["group_sizes"], d["group_offsets"], d["group_padded_offsets"],
                  d["group_idx_for_bx"], hid, out)
        y = torch.empty((T, H), dtype=torch.float16, device=dev)
        R.combine(out, d["padded_row_of_pair"], k, y)
        torch.cuda.synchronize()
        o = oracle_run(inp)
        want = CB.combine(o["out"], np.asarray(o["c"]["padded_row_of_pair"]), T, k).astype(np.float64)
        got = y.cpu().numpy().astype(np.float64)
        assert np.isfinite(got).all()
        assert (np.abs(got - want) <= 2e-2 + 2e-2 * np.abs(want)).all(), f"layer sweep {i}"
