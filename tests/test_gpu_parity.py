"""GPU parity: the HIP path (through the C-ABI) against the oracle.

Bar (the target's stated tolerance): every valid element of out satisfies
|gpu - oracle| <= 2e-2 + 2e-2 |oracle|; the contract tables match bit for
bit; padding rows of out and of the workspace are never written.  Tighter
diagnostics ride along: the fp16 hidden workspace within 2 fp16 ulps plus an
absolute 3e-5, with at most 1% of entries more than 1 ulp apart, and the
relative RMS error of out below 2e-3 (a dropped K tile would show as ~1e-1).

Why the absolute term: gate and up are fp32 sums of K = H products whose
magnitudes add up to ~40 at the workload sizes, so either side's summation
order leaves an absolute error of order 2^-24 * sqrt(K) * 40 ~ 1e-6..1e-5.
Where gate or up nearly cancels, the fp16 hidden is tiny and that absolute
error spans many of its ulps.  Measured against float64 on the decode
workload, the MFMA path was the closer of the two (worst 5.5 ulps vs 18.4
ulps for the oracle's sequential fp32 sum, mean 0.25 ulp for both)."""
import numpy as np
import pytest
import torch

import mixture_experts_routed_grouped_amd as R
import workloads
from _gpu_run import forward, fresh_outputs, prepare, untouched, valid_row_mask
from _oracle_run import run as oracle_run
from oracle import contract as C
from oracle import combine as CB
from oracle import ref

pytestmark = pytest.mark.gpu

ATOL = RTOL = 2e-2


def ulp16(v):
    a = np.abs(np.asarray(v, np.float64))
    return np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -14))) - 10)


def _assert_parity(gpu_hid, gpu_out, o_hid, o_out, what, ulp1_frac=0.01):
    gh, go_ = gpu_hid.astype(np.float64), gpu_out.astype(np.float64)
    oh, oo = o_hid.astype(np.float64), o_out.astype(np.float64)
    assert np.isfinite(gh).all() and np.isfinite(go_).all(), f"{what}: non-finite output"
    d = np.abs(go_ - oo)
    bad = d > ATOL + RTOL * np.abs(oo)
    assert not bad.any(), f"{what}: {bad.sum()} out elements beyond tolerance, max {d.max()}"
    dh = np.abs(gh - oh)
    u = ulp16(np.maximum(np.abs(gh), np.abs(oh)))
    over = dh > 2 * u + 3e-5
    assert not over.any(), f"{what}: {over.sum()} hidden entries beyond 2 ulps + 3e-5, max {dh.max()}"
    assert np.count_nonzero(dh > u) <= ulp1_frac * dh.size, f"{what}: too many hidden entries > 1 ulp"
    rel = np.sqrt((d ** 2).sum() / max((oo ** 2).sum(), 1e-30))
    assert rel < 2e-3, f"{what}: relative RMS error {rel}"
    return rel


def _full_compare(inp, variant):
    """Small inputs: the whole padded output against the oracle's."""
    orc = oracle_run(inp)
    d = forward(prepare(inp), variant)
    c = d["c"]
    for key in ["group_sizes", "group_offsets", "group_padded_offsets", "group_idx_for_bx",
                "padded_row_of_pair", "compact_pos_of_pair"]:
        assert np.asarray(c[key]).tolist() == list(orc["c"][key]), key
    mask = valid_row_mask(d)
    assert untouched(d["hid"], mask) and untouched(d["out"], mask), "padding rows written"
    if c["pairs"] == 0:
        return None
    rows = d["prow"].long()
    gh = d["hid"][rows].cpu().numpy()
    go_ = d["out"][rows].cpu().numpy()
    prow = np.asarray(orc["c"]["padded_row_of_pair"])
    return _assert_parity(gh, go_, orc["hid"][prow], orc["out"][prow], f"{inp.cfg.name}/{variant}")


VARIANTS = ["stream", "tile"]


@pytest.mark.parametrize("variant", VARIANTS)
def test_tiny(variant):
    _full_compare(workloads.make_inputs(workloads.CONFIGS["tiny"]), variant)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("seed,E,k,T,H,I,routing", [
    (1, 5, 2, 300, 256, 384, "zipf"),      # multi-block groups, ragged tails, H % 256 == 0
    (2, 3, 3, 200, 384, 256, "uniform"),   # H % 256 == 128: half-width last down slice
    (3, 8, 2, 37, 512, 128, "uniform"),    # tiny groups, empty-ish experts
    (4, 2, 1, 520, 128, 640, "uniform"),   # four full blocks per expert, long I
    (5, 40, 4, 3000, 512, 1024, "zipf"),   # more tiles than workgroup slots: each loops
    (6, 12, 2, 2000, 256, 2304, "uniform"),  # 18 gate/up slices: groups of 8, 8, 2
    (7, 256, 8, 64, 256, 256, "uniform"),  # many experts, about 2 rows each, some empty
    (8, 512, 2, 1500, 256, 384, "zipf"),   # mostly empty experts, a few multi-block ones
])
def test_random_shapes(variant, seed, E, k, T, H, I, routing):
    cfg = workloads.Config(f"r{seed}", T, E, k, H, I, routing=routing, zipf_s=1.4, seed=seed)
    _full_compare(workloads.make_inputs(cfg), variant)


def _sweep_configs(n=48, seed=2024):
    """Seeded random batches for the sweep: expert counts 1-64, top-k up to
    8, 1-400 tokens, H and I multiples of 128 up to 512, uniform or Zipf
    routing (so group sizes land on every streaming pass plan and on lone,
    full and multi-block tiled entries)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.integers(1, 65))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.integers(1, 401))
        H = 128 * int(rng.integers(1, 5))
        I = 128 * int(rng.integers(1, 5))
        routing = "zipf" if rng.random() < 0.5 and E > 1 else "uniform"
        out.append((100 + i, E, k, T, H, I, routing))
    return out


def test_random_shape_sweep():
    """48 seeded random batches, each through both kernel families, AUTO and
    the single-launch forward (both hand-overs), the whole padded output
    against one oracle run: tables bit for bit, padding rows untouched, every
    valid element within tolerance."""
    for seed, E, k, T, H, I, routing in _sweep_configs():
        cfg = workloads.Config(f"s{seed}", T, E, k, H, I, routing=routing, zipf_s=1.3, seed=seed)
        inp = workloads.make_inputs(cfg)
        print(f"[sweep] seed={seed} E={E} k={k} T={T} H={H} I={I} {routing}", flush=True)
        orc = oracle_run(inp)
        prow = np.asarray(orc["c"]["padded_row_of_pair"])
        for variant in ("stream", "tile", "auto", "local", "global"):
            d = prepare(inp)
            if variant in ("local", "global"):
                fresh_outputs(d)
                sync = R.fused_sync(d["stacked"].device, d["gidx"].numel())
                R.forward_fused(d["stacked"], d["wg"], d["wu"], d["wd"], d["w_compact"], d["gs"],
                                d["go"], d["gpo"], d["gidx"], d["hid"], d["out"], sync=sync,
                                handover=variant)
                torch.cuda.synchronize()
                assert R.fused_sync_errors(sync) == 0, "a down tile's wait timed out"
            else:
                forward(d, variant)
            for key in ["group_sizes", "group_offsets", "group_padded_offsets", "group_idx_for_bx",
                        "padded_row_of_pair"]:
                assert np.asarray(d["c"][key]).tolist() == list(orc["c"][key]), key
            mask = valid_row_mask(d)
            assert untouched(d["hid"], mask) and untouched(d["out"], mask), "padding rows written"
            rows = d["prow"].long()
            _assert_parity(d["hid"][rows].cpu().numpy(), d["out"][rows].cpu().numpy(),
                           orc["hid"][prow], orc["out"][prow], f"sweep {seed}/{variant}")


@pytest.mark.parametrize("H,I", [(1 << 20, 128), (128, 1 << 20)])
def test_maximum_hidden_and_intermediate(H, I):
    """The largest H and I the entries accept (2^20 each): 64-bit row offsets,
    K sweeps of 16384 chunks, 4096 or 8192 weight slices, the narrow last
    down slice; both families, AUTO and the single launch, whole against the
    oracle (two experts, three routed rows).  The stated bar (out within
    2e-2 + 2e-2|oracle|) and the hidden bar of 2 ulps + 3e-5 hold as
    everywhere; the share of hidden entries more than 1 ulp apart, a
    diagnostic of the two sides' fp32 summation orders, grows with sqrt(K):
    1% at the workloads' K (up to 14336) scales to about 9% at K = 2^20,
    so it is bounded by 10% here."""
    cfg = workloads.Config("maxdim", 3, 2, 1, H, I, seed=41)
    inp = workloads.make_inputs(cfg, topk_ids=np.array([[0], [1], [1]], np.int32))
    print(f"[max-dim] H={H} I={I}", flush=True)
    orc = oracle_run(inp)
    prow = np.asarray(orc["c"]["padded_row_of_pair"])
    d = prepare(inp)
    for variant in ("stream", "tile", "auto", "global"):
        if variant == "global":
            fresh_outputs(d)
            sync = R.fused_sync(d["stacked"].device, d["gidx"].numel())
            R.forward_fused(d["stacked"], d["wg"], d["wu"], d["wd"], d["w_compact"], d["gs"], d["go"],
                            d["gpo"], d["gidx"], d["hid"], d["out"], sync=sync, handover="global")
            torch.cuda.synchronize()
            assert R.fused_sync_errors(sync) == 0
        else:
            forward(d, variant)
        mask = valid_row_mask(d)
        assert untouched(d["hid"], mask) and untouched(d["out"], mask), "padding rows written"
        rows = d["prow"].long()
        _assert_parity(d["hid"][rows].cpu().numpy(), d["out"][rows].cpu().numpy(), orc["hid"][prow],
                       orc["out"][prow], f"max-dim H={H} I={I} {variant}", ulp1_frac=0.10)


@pytest.mark.parametrize("variant", VARIANTS)
def test_edge_group_sizes(variant):
    """Empty experts, groups of 1, 127, 128, 129 and 256 rows (the +1 slack
    block of a full group must stay unwritten)."""
    counts = [0, 127, 128, 129, 256, 0, 1, 3]
    ids = workloads.routing_from_counts(counts, seed=5)
    cfg = workloads.Config("edge", ids.shape[0], len(counts), 1, 256, 256, seed=5)
    _full_compare(workloads.make_inputs(cfg, topk_ids=ids), variant)


@pytest.mark.parametrize("variant", VARIANTS)
def test_single_expert_and_no_pairs(variant):
    cfg = workloads.Config("e1", 300, 1, 1, 128, 128, seed=6)
    _full_compare(workloads.make_inputs(cfg), variant)
    ids = np.zeros((0, 2), np.int32)
    cfg = workloads.Config("empty", 0, 4, 2, 128, 128, seed=6)
    _full_compare(workloads.make_inputs(cfg, topk_ids=ids), variant)


def test_stream_pass_widths():
    """Every pass plan of the streaming kernels, one block per expert: 1-32
    rows (one 32-token pass moving 1-4 groups of 8 rows), 33-64 (one
    64-token pass, 5-6 or 7-8 groups), 65-96 (one 96-token pass, 9-10 or
    11-12 groups) and 97-128 (a 96-token pass, then a 32-token one with 1-32
    rows), each on the edges of its row groups; then a uniform k=2 batch of
    about 85 rows per expert.  Compared with the oracle whole."""
    sizes = [1, 9, 17, 25, 32, 33, 48, 49, 64, 65, 80, 81, 96, 97, 105, 113, 121, 128]
    ids = np.concatenate([np.full(n, e, np.int32) for e, n in enumerate(sizes)])[:, None]
    ids = np.random.default_rng(3).permutation(ids)
    cfg = workloads.Config("passes", len(ids), len(sizes), 1, 256, 256, seed=15)
    _full_compare(workloads.make_inputs(cfg, topk_ids=ids), "stream")
    cfg = workloads.Config("passes_u", 170, 4, 2, 512, 384, routing="uniform", seed=16)
    _full_compare(workloads.make_inputs(cfg), "stream")


@pytest.mark.parametrize("T,E,k,routing", [(128, 8, 2, "uniform"), (96, 6, 2, "uniform"),
                                           (192, 8, 2, "uniform"), (176, 8, 2, "zipf")])
def test_auto_mid_batch(T, E, k, routing):
    """25-32 routed rows per expert on average, and up to 48 with at most 8
    experts: the automatic choice streams with 64-token passes (two MFMA
    token tiles per pass; groups above 64 rows take a second pass)."""
    cfg = workloads.Config(f"mid{T}", T, E, k, 512, 1024, routing=routing, zipf_s=1.2, seed=12)
    inp = workloads.make_inputs(cfg)
    assert R.pick_variant(T * k, E) == "stream"
    _full_compare(inp, "auto")


def test_determinism():
    cfg = workloads.Config("det", 400, 6, 2, 256, 256, routing="zipf", zipf_s=1.3, seed=8)
    inp = workloads.make_inputs(cfg)
    d = prepare(inp)
    outs = {}
    for v in ["stream", "tile", "tile"]:
        forward(d, v)
        outs.setdefault(v, []).append(d["out"].clone())
    assert torch.equal(outs["tile"][0].view(torch.int16), outs["tile"][1].view(torch.int16))


def test_run_kernel_signature():
    """The submission-style entry with its cached workspace."""
    inp = workloads.make_inputs(workloads.CONFIGS["tiny"])
    d = prepare(inp)
    out = torch.zeros((d["Tp"], d["H"]), dtype=torch.float16, device="cuda")
    R.run_kernel(d["stacked"], d["wg"], d["wu"], d["wd"], d["w_compact"], d["gs"], d["go"],
                 d["gpo"], d["gidx"], out)
    torch.cuda.synchronize()
    ref_d = forward(d, "auto")
    rows = d["prow"].long()
    assert torch.equal(out[rows].view(torch.int16), ref_d["out"][rows].view(torch.int16))


def test_pack_and_combine():
    cfg = workloads.Config("pc", 333, 7, 3, 256, 128, routing="zipf", zipf_s=1.2, seed=9)
    inp = workloads.make_inputs(cfg)
    d = forward(prepare(inp), "auto")
    c = d["c"]
    oc = C.build_contract(inp.topk_ids.tolist(), cfg.experts)
    xs, wc = C.pack_rows(oc, list(inp.x.numpy()), list(inp.topk_w.reshape(-1)), None)
    prow = np.asarray(oc["padded_row_of_pair"])
    stacked = d["stacked"].cpu().numpy()
    for p in range(0, c["pairs"], 7):
        assert np.array_equal(stacked[prow[p]].view(np.uint16), xs[prow[p]].view(np.uint16))
    assert np.array_equal(d["w_compact"].cpu().numpy(), np.asarray(wc, np.float32))
    y = torch.empty((333, 256), dtype=torch.float16, device="cuda")
    R.combine(d["out"], d["prow"], 3, y)
    torch.cuda.synchronize()
    want = CB.combine(d["out"].cpu().numpy(), prow, 333, 3)
    assert np.array_equal(y.cpu().numpy().view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("T,k,E,H", [
    (100, 12, 16, 64),     # top_k above the lanes per token row (8 chunks): weights in two passes
    (300, 1, 3, 8),        # one chunk per row: 256 tokens per workgroup, a ragged last pass
    (77, 4, 9, 16384),     # 2048 chunks per row: two chunk batches per thread
    (150, 8, 20, 7168),    # the large workload's row length (896 chunks, a partial last batch)
])
def test_pack_and_combine_row_shapes(T, k, E, H):
    """Pack at every row shape of the token-major kernel: each packed row,
    every routed weight and the untouched padding rows against the oracle's
    pack; combine of a random routed output against the oracle's combine,
    all bit for bit."""
    from _gpu_run import SENTINEL
    rng = np.random.default_rng(T * 7 + k)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    x = torch.from_numpy(rng.standard_normal((T, H)).astype(np.float16))
    tw = rng.random(T * k).astype(np.float32)
    oc = C.build_contract(ids.tolist(), E)
    xs, wc = C.pack_rows(oc, list(x.numpy()), list(tw), np.zeros(H, np.float16))
    prow = np.asarray(oc["padded_row_of_pair"])
    Tp, pairs = oc["total_padded_tokens"], oc["pairs"]
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    stacked = torch.full((Tp, H), SENTINEL, dtype=torch.int16, device="cuda").view(torch.float16)
    w_compact = torch.zeros(pairs, dtype=torch.float32, device="cuda")
    print(f"[pack] T={T} k={k} E={E} H={H}: {pairs} pairs into {Tp} rows", flush=True)
    R.pack(x.cuda(), torch.from_numpy(tw).cuda(), i32(prow), i32(oc["compact_pos_of_pair"]), stacked,
           w_compact)
    out = torch.from_numpy(rng.standard_normal((Tp, H)).astype(np.float16)).cuda()
    y = torch.empty((T, H), dtype=torch.float16, device="cuda")
    R.combine(out, i32(prow), k, y)
    torch.cuda.synchronize()
    got = stacked.cpu().numpy().view(np.uint16)
    valid = np.zeros(Tp, dtype=bool)
    valid[prow] = True
    assert np.array_equal(got[valid], np.asarray(xs)[valid].view(np.uint16))
    assert (got[~valid] == np.uint16(SENTINEL)).all()
    assert np.array_equal(w_compact.cpu().numpy(), np.asarray(wc, np.float32))
    want = CB.combine(out.cpu().numpy(), prow, T, k)
    assert np.array_equal(y.cpu().numpy().view(np.uint16), want.view(np.uint16))


# ------------------------------------------------------------ full size
def _block_sample(c, seed=0):
    """Pairs to hold against the oracle at full size: one row of every block
    that holds valid rows (found through the kernel-side addressing:
    group_idx_for_bx, padded and compact offsets), the first row of each
    expert's first block and the last row of its last block, else a seeded
    random row of the block."""
    gs = np.asarray(c["group_sizes"])
    go = np.asarray(c["group_offsets"])
    gpo = np.asarray(c["group_padded_offsets"])
    gidx = np.asarray(c["group_idx_for_bx"])
    order = np.asarray(c["order"])
    rng = np.random.default_rng(seed)
    pairs, blocks = [], 0
    for bx in range(c["num_blocks_m"]):
        e = int(gidx[bx])
        off = bx * 128 - int(gpo[e])
        rows = max(0, min(128, int(gs[e]) - off))
        if rows == 0:
            continue
        blocks += 1
        if off == 0:
            r = 0
        elif off + rows == gs[e]:
            r = rows - 1
        else:
            r = int(rng.integers(0, rows))
        pairs.append(int(order[go[e] + off + r]))
    return pairs, blocks


def _oracle_rows(inp, pairs, group_rows=32):
    """Oracle rows for the given pairs, experts taken a few at a time so that
    at most a handful of experts' weights are copied to the host at once."""
    k = inp.topk_ids.shape[1]
    by_e = {}
    for i, p in enumerate(pairs):
        by_e.setdefault(int(inp.topk_ids[p // k][p % k]), []).append(i)
    x_host = inp.x.cpu().numpy()
    I, H = inp.wg.shape[1], inp.wg.shape[2]
    o_hid = np.zeros((len(pairs), I), np.float16)
    o_out = np.zeros((len(pairs), H), np.float16)
    experts = sorted(by_e)
    j = 0
    while j < len(experts):
        group, n = [], 0
        while j < len(experts) and (n < group_rows or not group) and len(group) < 8:
            group.append(experts[j])
            n += len(by_e[experts[j]])
            j += 1
        host = {e: (inp.wg[e].cpu().numpy(), inp.wu[e].cpu().numpy(), inp.wd[e].cpu().numpy())
                for e in group}
        idx = [i for e in group for i in by_e[e]]
        xs, gl, ul, dl, ws = [], [], [], [], []
        for i in idx:
            t, jj = divmod(pairs[i], k)
            e = int(inp.topk_ids[t][jj])
            xs.append(x_host[t])
            gl.append(host[e][0])
            ul.append(host[e][1])
            dl.append(host[e][2])
            ws.append(float(inp.topk_w[t][jj]))
        h, o = ref.moe_rows(xs, gl, ul, dl, ws)
        o_hid[idx] = h
        o_out[idx] = o
        del host
    return o_hid, o_out


def _all_valid_rows_written(d):
    """Every valid row of the workspace and of out was overwritten (the
    sentinel is a NaN pattern) and holds finite values: checked on the GPU
    over the whole buffers ("MetaX-TileLang工具链" 2.10: NaN/Inf in the
    output, and a substitute check where the full golden is too costly)."""
    rows = d["prow"].long()
    for name in ("hid", "out"):
        ok = torch.isfinite(d[name][rows]).all(dim=1)
        assert bool(ok.all()), f"{name}: {int((~ok).sum())} valid rows unwritten or non-finite"


@pytest.mark.parametrize("name", ["decode", "prefill", "fine", "large"])
def test_full_size(name):
    """The workloads at full size, in the launch configuration the benchmark
    times (variant auto): tables bit for bit; padding rows untouched and
    every valid row written and finite, over the whole buffers; against the
    oracle, every routed row of decode and one row of every live block of
    the others (plus each expert's first and last row); a second run
    bit-identical."""
    cfg = workloads.CONFIGS[name]
    print(f"[full-size] {name}: generating inputs", flush=True)
    inp = workloads.make_inputs(cfg, device="cuda")
    d = prepare(inp)
    oc = C.build_contract(inp.topk_ids.tolist(), cfg.experts)
    for key in ["group_sizes", "group_offsets", "group_padded_offsets", "group_idx_for_bx",
                "padded_row_of_pair"]:
        assert np.asarray(d["c"][key]).tolist() == list(oc[key]), key
    print(f"[full-size] {name}: forward ({R.pick_variant(d['c']['pairs'], cfg.experts)})", flush=True)
    forward(d, "auto")
    mask = valid_row_mask(d)
    assert untouched(d["hid"], mask) and untouched(d["out"], mask), "padding rows written"
    _all_valid_rows_written(d)
    out1 = d["out"].clone()
    forward(d, "auto")
    assert torch.equal(out1.view(torch.int16), d["out"].view(torch.int16)), "not deterministic"
    del out1
    if name == "decode":
        pairs, blocks = list(range(d["c"]["pairs"])), None
    else:
        pairs, blocks = _block_sample(d["c"])
    print(f"[full-size] {name}: oracle on {len(pairs)} rows "
          f"({'all routed rows' if blocks is None else f'{blocks} live blocks'})", flush=True)
    o_hid, o_out = _oracle_rows(inp, pairs)
    rows = d["prow"][torch.tensor(pairs, device="cuda")].long()
    rel = _assert_parity(d["hid"][rows].cpu().numpy(), d["out"][rows].cpu().numpy(), o_hid, o_out,
                         name)
    print(f"[full-size] {name}: {len(pairs)} rows within tolerance, rel RMS {rel:.2e}", flush=True)


@pytest.mark.parametrize("name,cfg", [
    ("large-shape Zipf, 384 tokens", workloads.Config("zipf_e128", 384, 128, 8, 7168, 2048,
                                                      routing="zipf", zipf_s=1.2, seed=21)),
    ("fine-shape Zipf, 384 tokens", workloads.Config("zipf_e64", 384, 64, 6, 2048, 1408,
                                                     routing="zipf", zipf_s=1.1, seed=22)),
])
def test_stream_skewed_mid_batch(name, cfg):
    """Streaming on the workloads' shapes under skew, where AUTO streams with
    the largest group known although that group spans several blocks (one
    96-token pass then a 32-token one per full block): padding rows
    untouched, every valid row written and finite, one row of every live
    block (plus each expert's first and last row) against the oracle."""
    inp = workloads.make_inputs(cfg, device="cuda")
    d = prepare(inp)
    gs = np.asarray(d["c"]["group_sizes"])
    assert gs.max() > 256                                    # a group of three or more blocks
    assert R.pick_variant(d["c"]["pairs"], cfg.experts, max_group_rows=int(gs.max())) == "stream"
    print(f"[stream-skew] {name}: forward, largest group {int(gs.max())}", flush=True)
    forward(d, "stream")
    mask = valid_row_mask(d)
    assert untouched(d["hid"], mask) and untouched(d["out"], mask), "padding rows written"
    _all_valid_rows_written(d)
    pairs, blocks = _block_sample(d["c"], seed=5)
    print(f"[stream-skew] {name}: oracle on {len(pairs)} rows ({blocks} live blocks)", flush=True)
    o_hid, o_out = _oracle_rows(inp, pairs)
    rows = d["prow"][torch.tensor(pairs, device="cuda")].long()
    rel = _assert_parity(d["hid"][rows].cpu().numpy(), d["out"][rows].cpu().numpy(), o_hid, o_out,
                         name)
    print(f"[stream-skew] {name}: {len(pairs)} rows within tolerance, rel RMS {rel:.2e}", flush=True)


@pytest.mark.parametrize("E", [8192, 65000])
def test_many_experts(E):
    """Many experts, nearly all of them empty (600 routed rows, top-2): every
    empty expert still owns one slack block, so num_blocks_m is about E;
    both families, AUTO and the single launch, whole against the oracle."""
    cfg = workloads.Config(f"manyE{E}", 300, E, 2, 128, 128, seed=47)
    inp = workloads.make_inputs(cfg, device="cuda")
    inp.x, inp.wg, inp.wu, inp.wd = (t.cpu() for t in (inp.x, inp.wg, inp.wu, inp.wd))
    print(f"[many-experts] E={E}", flush=True)
    orc = oracle_run(inp)
    prow = np.asarray(orc["c"]["padded_row_of_pair"])
    d = prepare(inp)
    for variant in ("stream", "tile", "auto", "global"):
        if variant == "global":
            fresh_outputs(d)
            sync = R.fused_sync(d["stacked"].device, d["gidx"].numel())
            R.forward_fused(d["stacked"], d["wg"], d["wu"], d["wd"], d["w_compact"], d["gs"], d["go"],
                            d["gpo"], d["gidx"], d["hid"], d["out"], sync=sync, handover="global")
            torch.cuda.synchronize()
            assert R.fused_sync_errors(sync) == 0
        else:
            forward(d, variant)
        for key in ["group_sizes", "group_offsets", "group_padded_offsets", "group_idx_for_bx"]:
            assert np.asarray(d["c"][key]).tolist() == list(orc["c"][key]), key
        mask = valid_row_mask(d)
        assert untouched(d["hid"], mask) and untouched(d["out"], mask), "padding rows written"
        rows = d["prow"].long()
        _assert_parity(d["hid"][rows].cpu().numpy(), d["out"][rows].cpu().numpy(), orc["hid"][prow],
                       orc["out"][prow], f"E={E} {variant}")


def test_maximum_blocks():
    """The largest block table the entries accept (num_blocks_m = 65535, the
    streaming grid's y limit): two experts share 8388224 tokens (k = 1,
    H = I = 128).  Both families and AUTO: padding rows untouched and every
    valid row written and finite over the whole buffers, one row of every
    live block (plus each expert's first and last row) against the oracle."""
    T = 65533 * 128
    ids = workloads.routing_from_counts([T // 2, T - T // 2], seed=43)
    cfg = workloads.Config("maxblocks", T, 2, 1, 128, 128, seed=43)
    inp = workloads.make_inputs(cfg, topk_ids=ids)
    print(f"[max-blocks] T={T}", flush=True)
    d = prepare(inp)
    assert d["c"]["num_blocks_m"] == 65535
    pairs, blocks = _block_sample(d["c"], seed=9)
    o_hid, o_out = _oracle_rows(inp, pairs)
    mask = valid_row_mask(d)
    sel = d["prow"][torch.tensor(pairs, device="cuda")].long()
    for variant in ("stream", "tile", "auto"):
        forward(d, variant)
        assert untouched(d["hid"], mask) and untouched(d["out"], mask), "padding rows written"
        _all_valid_rows_written(d)
        _assert_parity(d["hid"][sel].cpu().numpy(), d["out"][sel].cpu().numpy(), o_hid, o_out,
                       f"max-blocks {variant}")
    print(f"[max-blocks] {len(pairs)} rows of {blocks} live blocks within tolerance", flush=True)


def test_pack_large_batch_nontemporal_path():
    """The large workload packs 1.9 GB of rows, above the size where pack
    stores them non-temporally: sampled rows equal their token's row bit for
    bit at the oracle contract's padded position, every routed weight lands
    at its compact position, and padding rows stay untouched."""
    from _gpu_run import SENTINEL
    cfg = workloads.CONFIGS["large"]
    inp = workloads.make_inputs(cfg, device="cuda")
    oc = C.build_contract(inp.topk_ids.tolist(), cfg.experts)
    prow = np.asarray(oc["padded_row_of_pair"])
    cpos = np.asarray(oc["compact_pos_of_pair"])
    Tp, H, k = oc["total_padded_tokens"], cfg.hidden, cfg.top_k
    assert oc["pairs"] * H * 2 > 512 << 20
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    stacked = torch.full((Tp, H), SENTINEL, dtype=torch.int16, device="cuda").view(torch.float16)
    wc = torch.zeros(oc["pairs"], dtype=torch.float32, device="cuda")
    topk_w = torch.from_numpy(np.ascontiguousarray(inp.topk_w.reshape(-1))).cuda()
    print("[pack] large workload, 131072 pairs", flush=True)
    R.pack(inp.x, topk_w, i32(prow), i32(cpos), stacked, wc)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    sample = np.concatenate([[0, oc["pairs"] - 1], rng.integers(0, oc["pairs"], size=3000)])
    got = stacked[torch.from_numpy(prow[sample]).long().cuda()].view(torch.int16)
    want = inp.x[torch.from_numpy(sample // k).long().cuda()].view(torch.int16)
    assert torch.equal(got, want)
    wc_host = wc.cpu().numpy()
    assert np.array_equal(wc_host[cpos], inp.topk_w.reshape(-1).astype(np.float32))
    valid = torch.zeros(Tp, dtype=torch.bool, device="cuda")
    valid[torch.from_numpy(prow).long().cuda()] = True
    assert bool((stacked.view(torch.int16)[~valid] == SENTINEL).all())
