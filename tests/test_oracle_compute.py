"""Pins for the compute oracle (oracle/moe_ref.c) against things other than
itself: the float64 brute-force per-(token, expert) loop (no contract, no
padding), a dense SwiGLU MLP through numpy matmul (E=1, k=1, w=1), closed
forms, permutation equivariance, and planted mistakes the pins must catch."""
import numpy as np
import pytest
import torch

import workloads
from oracle import brute, ref
from _oracle_run import SENTINEL, per_pair, run


def ulp16(v):
    """Spacing of binary16 at |v| (2^-24 below the normal range)."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return np.exp2(e - 10)


def _assert_near_brute(res, inp, hid_ulps=1.0, out_ulps=1.0):
    """Oracle (fp32 sums, fp16 hidden) vs brute force (fp64 sums, fp16
    hidden), stage by stage.

    hidden: the only legitimate gaps are an fp16 value whose fp32 and fp64
    pre-images straddle a rounding boundary (1 ulp) and the fp32-vs-fp64 sum
    error, which is absolute (about n * 2^-24 * sum|terms|, below 2^-20 at
    these sizes) and shows only where a sum cancels to near zero.
    out: recomputed in fp64 from the oracle's OWN fp16 hidden, it may differ
    by the final fp16 rounding plus the same absolute sum error; end to end,
    the brute force's out may further differ by the hidden gaps pushed
    through |Wd| * |w| (an exact bound, computed below)."""
    c = res["c"]
    hb, yb = brute.routed_pairs(inp.x.float().numpy(), inp.topk_ids, inp.topk_w,
                                inp.wg.float().numpy(), inp.wu.float().numpy(),
                                inp.wd.float().numpy())
    T, k = inp.topk_ids.shape
    ho = per_pair(c, res["hid"]).astype(np.float64).reshape(T, k, -1)
    oo = per_pair(c, res["out"]).astype(np.float64).reshape(T, k, -1)
    dh = np.abs(ho - hb)
    assert np.all(dh <= hid_ulps * ulp16(np.maximum(np.abs(ho), np.abs(hb))) + 2.0 ** -20), dh.max()
    flips = np.count_nonzero(dh > 2.0 ** -20)
    assert flips <= max(3, hb.size // 100)       # boundary straddles are rare
    wd = inp.wd.double().numpy()
    y_own = np.zeros_like(yb)
    spread = np.zeros_like(yb)
    for t in range(T):
        for j in range(k):
            e = int(inp.topk_ids[t][j])
            w = float(inp.topk_w[t][j])
            y_own[t, j] = (wd[e] @ ho[t, j]) * w
            spread[t, j] = (np.abs(wd[e]) @ dh[t, j]) * abs(w)
    tol = out_ulps * ulp16(np.maximum(np.abs(oo), np.abs(y_own))) + 2.0 ** -20
    d_own = np.abs(oo - y_own)
    assert np.all(d_own <= tol), (d_own / tol).max()
    d_e2e = np.abs(oo - yb)
    assert np.all(d_e2e <= tol + spread), (d_e2e / (tol + spread)).max()
    return hb, yb


def test_tiny_vs_brute():
    inp = workloads.make_inputs(workloads.CONFIGS["tiny"])
    res = run(inp)
    _assert_near_brute(res, inp)


@pytest.mark.parametrize("seed,E,k,T,H,I,routing", [
    (1, 3, 2, 40, 128, 256, "uniform"),
    (2, 5, 3, 300, 256, 128, "zipf"),          # groups over 128 rows -> multi-block experts
    (3, 1, 1, 260, 128, 128, "uniform"),
    (4, 6, 1, 7, 384, 128, "uniform"),         # empty experts
])
def test_random_vs_brute(seed, E, k, T, H, I, routing):
    cfg = workloads.Config("r", T, E, k, H, I, routing=routing, zipf_s=1.5, seed=seed)
    inp = workloads.make_inputs(cfg)
    res = run(inp)
    _assert_near_brute(res, inp)


def test_padding_untouched_and_poison_contained():
    cfg = workloads.Config("r", 300, 5, 3, 128, 128, routing="zipf", zipf_s=1.5, seed=2)
    inp = workloads.make_inputs(cfg)
    res = run(inp)
    c = res["c"]
    written = np.zeros(c["total_padded_tokens"], bool)
    written[np.asarray(c["padded_row_of_pair"])] = True
    hv, ov = res["hid"].view(np.uint16), res["out"].view(np.uint16)
    assert np.all(hv[~written] == SENTINEL) and np.all(ov[~written] == SENTINEL)
    assert np.all(np.isfinite(res["out"][written].astype(np.float32)))
    assert np.all(np.isfinite(res["hid"][written].astype(np.float32)))
    # the padding rows of x really are NaN, so containment is being tested
    assert np.all(np.isnan(res["x_stacked"][~written].astype(np.float32)))


def test_dense_swiglu_special_case():
    """E=1, k=1, w=1: every row is a dense SwiGLU MLP.  Reference through
    numpy float32 matmul (BLAS summation order) with the hidden rounded to
    fp16; gaps allowed as in the brute-force pin (hidden straddles, fp32 sum
    error, final rounding)."""
    T, H, I = 200, 256, 384
    cfg = workloads.Config("d", T, 1, 1, H, I, seed=11)
    inp = workloads.make_inputs(cfg)
    inp.topk_w[:] = 1.0
    res = run(inp)
    X = inp.x.float().numpy()
    g = X @ inp.wg[0].float().numpy().T
    u = X @ inp.wu[0].float().numpy().T
    h = (g / (1 + np.exp(-g)) * u).astype(np.float16).astype(np.float64)
    ho = per_pair(res["c"], res["hid"]).astype(np.float64)
    dh = np.abs(ho - h)
    assert np.all(dh <= ulp16(np.maximum(np.abs(ho), np.abs(h))) + 2.0 ** -20)
    assert np.count_nonzero(dh > 2.0 ** -20) <= h.size // 100
    wd = inp.wd[0].float().numpy()
    y = (ho.astype(np.float32) @ wd.T).astype(np.float64)
    o = per_pair(res["c"], res["out"]).astype(np.float64)
    assert np.all(np.abs(o - y) <= ulp16(np.maximum(np.abs(o), np.abs(y))) + 2.0 ** -20)


def test_closed_forms():
    cfg = workloads.Config("z", 50, 3, 2, 128, 128, seed=5)
    base = workloads.make_inputs(cfg)
    r0 = run(base)
    o0 = r0["out"].astype(np.float32)
    # routed weights x2 -> out x2 bit for bit wherever fp16 stays normal
    inp = workloads.make_inputs(cfg)
    inp.topk_w[:] = base.topk_w * 2
    r2 = run(inp)
    c = r0["c"]
    a, b = per_pair(c, r0["out"]).astype(np.float32), per_pair(c, r2["out"]).astype(np.float32)
    normal = np.abs(a) >= 2.0 ** -13
    assert normal.mean() > 0.9
    assert np.array_equal(b[normal], 2 * a[normal])
    # x = 0 -> hidden = 0 and out = 0
    inp = workloads.make_inputs(cfg)
    inp.x.zero_()
    r = run(inp)
    assert np.all(per_pair(c, r["hid"]).astype(np.float32) == 0)
    assert np.all(per_pair(c, r["out"]).astype(np.float32) == 0)
    # Wu = 0 -> hidden = 0; Wg = 0 -> silu(0) = 0 -> hidden = 0
    for name in ["wu", "wg"]:
        inp = workloads.make_inputs(cfg)
        getattr(inp, name).zero_()
        r = run(inp)
        assert np.all(per_pair(c, r["hid"]).astype(np.float32) == 0)
        assert np.all(per_pair(c, r["out"]).astype(np.float32) == 0)
    # Wd = 0 -> out = 0 while hidden is untouched by the change
    inp = workloads.make_inputs(cfg)
    inp.wd.zero_()
    r = run(inp)
    assert np.all(per_pair(c, r["out"]).astype(np.float32) == 0)
    assert np.array_equal(per_pair(c, r["hid"]).view(np.uint16), per_pair(c, r0["hid"]).view(np.uint16))
    assert np.isfinite(o0[np.asarray(c["padded_row_of_pair"])]).all()


def test_silu_values():
    """One-row cases where gate and up are known exactly: x = e_0, Wg[:,0] = g,
    Wu[:,0] = 1 gives hidden = fp16(silu(g)), silu(g) = g / (1 + e^-g)."""
    H, I = 128, 128
    x = np.zeros(H, np.float16)
    x[0] = 1.0
    gv = np.array([0.0, 1.0, -1.0, 8.0, -8.0, 20.0, -20.0, 0.5] * 16, np.float16)
    wg = np.zeros((I, H), np.float16)
    wg[:, 0] = gv
    wu = np.zeros((I, H), np.float16)
    wu[:, 0] = 1.0
    wd = np.zeros((H, I), np.float16)
    hid, out = ref.moe_rows([x], [wg], [wu], [wd], [1.0])
    g = gv.astype(np.float64)
    want = (g / (1 + np.exp(-g))).astype(np.float16)
    assert np.array_equal(hid[0].view(np.uint16), want.view(np.uint16))
    assert hid[0][0] == 0 and np.all(out == 0)


def test_permutation_equivariance():
    """Tokens are independent: permuting token order permutes the per-pair
    outputs bit for bit (the contract and packing change, the rows do not)."""
    cfg = workloads.Config("p", 64, 4, 2, 128, 128, seed=9)
    inp = workloads.make_inputs(cfg)
    r0 = run(inp)
    perm = np.random.default_rng(1).permutation(64)
    inp2 = workloads.make_inputs(cfg, topk_ids=inp.topk_ids[perm])
    inp2.x.copy_(inp.x[torch.from_numpy(perm)])
    inp2.topk_w[:] = inp.topk_w[perm]
    r1 = run(inp2)
    a = per_pair(r0["c"], r0["out"]).view(np.uint16).reshape(64, 2, -1)
    b = per_pair(r1["c"], r1["out"]).view(np.uint16).reshape(64, 2, -1)
    assert np.array_equal(a[perm], b)


# ---------------------------------------------------------- planted mistakes
def test_planted_mistakes_fail_the_brute_pin():
    """Mistakes planted in the oracle's call (a transposed down weight, gate
    and up swapped, the routed weight of the neighbouring compact row, a
    dropped last K term) must all fail the brute-force pin."""
    cfg = workloads.Config("m", 20, 3, 2, 128, 128, seed=4)   # k=2: routed weights are not all 1
    inp = workloads.make_inputs(cfg)
    res = run(inp)
    _assert_near_brute(res, inp)
    from oracle import contract as C
    c = res["c"]

    def rerun(wg, wu, wd, wc, xs):
        Tp = c["total_padded_tokens"]
        hid = np.full((Tp, 128), SENTINEL, np.uint16).view(np.float16)
        out = np.full((Tp, 128), SENTINEL, np.uint16).view(np.float16)
        ref.moe_forward(xs, wg, wu, wd, wc, c["group_sizes"], c["group_offsets"],
                        c["group_padded_offsets"], c["group_idx_for_bx"], hid, out)
        return {"c": c, "hid": hid, "out": out}

    wg, wu, wd = inp.wg.numpy(), inp.wu.numpy(), inp.wd.numpy()
    xs, wc = res["x_stacked"], res["w_compact"]
    xs_drop = xs.copy()
    xs_drop[:, -1] = 0
    planted = [
        (wg, wu, np.ascontiguousarray(wd.transpose(0, 2, 1)), wc, xs),
        (wu, wg, wd, wc, xs),
        (wg, wu, wd, np.roll(wc, 1), xs),
        (wg, wu, wd, wc, xs_drop),
    ]
    for args in planted:
        with pytest.raises(AssertionError):
            _assert_near_brute(rerun(*args), inp)
    assert C.block_rows(c, 0)[2] > 0
