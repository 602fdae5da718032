"""Benchmark of the routed fused-MoE expert FFN on one MI355X.

One step = one forward of the routed kernel (gate/up into the fp16 hidden
workspace, then down with the routed-weight scale) over one batch of
synthetic, already packed, HBM-resident inputs with prebuilt tables -- the
"routed_kernel_only" timing scope of the benchmark write-up
("MetaX-TileLang工具链", section 1.12.2).  Contract building, packing and
allocation are outside the timed region.

Prints ONE JSON line.  The headline workload is the large one (16384 tokens,
E=128, top_k=8, Zipf 1.2, H=7168, I=2048: the largest that fits one GPU);
value = useful TFLOP/s = 6*pairs*H*I / step time.  roofline: the dominant
kernel (gate/up) against HBM (decode-shaped) or dense fp16 MFMA
(prefill-shaped) peak, its launch duration measured with HIP events
recorded on the stream the kernels run on.  cpu_baseline: the oracle timed
on the host cores on a bounded sample of rows of the same workload.  The
other workloads (decode, prefill, fine) are timed in the same run under
"other_workloads".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
PEAK_F16_TFLOPS = 2500.0     # MI355X dense fp16 MFMA, TFLOP/s
METRIC = "fused MoE TFLOP/s (useful 6·pairs·H·I) + % MFMA/HBM roofline, 1×MI355X"
# sources that define a variant's kernels: a traffic record is valid only for
# the exact sources it was measured on
KERNEL_SOURCES = {"stream": ["rmoe_stream.hip", "rmoe_device.h"],
                  "tile": ["rmoe_tile.hip", "rmoe_device.h", "rmoe_sched.h"]}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="large",
                    help="tiny | decode | prefill | fine | large (default: large, the largest "
                         "workload that fits one GPU)")
    ap.add_argument("--also", default="decode,prefill,fine",
                    help="comma-separated workloads also timed in the same run (extra keys)")
    ap.add_argument("--also-steps", type=int, default=30)
    ap.add_argument("--no-aux", action="store_true",
                    help="skip the timings of the steps around the routed kernels")
    ap.add_argument("--variant", default="auto", choices=["auto", "stream", "tile"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target wall time of the oracle sample")
    ap.add_argument("--crossover", action="store_true",
                    help="only sweep the streaming/tiled forward times across batch sizes under "
                         "Zipf routing")
    ap.add_argument("--dense-compare", action="store_true",
                    help="only time the tiled stages on one expert (a dense SwiGLU FFN) beside "
                         "torch's fp16 matmul on the same GEMM shapes")
    ap.add_argument("--phase-timing", default="",
                    help="only report where the tiled stages' time goes, per phase of their work "
                         "items, for these comma-separated workloads (dense = one expert, 8192 "
                         "tokens, H=4096, I=14336), with the phase-timing diagnostic library")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (x steps), the "
                         "reference that scales rocprofv3 FETCH_SIZE/WRITE_SIZE to bytes")
    return ap.parse_args()


def calibrate_copy(mib: int, steps: int):
    """A plain copy kernel of known size for counter calibration: each launch
    reads and writes exactly mib MiB."""
    import torch
    n = mib * (1 << 20) // 2
    a = torch.ones(n, dtype=torch.float16, device="cuda")
    b = torch.empty_like(a)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read_per_launch": n * 2,
                      "bytes_written_per_launch": n * 2, "launches": steps}), flush=True)


def kernel_src_hash(variant: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[variant]:
        with open(os.path.join(ROOT, "mixture_experts_routed_grouped_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stats_ms(xs):
    s = sorted(xs)
    q = lambda f: s[min(len(s) - 1, int(round(f * (len(s) - 1))))]
    return {"mean": statistics.fmean(s), "median": q(0.5), "p90": q(0.9), "p99": q(0.99),
            "min": s[0], "std": statistics.pstdev(s)}


def algorithmic(cfg, c, variant):
    """Algorithmic bytes and useful flops per launch of each kernel.

    gate/up: both weight matrices of every expert that has rows, the valid
    token rows, the hidden rows written.  down: the down weights of every
    active expert, the hidden rows read, the out rows written, the routed
    weights.  Padding rows and empty experts move nothing."""
    import numpy as np
    H, I = cfg.hidden, cfg.intermediate
    pairs = c["pairs"]
    e_act = int(np.count_nonzero(np.asarray(c["group_sizes"])))
    gu_bytes = 2 * e_act * I * H * 2 + pairs * H * 2 + pairs * I * 2
    dn_bytes = e_act * H * I * 2 + pairs * I * 2 + pairs * H * 2 + pairs * 4
    return {"gate_up": {"bytes": gu_bytes, "flops": 4.0 * pairs * H * I},
            "down": {"bytes": dn_bytes, "flops": 2.0 * pairs * H * I},
            "experts_active": e_act}


def aux_timings(cfg, inp, hid, out, variant, reps=20):
    """Average time per call of the steps around the routed kernels (outside
    the headline scope): the router (synthetic gate [E, H]), the device-side
    contract build from device top-k ids, the pack, the combine, and the
    whole layer -- router, device contract, pack, both expert kernels,
    combine -- with no host round trip; for the tiled family also the
    single-launch forward, in both hand-overs (hidden rows kept in one XCD's
    L2, or handed across XCDs through memory), beside the two-launch one."""
    import torch
    import mixture_experts_routed_grouped_amd as R
    import workloads
    dev = inp.x.device
    ids = torch.from_numpy(inp.topk_ids).to(dev)
    topk_w = torch.from_numpy(inp.topk_w.reshape(-1).copy()).to(dev)
    wr = workloads.make_router_weight(cfg, device=dev)
    d = R.build_contract_device(ids, cfg.experts)
    stacked = torch.empty((d["total_padded_tokens"], cfg.hidden), dtype=torch.float16, device=dev)
    w_compact = torch.empty(d["pairs"], dtype=torch.float32, device=dev)
    y = torch.empty((cfg.tokens, cfg.hidden), dtype=torch.float16, device=dev)
    r_ids = torch.empty((cfg.tokens, cfg.top_k), dtype=torch.int32, device=dev)
    r_w = torch.empty((cfg.tokens, cfg.top_k), dtype=torch.float32, device=dev)

    c_buf = R.build_contract_device(r_ids, cfg.experts)  # reused: the layer allocates nothing

    def layer():
        R.router(inp.x, wr, cfg.top_k, r_ids, r_w)
        c = R.build_contract_device(r_ids, cfg.experts, out=c_buf)
        R.pack(inp.x, r_w.reshape(-1), c["padded_row_of_pair"], c["compact_pos_of_pair"], stacked,
               w_compact)
        R.gate_up(stacked, inp.wg, inp.wu, c["group_sizes"], c["group_padded_offsets"],
                  c["group_idx_for_bx"], hid, c["pairs"], variant=variant)
        R.down(hid, inp.wd, w_compact, c["group_sizes"], c["group_offsets"],
               c["group_padded_offsets"], c["group_idx_for_bx"], out, variant=variant)
        R.combine(out, c["padded_row_of_pair"], cfg.top_k, y)

    steps = {
        "router": lambda: R.router(inp.x, wr, cfg.top_k, r_ids, r_w),
        "contract_device": lambda: R.build_contract_device(ids, cfg.experts, out=c_buf),
        "pack": lambda: R.pack(inp.x, topk_w, d["padded_row_of_pair"], d["compact_pos_of_pair"],
                               stacked, w_compact),
        "combine": lambda: R.combine(out, d["padded_row_of_pair"], cfg.top_k, y),
        "layer_e2e": layer,
    }
    if variant == "tile":
        # both tiled stages in one launch, against the two launches, on the
        # same device tables (tiled family only: prefill-shaped batches)
        sync = R.fused_sync(dev, d["num_blocks_m"])
        tables = (d["group_sizes"], d["group_offsets"], d["group_padded_offsets"], d["group_idx_for_bx"])
        steps["forward_two_launch"] = lambda: R.forward(stacked, inp.wg, inp.wu, inp.wd, w_compact,
                                                        *tables, hid, out, variant="tile")
        for ho in ("local", "global"):
            steps[f"forward_fused_{ho}"] = (
                lambda ho=ho: R.forward_fused(stacked, inp.wg, inp.wu, inp.wd, w_compact, *tables,
                                              hid, out, sync=sync, handover=ho))
    res = {}
    for name, fn in steps.items():
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) * 1e3 / reps
    return res


def traffic_for(kernel: str, workload: str, variant: str):
    """Measured HBM bytes per launch from a committed rocprofv3 counter
    summary, only if it was taken on this variant and its kernel sources
    have not changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("variant") != variant or rec.get("kernel_src_sha") != kernel_src_hash(variant):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, inp, c, target_s):
    """Time the oracle (as it stands) on a bounded sample of rows of the same
    workload, on every host core OpenMP gets; scale to TFLOP/s of useful
    work.  The sample takes routed rows in expert-sorted order from at most
    four experts spread over the routing (so at most four experts' weights
    are copied to the host), as many as fit about target_s of oracle time."""
    import numpy as np
    from oracle import ref
    nt = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    k = cfg.top_k
    ids = inp.topk_ids
    gs, go = np.asarray(c["group_sizes"]), np.asarray(c["group_offsets"])
    order = np.asarray(c["order"])
    live = [int(e) for e in np.nonzero(gs)[0]]
    experts = sorted({live[int(i)] for i in np.linspace(0, len(live) - 1, min(4, len(live)))})
    # round robin over the chosen experts, each in its compact order
    cand, r = [], 0
    while len(cand) < ids.size and any(r < gs[e] for e in experts):
        cand += [int(order[go[e] + r]) for e in experts if r < gs[e]]
        r += 1
    x_host = inp.x.cpu().numpy()
    host = {e: (inp.wg[e].cpu().numpy(), inp.wu[e].cpu().numpy(), inp.wd[e].cpu().numpy())
            for e in experts}

    def rows_for(sel):
        xs, gl, ul, dl, ws = [], [], [], [], []
        for p in sel:
            t, j = divmod(int(p), k)
            e = int(ids[t][j])
            xs.append(x_host[t])
            gl.append(host[e][0])
            ul.append(host[e][1])
            dl.append(host[e][2])
            ws.append(float(inp.topk_w[t][j]))
        return xs, gl, ul, dl, ws

    # calibrate with one row per thread, then size the sample to ~target_s
    args = rows_for(cand[:nt])
    t0 = time.perf_counter()
    ref.moe_rows(*args, n_threads=nt)
    t_cal = time.perf_counter() - t0
    n_rounds = max(1, int(target_s / max(t_cal, 1e-6)))
    n_rows = min(len(cand), nt * n_rounds)
    args = rows_for(cand[:n_rows])
    t0 = time.perf_counter()
    ref.moe_rows(*args, n_threads=nt)
    dt = time.perf_counter() - t0
    flops = 6.0 * n_rows * cfg.hidden * cfg.intermediate
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": nt, "kind": "oracle",
            "sample": f"{n_rows} of {ids.size} routed rows, taken in turn from experts "
                      f"{experts} in expert-sorted order, full H and I; {dt:.2f} s wall"}


def measure(cfg, variant, steps, warmup, with_aux=False):
    """Inputs of one workload resident on the GPU, prebuilt tables, then
    `warmup` untimed and `steps` timed forwards (gate/up and down launches,
    HIP events recorded around each on the stream they run on)."""
    import numpy as np
    import torch

    import mixture_experts_routed_grouped_amd as R
    import workloads

    dev = torch.device("cuda:0")
    inp = workloads.make_inputs(cfg, device=dev)
    c = R.build_contract(inp.topk_ids, cfg.experts)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    gs, go, gpo, gidx = (i32(c[k]) for k in ["group_sizes", "group_offsets",
                                             "group_padded_offsets", "group_idx_for_bx"])
    prow, cpos = i32(c["padded_row_of_pair"]), i32(c["compact_pos_of_pair"])
    Tp, H, I, E = c["total_padded_tokens"], cfg.hidden, cfg.intermediate, cfg.experts
    stacked = torch.zeros((Tp, H), dtype=torch.float16, device=dev)
    w_compact = torch.zeros(c["pairs"], dtype=torch.float32, device=dev)
    topk_w = torch.from_numpy(inp.topk_w.reshape(-1).copy()).to(dev)
    R.pack(inp.x, topk_w, prow, cpos, stacked, w_compact)
    hid = torch.empty((Tp, I), dtype=torch.float16, device=dev)
    out = torch.empty((Tp, H), dtype=torch.float16, device=dev)
    # the family for this batch: the library's choice, asked through the C-ABI
    # with the largest group from the host tables
    resolved = R.pick_variant(c["pairs"], E, variant, max_group_rows=int(max(c["group_sizes"])))

    def step(evs=None):
        if evs is not None:
            evs[0].record()
        R.gate_up(stacked, inp.wg, inp.wu, gs, gpo, gidx, hid, c["pairs"], variant=resolved)
        if evs is not None:
            evs[1].record()
        R.down(hid, inp.wd, w_compact, gs, go, gpo, gidx, out, variant=resolved)
        if evs is not None:
            evs[2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gu_ms = [e[0].elapsed_time(e[1]) for e in evs]
    dn_ms = [e[1].elapsed_time(e[2]) for e in evs]
    step_ms = [e[0].elapsed_time(e[2]) for e in evs]
    ms_per_step = wall * 1e3 / steps
    alg = algorithmic(cfg, c, resolved)
    value = cfg.useful_flops() / (ms_per_step * 1e-3) / 1e12
    gu_s = statistics.fmean(gu_ms) * 1e-3
    dn_s = statistics.fmean(dn_ms) * 1e-3
    hbm_bound = resolved == "stream"
    if hbm_bound:
        ach = alg["gate_up"]["bytes"] / gu_s / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": ach / PEAK_HBM_GBS}
    else:
        ach = alg["gate_up"]["flops"] / gu_s / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / PEAK_F16_TFLOPS}
    roof["kernel"] = "gate_up: " + ("stream_kernel<true,...> (LDS-DMA weight streaming)" if hbm_bound
                                    else "tile_kernel<true> (256x256 LDS-tiled MFMA)")
    roof["traffic"] = traffic_for("gate_up", cfg.name, resolved)
    total_bytes = alg["gate_up"]["bytes"] + alg["down"]["bytes"]
    res = {
        "value": value, "ms_per_step": ms_per_step,
        "config": {"workload": f"{cfg.name}: {cfg.tokens} tokens, E={E}, top_k={cfg.top_k}, "
                               f"H={H}, I={I}, {cfg.routing} routing"
                               + (f" s={cfg.zipf_s}" if cfg.routing == "zipf" else "")
                               + f", seed {cfg.seed}",
                   "tokens": cfg.tokens, "experts": E, "top_k": cfg.top_k, "hidden": H,
                   "intermediate": I, "pairs": c["pairs"], "num_blocks_m": c["num_blocks_m"],
                   "experts_active": alg["experts_active"], "scope": "routed_kernel_only",
                   "variant": resolved},
        "roofline": roof,
        "step_hbm_gbs": total_bytes / (ms_per_step * 1e-3) / 1e9,
        "step_hbm_frac": total_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "step_mfma_frac": value / PEAK_F16_TFLOPS,
        "kernels": {
            "gate_up": {"avg_us": gu_s * 1e6, "alg_bytes": alg["gate_up"]["bytes"],
                        "gbs": alg["gate_up"]["bytes"] / gu_s / 1e9,
                        "tflops": alg["gate_up"]["flops"] / gu_s / 1e12},
            "down": {"avg_us": dn_s * 1e6, "alg_bytes": alg["down"]["bytes"],
                     "gbs": alg["down"]["bytes"] / dn_s / 1e9,
                     "tflops": alg["down"]["flops"] / dn_s / 1e12},
        },
        "latency_ms": stats_ms(step_ms),
    }
    if with_aux:
        res["aux_kernels_us"] = aux_timings(cfg, inp, hid, out, resolved)
    return res, inp, c


# token counts of the crossover sweep, per (E, top_k, H, I, Zipf s or None
# for uniform routing): decode-to-mid batch sizes on the shapes of the
# workloads and on few-expert shapes, each on both sides of the family
# thresholds (16-112 rows per expert)
CROSSOVER = {
    "E128_k8_H7168_I2048_zipf1.2": (128, 8, 7168, 2048, 1.2, [16, 64, 128, 256, 384, 512, 640]),
    "E128_k8_H7168_I2048_uniform": (128, 8, 7168, 2048, None, [256, 384, 512, 640]),
    "E64_k6_H2048_I1408_zipf1.1": (64, 6, 2048, 1408, 1.1, [32, 128, 256, 384, 512, 768]),
    "E64_k6_H2048_I1408_uniform": (64, 6, 2048, 1408, None, [256, 320, 384, 448, 512]),
    "E32_k4_H4096_I2048_zipf1.2": (32, 4, 4096, 2048, 1.2, [256, 384, 512, 768]),
    "E32_k4_H4096_I2048_uniform": (32, 4, 4096, 2048, None, [256, 320, 384, 448, 512]),
    "E16_k2_H4096_I14336_zipf1.2": (16, 2, 4096, 14336, 1.2, [192, 256, 320, 384]),
    "E16_k2_H4096_I14336_uniform": (16, 2, 4096, 14336, None, [256, 320, 384, 448, 512]),
    "E8_k2_H4096_I14336_zipf1.2": (8, 2, 4096, 14336, 1.2, [64, 128, 192, 224, 256, 288]),
    "E8_k2_H4096_I14336_uniform": (8, 2, 4096, 14336, None, [64, 128, 192, 224, 256, 288, 320, 352, 384]),
    "E8_k2_H6144_I16384_uniform": (8, 2, 6144, 16384, None, [192, 224, 256, 288, 320]),
    "E8_k2_H2048_I5632_uniform": (8, 2, 2048, 5632, None, [192, 256, 320, 384, 448]),
    "E4_k2_H4096_I14336_uniform": (4, 2, 4096, 14336, None, [96, 128, 160, 192, 224]),
}


def crossover_sweep(reps=20):
    """Forward time of both kernel families across batch sizes under uniform
    and Zipf routing (one JSON line per batch), with the family the library
    picks from the average alone and from the average and the largest group."""
    import numpy as np
    import torch

    import mixture_experts_routed_grouped_amd as R
    import workloads
    dev = torch.device("cuda:0")
    for name, (E, k, H, I, zs, Ts) in CROSSOVER.items():
        routing = "zipf" if zs else "uniform"
        base = workloads.make_inputs(workloads.Config("sweep", max(Ts), E, k, H, I, routing=routing,
                                                      zipf_s=zs or 0.0), device=dev)
        for T in Ts:
            ids = workloads.draw_routing(workloads.Config("sweep", T, E, k, H, I, routing=routing,
                                                          zipf_s=zs or 0.0))
            c = R.build_contract(ids, E)
            i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
            tabs = [i32(c[q]) for q in ("group_sizes", "group_offsets", "group_padded_offsets",
                                        "group_idx_for_bx")]
            Tp = c["total_padded_tokens"]
            stacked = torch.zeros((Tp, H), dtype=torch.float16, device=dev)
            wc = torch.zeros(c["pairs"], dtype=torch.float32, device=dev)
            tw = torch.from_numpy(workloads.draw_routed_weights(T, k, 7).reshape(-1).copy()).to(dev)
            R.pack(base.x[:T].contiguous(), tw, i32(c["padded_row_of_pair"]),
                   i32(c["compact_pos_of_pair"]), stacked, wc)
            hid = torch.empty((Tp, I), dtype=torch.float16, device=dev)
            out = torch.empty((Tp, H), dtype=torch.float16, device=dev)
            res = {}
            for v in ("stream", "tile"):
                fn = lambda: R.forward(stacked, base.wg, base.wu, base.wd, wc, *tabs, hid, out, variant=v)
                for _ in range(3):
                    fn()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    fn()
                e1.record()
                torch.cuda.synchronize()
                res[v + "_us"] = round(e0.elapsed_time(e1) / reps * 1e3, 1)
            gmax = int(max(c["group_sizes"]))
            print(json.dumps({"sweep": name, "tokens": T, "pairs": c["pairs"],
                              "avg_rows": round(c["pairs"] / E, 1), "max_rows": gmax,
                              "auto_avg": R.pick_variant(c["pairs"], E),
                              "auto_max": R.pick_variant(c["pairs"], E, max_group_rows=gmax),
                              **res}), flush=True)
        del base
        torch.cuda.empty_cache()


def dense_compare(reps=20):
    """The tiled stages on the dense special case of the method -- one expert,
    8192 tokens, H=4096, I=14336 (a plain SwiGLU FFN; gate/up is then an
    8192 x 28672 x 4096 GEMM, down 8192 x 4096 x 14336) -- beside torch's
    fp16 matmul (the vendor BLAS) on the same shapes, same box, same run: how
    far the tiled kernels are from the best dense GEMM the chip runs."""
    import numpy as np
    import torch

    import mixture_experts_routed_grouped_amd as R
    import workloads
    dev = torch.device("cuda:0")
    T, H, I = 8192, 4096, 14336
    cfg = workloads.Config("dense", T, 1, 1, H, I)
    inp = workloads.make_inputs(cfg, device=dev, topk_ids=np.zeros((T, 1), np.int32))
    c = R.build_contract(inp.topk_ids, 1)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    gs, go, gpo, gidx = (i32(c[q]) for q in ("group_sizes", "group_offsets", "group_padded_offsets",
                                             "group_idx_for_bx"))
    Tp = c["total_padded_tokens"]
    stacked = torch.zeros((Tp, H), dtype=torch.float16, device=dev)
    wc = torch.zeros(T, dtype=torch.float32, device=dev)
    R.pack(inp.x, torch.ones(T, dtype=torch.float32, device=dev), i32(c["padded_row_of_pair"]),
           i32(c["compact_pos_of_pair"]), stacked, wc)
    hid = torch.empty((Tp, I), dtype=torch.float16, device=dev)
    out = torch.empty((Tp, H), dtype=torch.float16, device=dev)

    def tm(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    gu = tm(lambda: R.gate_up(stacked, inp.wg, inp.wu, gs, gpo, gidx, hid, T, variant="tile"))
    dn = tm(lambda: R.down(hid, inp.wd, wc, gs, go, gpo, gidx, out, variant="tile"))
    x, wgu = inp.x.contiguous(), torch.cat([inp.wg[0], inp.wu[0]], 0).contiguous()  # [2I, H]
    y1 = torch.empty((T, 2 * I), dtype=torch.float16, device=dev)
    h = hid[:T].contiguous()
    wd = inp.wd[0].contiguous()
    y2 = torch.empty((T, H), dtype=torch.float16, device=dev)
    mm1 = tm(lambda: torch.matmul(x, wgu.t(), out=y1))
    mm2 = tm(lambda: torch.matmul(h, wd.t(), out=y2))
    f1, f2 = 4.0 * T * H * I, 2.0 * T * H * I
    print(json.dumps({"dense_compare": f"one expert, {T} tokens, H={H}, I={I}",
                      "gate_up_us": round(gu, 1), "gate_up_tflops": round(f1 / gu / 1e6, 1),
                      "down_us": round(dn, 1), "down_tflops": round(f2 / dn / 1e6, 1),
                      "vendor_gemm_gate_up_us": round(mm1, 1),
                      "vendor_gemm_gate_up_tflops": round(f1 / mm1 / 1e6, 1),
                      "vendor_gemm_down_us": round(mm2, 1),
                      "vendor_gemm_down_tflops": round(f2 / mm2 / 1e6, 1)}), flush=True)


def phase_timing(names, reps=3):
    """Where the tiled stages' time goes, from the phase-timing build of the
    library (librmoe_phase.so: the same kernels, bit-identical results, four
    shader-clock reads per work item; include/routed_moe_phase.h).  For each
    workload and stage (tiled family, one launch at a time): the shares of
    the workgroups' summed run time spent in item prologues (until the first
    K step's operands have landed), K loops, epilogues (until the last output
    store is issued) and between items; the idle tail, 1 - mean / max of the
    workgroups' run times (workgroups that ran out of items while others
    still work); the items per workgroup; and the shader clock, the longest
    workgroup run in ticks over the launch time.  Medians over ``reps``
    launches."""
    import numpy as np
    import torch

    import mixture_experts_routed_grouped_amd as R
    import workloads
    R.use_library(R.PHASE_LIB_PATH)
    dev = torch.device("cuda:0")
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    for name in names:
        if name == "dense":
            cfg = workloads.Config("dense", 8192, 1, 1, 4096, 14336)
            inp = workloads.make_inputs(cfg, device=dev, topk_ids=np.zeros((8192, 1), np.int32))
        else:
            cfg = workloads.CONFIGS[name]
            inp = workloads.make_inputs(cfg, device=dev)
        c = R.build_contract(inp.topk_ids, cfg.experts)
        gs, go, gpo, gidx = (i32(c[q]) for q in ("group_sizes", "group_offsets",
                                                 "group_padded_offsets", "group_idx_for_bx"))
        Tp = c["total_padded_tokens"]
        stacked = torch.zeros((Tp, cfg.hidden), dtype=torch.float16, device=dev)
        wc = torch.zeros(max(c["pairs"], 1), dtype=torch.float32, device=dev)
        R.pack(inp.x.to(dev), torch.from_numpy(inp.topk_w.reshape(-1).copy()).to(dev),
               i32(c["padded_row_of_pair"]), i32(c["compact_pos_of_pair"]), stacked, wc)
        hid = torch.empty((Tp, cfg.intermediate), dtype=torch.float16, device=dev)
        out = torch.empty((Tp, cfg.hidden), dtype=torch.float16, device=dev)
        stages = (("gate_up", 0, lambda: R.gate_up(stacked, inp.wg, inp.wu, gs, gpo, gidx, hid,
                                                  c["pairs"], variant="tile")),
                  ("down", 1, lambda: R.down(hid, inp.wd, wc, gs, go, gpo, gidx, out,
                                             variant="tile")))
        for stage, idx, fn in stages:
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            runs = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3
                rec = R.phase_cycles()[idx].astype(np.float64)
                ran = rec[:, 3] > 0
                pro, loop, epi, items, whole = (rec[ran, j] for j in range(5))
                tot = whole.sum()
                runs.append({"us": us, "prologue": pro.sum() / tot, "k_loop": loop.sum() / tot,
                             "epilogue": epi.sum() / tot,
                             "between_items": (tot - pro.sum() - loop.sum() - epi.sum()) / tot,
                             "idle_tail": 1.0 - whole.mean() / whole.max(),
                             "clock_ghz": float(whole.max()) / us / 1e3,
                             "items_min": int(items.min()), "items_max": int(items.max()),
                             "workgroups": int(ran.sum())})
            med = {k: statistics.median(r[k] for r in runs) for k in runs[0]}
            print(json.dumps({"phase_timing": name, "stage": stage, "launch_us": round(med["us"], 1),
                              **{k: round(med[k], 4) for k in ("prologue", "k_loop", "epilogue",
                                                               "between_items", "idle_tail")},
                              "clock_ghz": round(med["clock_ghz"], 3),
                              "items_per_workgroup": [runs[0]["items_min"], runs[0]["items_max"]],
                              "workgroups": runs[0]["workgroups"]}), flush=True)
        del inp, stacked, hid, out
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.phase_timing:
        phase_timing(args.phase_timing.split(","))
        return
    if args.calibrate_copy_mib:
        calibrate_copy(args.calibrate_copy_mib, args.steps)
        return
    if args.crossover:
        crossover_sweep()
        return
    if args.dense_compare:
        dense_compare()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(expert or tensor sharding is described, not implemented). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import workloads

    torch.cuda.set_device(0)
    cfg = workloads.CONFIGS[args.config]
    head, inp, c = measure(cfg, args.variant, args.steps, args.warmup, with_aux=not args.no_aux)
    result = {
        "metric": METRIC, "value": head.pop("value"), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic", "config": head.pop("config"), "roofline": head.pop("roofline"),
    }
    result.update(head)
    result["device"] = torch.cuda.get_device_name(0)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, inp, c, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    del inp
    torch.cuda.empty_cache()
    # the other workloads, same protocol, fewer steps: each one's step time,
    # useful TFLOP/s and the gate/up kernel's roofline
    also = {}
    for name in [w for w in args.also.split(",") if w and w != cfg.name]:
        r, inp_o, _ = measure(workloads.CONFIGS[name], args.variant, args.also_steps,
                              max(2, args.warmup // 2))
        also[name] = {"value": r["value"], "ms_per_step": r["ms_per_step"],
                      "steps": args.also_steps, "workload": r["config"]["workload"],
                      "variant": r["config"]["variant"], "roofline": r["roofline"],
                      "step_mfma_frac": r["step_mfma_frac"], "step_hbm_frac": r["step_hbm_frac"],
                      "kernels_us": {k: v["avg_us"] for k, v in r["kernels"].items()}}
        del inp_o
        torch.cuda.empty_cache()
    if also:
        result["other_workloads"] = also
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
