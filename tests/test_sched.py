"""Host check of the tiled kernels' work sequence.

`csrc/rmoe_sched.h` decides which (blocks, weight slice) each persistent
workgroup computes.  Built here with g++ (the header is plain C++) into
`sched_check.cpp`, it must cover every (block with valid rows, slice) exactly
once, with the right row counts, for the benchmark workloads' routings,
random and edge-case group sizes, and any number of locality groups and
workgroups per group, whether the workgroups take the items round robin or
one after another from a queue.  A block with no valid rows must get no item (the row
predicate of "Fused MoE GEMM 提交说明", 完整算子代码).
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("sched") / "sched_check")
    subprocess.run([gxx, "-O2", "-Wall", "-Werror", "-o", exe, os.path.join(HERE, "sched_check.cpp")],
                   check=True)
    return exe


def _run(exe, gs, NT, ngrp=8, lanes=32):
    inp = f"{len(gs)} {NT} {ngrp} {lanes}\n" + " ".join(str(int(g)) for g in gs) + "\n"
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=False)
    return out.returncode, out.stdout.strip()


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "fine", "large"])
def test_workload_routings(checker, name):
    cfg = workloads.CONFIGS[name]
    gs = np.bincount(workloads.draw_routing(cfg).ravel(), minlength=cfg.experts)
    for NT in (max(1, cfg.intermediate // 128), (cfg.hidden + 255) // 256):
        rc, out = _run(checker, gs, NT)
        assert rc == 0 and out.startswith("ok"), out


def test_edge_group_sizes(checker):
    cases = [
        [0],                       # no rows at all
        [0, 0, 0, 5],              # only the last expert has rows
        [128, 256, 384],           # counts on block multiples: wholly empty slack blocks
        [127, 129, 255, 257],      # one row short of / past a block
        [1] * 33,                  # many experts with one row each
        [4096],                    # one expert, an even number of full blocks
        [128 * 5 + 1, 0, 3],       # an odd number of live blocks, then a lone tiny block
    ]
    for gs in cases:
        for NT in (1, 3, 8, 9, 112):
            for ngrp, lanes in ((8, 32), (1, 1), (8, 1), (3, 7)):
                rc, out = _run(checker, gs, NT, ngrp, lanes)
                assert rc == 0 and out.startswith("ok"), (gs, NT, ngrp, lanes, out)


def test_random_group_sizes(checker):
    rng = np.random.default_rng(11)
    for _ in range(150):
        E = int(rng.integers(1, 40))
        gs = rng.integers(0, 900, E)
        gs[rng.random(E) < 0.2] = 0
        gs[rng.random(E) < 0.2] = 128 * rng.integers(0, 5)
        rc, out = _run(checker, gs, int(rng.integers(1, 40)), int(rng.integers(1, 9)),
                       int(rng.integers(1, 40)))
        assert rc == 0 and out.startswith("ok"), (list(gs), out)


def test_item_counts_of_the_prefill_stages(checker):
    # prefill routing: 37 entries (32 pairs, 5 lone blocks); gate/up has
    # 112 slices of 128 features (4144 items, 518 per locality group), down
    # 16 slices of 256 (592 items, 74 per group)
    cfg = workloads.CONFIGS["prefill"]
    gs = np.bincount(workloads.draw_routing(cfg).ravel(), minlength=cfg.experts)
    for NT, items, largest in ((112, 4144, 518), (16, 592, 74)):
        rc, out = _run(checker, gs, NT)
        assert rc == 0, out
        assert out.split()[1:] == [str(items), str(largest)], out
