"""Host check of the single-launch forward's work queues and its progress.

`csrc/rmoe_sched.h` holds the ticket order the fused kernel runs; built here
with g++ into `fused_check.cpp`, which replays those queues with the
kernel's ticket and done[] logic (a down tile of the pair at bx waits until
done[bx] holds every gate/up slice) as a discrete-event run with random
item times.  It must cover every (live block, slice) of both stages exactly
once and finish every ticket:

* LOCAL hand-over (each XCD runs whole entries, hidden rows stay in its L2):
  for every workload's routing, with 32, 1 or a random number of resident
  workgroups per queue, and with queues that have none at all (then the
  last workgroup out serves them, as the kernel does).  Its queues put every
  gate/up ticket of an entry before its down tickets, so a down ticket's
  inputs are always in tickets already handed out.
* GLOBAL hand-over: finishes whenever every queue has a resident workgroup;
  with a queue that has none, a down ticket whose pair's gate/up slices sit
  in that queue is handed out while they are unreachable -- the checker must
  report exactly that (its wait then ends only at the kernel's deadline).
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
    exe = str(tmp_path_factory.mktemp("fused") / "fused_check")
    subprocess.run([gxx, "-O2", "-Wall", "-Werror", "-o", exe, os.path.join(HERE, "fused_check.cpp")],
                   check=True)
    return exe


def _run(exe, gs, NT1, NT2, mode, resident, seed=1):
    inp = (f"{len(gs)} {NT1} {NT2} {mode} {seed}\n" + " ".join(str(int(r)) for r in resident) + "\n"
           + " ".join(str(int(g)) for g in gs) + "\n")
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=False)
    return out.returncode, out.stdout.strip()


def _shape(cfg):
    return max(1, cfg.intermediate // 128), (cfg.hidden + 255) // 256


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "fine", "large"])
@pytest.mark.parametrize("mode", [1, 2])
def test_workload_queues_finish(checker, name, mode):
    cfg = workloads.CONFIGS[name]
    gs = np.bincount(workloads.draw_routing(cfg).ravel(), minlength=cfg.experts)
    NT1, NT2 = _shape(cfg)
    for resident in ([32] * 8, [1] * 8, [3, 1, 7, 2, 32, 1, 5, 9]):
        rc, out = _run(checker, gs, NT1, NT2, mode, resident)
        assert rc == 0 and out.startswith("ok"), (resident, out)


@pytest.mark.parametrize("name", ["fine", "large", "prefill"])
def test_local_queues_need_no_other_xcd(checker, name):
    """Queues with no resident workgroup: LOCAL still finishes (the last
    workgroup out runs them, gate/up before down); GLOBAL hands out a down
    ticket whose gate/up inputs no running workgroup can reach."""
    cfg = workloads.CONFIGS[name]
    gs = np.bincount(workloads.draw_routing(cfg).ravel(), minlength=cfg.experts)
    NT1, NT2 = _shape(cfg)
    for resident in ([0, 32, 32, 32, 32, 32, 32, 32], [1, 0, 0, 0, 0, 0, 0, 0], [0, 0, 2, 0, 5, 0, 0, 1]):
        rc, out = _run(checker, gs, NT1, NT2, 1, resident)
        assert rc == 0 and out.startswith("ok"), (resident, out)
        rc, out = _run(checker, gs, NT1, NT2, 2, resident)
        assert rc == 3 and out.startswith("UNREACHABLE"), (resident, out)


def test_random_group_sizes_and_residency(checker):
    rng = np.random.default_rng(17)
    for i in range(120):
        E = int(rng.integers(1, 48))
        gs = rng.integers(0, 1500, E)
        gs[rng.random(E) < 0.2] = 0
        gs[rng.random(E) < 0.2] = 128 * rng.integers(0, 6)
        NT1, NT2 = int(rng.integers(1, 20)), int(rng.integers(1, 30))
        resident = rng.integers(0, 6, 8)
        rc, out = _run(checker, gs, NT1, NT2, 1, resident, seed=i)
        assert rc == 0 and out.startswith("ok"), (list(gs), NT1, NT2, list(resident), out)
        resident = np.maximum(resident, 1)
        rc, out = _run(checker, gs, NT1, NT2, 2, resident, seed=i)
        assert rc == 0 and out.startswith("ok"), (list(gs), NT1, NT2, list(resident), out)


def test_edge_group_sizes(checker):
    for gs in ([0], [0, 0, 0, 5], [128, 256, 384], [127, 129, 255, 257], [1] * 33, [4096],
               [128 * 5 + 1, 0, 3]):
        for NT1, NT2 in ((1, 1), (3, 8), (16, 28), (112, 16)):
            for mode in (1, 2):
                rc, out = _run(checker, gs, NT1, NT2, mode, [1] * 8)
                assert rc == 0 and out.startswith("ok"), (gs, NT1, NT2, mode, out)
