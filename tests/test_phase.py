"""The phase-timing diagnostic build (librmoe_phase.so,
include/routed_moe_phase.h): the same C ABI plus rmoe_phase_cycles, which
the product library does not export.

CPU: both libraries load, the diagnostic one exports every symbol of both
headers, the product one not rmoe_phase_cycles, and bad arguments return the
documented status without a device call.
GPU: the diagnostic build's outputs equal the product build's bit for bit
(the instrumentation only reads the clock), and its records are consistent:
every item of each stage is counted once (the tiled schedule's item count:
entries = ceil(live blocks / 2) per expert, times I/128 weight slices for
gate/up and ceil(H/256) for down), and no workgroup's phases add up to more
than its whole run."""
import ctypes
import os
import re

import numpy as np
import pytest

import mixture_experts_routed_grouped_amd as R
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared(header):
    text = open(os.path.join(ROOT, "include", header)).read()
    return re.findall(r"RMOE_API\s+[\w\s\*]+?\b(rmoe_\w+)\s*\(", text)


def _phase_lib():
    if not os.path.exists(R.PHASE_LIB_PATH):
        pytest.skip("librmoe_phase.so is not built")
    return ctypes.CDLL(R.PHASE_LIB_PATH)


def test_phase_library_exports():
    P = _phase_lib()
    names = _declared("routed_moe.h") + _declared("routed_moe_phase.h")
    assert "rmoe_phase_cycles" in names
    for n in names:
        assert hasattr(P, n), n
    assert not hasattr(ctypes.CDLL(R.LIB_PATH), "rmoe_phase_cycles")


def test_phase_cycles_argument_errors_without_gpu():
    P = _phase_lib()
    P.rmoe_phase_cycles.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    P.rmoe_phase_cycles.restype = ctypes.c_int
    buf = np.zeros(10, dtype=np.uint64)
    assert P.rmoe_phase_cycles(None, 2 * 1024 * 5 * 8) == -1
    assert P.rmoe_phase_cycles(ctypes.c_void_p(buf.ctypes.data), buf.nbytes) == -1   # too small


def _items(gs, E, H, I):
    entries = sum(((int(n) + 127) // 128 + 1) // 2 for n in gs[:E])
    return entries * (I // 128), entries * ((H + 255) // 256)


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", [
    workloads.Config("ph_uniform", 1500, 8, 2, 512, 768, routing="uniform", seed=41),
    workloads.Config("ph_zipf", 3000, 24, 4, 384, 640, routing="zipf", zipf_s=1.2, seed=42),
])
def test_phase_build_matches_product_and_counts_items(cfg):
    import torch
    from _gpu_run import forward, prepare

    _phase_lib()
    d = prepare(workloads.make_inputs(cfg))
    print(f"[phase] {cfg.name}: product forward (tile)", flush=True)
    forward(d, "tile")
    want_hid, want_out = d["hid"].clone(), d["out"].clone()
    prev = R.use_library(R.PHASE_LIB_PATH)
    try:
        print(f"[phase] {cfg.name}: diagnostic forward (tile)", flush=True)
        forward(d, "tile")
        rec = R.phase_cycles()
    finally:
        R.use_library(prev)
    assert torch.equal(d["hid"].view(torch.int16), want_hid.view(torch.int16))
    assert torch.equal(d["out"].view(torch.int16), want_out.view(torch.int16))
    gu_items, dn_items = _items(d["c"]["group_sizes"], cfg.experts, cfg.hidden, cfg.intermediate)
    for stage, n_items in ((0, gu_items), (1, dn_items)):
        r = rec[stage].astype(np.int64)
        ran = r[:, 3] > 0
        assert int(r[:, 3].sum()) == n_items, (stage, int(r[:, 3].sum()), n_items)
        assert (r[ran, 0] + r[ran, 1] + r[ran, 2] <= r[ran, 4]).all()
        assert (r[ran, 1] > 0).all()
