"""The C ABI used from plain C (tests/c_abi_layer.c): host contract, device
pack, forward and combine through include/routed_moe.h, with no Python in
the caller.

CPU: the caller compiles as C11 against the header, warnings as errors.
GPU: it runs a routed layer on seeded inputs written to files, and its
combined output must match the oracle's layer (oracle contract, packing,
the C reference forward, the k-way combine) at the stated tolerance
|y - oracle| <= 2e-2 + 2e-2 |oracle|, once for a batch the library streams
and once for a batch it tiles."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import workloads

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "mixture_experts_routed_grouped_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _compile(out_dir):
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("gcc or the HIP runtime headers are not available")
    if not os.path.exists(os.path.join(PKG, "librmoe.so")):
        pytest.skip("librmoe.so is not built")
    exe = os.path.join(out_dir, "c_abi_layer")
    subprocess.run([gcc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I" + os.path.join(ROCM, "include"), os.path.join(HERE, "c_abi_layer.c"),
                    "-L" + PKG, "-lrmoe", "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
                    "-Wl,-rpath," + PKG, "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe],
                   check=True)
    return exe


def test_c_caller_compiles(tmp_path):
    assert os.path.exists(_compile(str(tmp_path)))


@pytest.mark.gpu
@pytest.mark.parametrize("cfg,family", [
    (workloads.Config("c_stream", 20, 8, 2, 256, 256, routing="uniform", seed=21), "stream"),
    (workloads.Config("c_tile", 300, 12, 2, 256, 384, routing="zipf", zipf_s=1.3, seed=22), "tile"),
])
def test_c_caller_layer_matches_oracle(tmp_path, cfg, family):
    from oracle import combine as CB
    from _oracle_run import run as oracle_run

    exe = _compile(str(tmp_path))
    inp = workloads.make_inputs(cfg)
    d = str(tmp_path)
    inp.x.numpy().view(np.uint16).tofile(os.path.join(d, "x.bin"))
    np.ascontiguousarray(inp.topk_ids, np.int32).tofile(os.path.join(d, "ids.bin"))
    np.ascontiguousarray(inp.topk_w, np.float32).tofile(os.path.join(d, "w.bin"))
    for name, t in (("wg", inp.wg), ("wu", inp.wu), ("wd", inp.wd)):
        t.numpy().view(np.uint16).tofile(os.path.join(d, name + ".bin"))
    print(f"[c caller] {cfg.name}: {cfg.tokens} tokens, E={cfg.experts}, k={cfg.top_k}", flush=True)
    r = subprocess.run([exe, d, str(cfg.tokens), str(cfg.top_k), str(cfg.experts), str(cfg.hidden),
                        str(cfg.intermediate)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("ok") and f"family {family}" in r.stdout, r.stdout
    got = np.fromfile(os.path.join(d, "y.bin"), np.float16).reshape(cfg.tokens, cfg.hidden)
    o = oracle_run(inp)
    want = CB.combine(o["out"], np.asarray(o["c"]["padded_row_of_pair"]), cfg.tokens, cfg.top_k)
    got64, want64 = got.astype(np.float64), want.astype(np.float64)
    assert np.isfinite(got64).all()
    err = np.abs(got64 - want64)
    assert (err <= 2e-2 + 2e-2 * np.abs(want64)).all(), float(err.max())
