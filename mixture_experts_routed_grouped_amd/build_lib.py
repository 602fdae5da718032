"""Build librmoe.so (the C-ABI library) in-tree with hipcc for gfx950.

Every source is compiled to an object in parallel, then linked into
``mixture_experts_routed_grouped_amd/librmoe.so``.  The tiled kernels'
source is compiled a second time with ``RMOE_PHASE_TIMING=1`` and linked
with the same other objects into the diagnostic ``librmoe_phase.so``
(include/routed_moe_phase.h).  Run as a script, or call ``build()``;
``RMOE_RESOURCE_USAGE=1`` prints each kernel's register, LDS and spill usage
from the compiler.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "librmoe.so")
PHASE_LIB = os.path.join(PKG, "librmoe_phase.so")
SOURCES = ["rmoe_api.cpp", "rmoe_stream.hip", "rmoe_tile.hip", "rmoe_pack.hip", "rmoe_contract.hip", "rmoe_router.hip"]
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    extra = ["-Rpass-analysis=kernel-resource-usage"] if os.environ.get("RMOE_RESOURCE_USAGE") else []
    procs = []
    objs = []
    phase_obj = os.path.join(BUILD, "rmoe_tile_phase.o")
    jobs = [(src, os.path.join(BUILD, os.path.splitext(src)[0] + ".o"), []) for src in SOURCES]
    jobs.append(("rmoe_tile.hip", phase_obj, ["-DRMOE_PHASE_TIMING=1"]))
    for src, obj, defs in jobs:
        if not defs:
            objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *COMMON, *extra, *defs, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the device-only target feature
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if lines and (verbose or p.returncode or extra):
            print("\n".join(lines), flush=True)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed on {failed}")
    phase_objs = [phase_obj if o.endswith("rmoe_tile.o") else o for o in objs]
    for out, link in ((LIB, objs), (PHASE_LIB, phase_objs)):
        tmp = out + ".tmp"
        cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *link, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
