"""CPU checks of bench.py's contract: it measures one GPU and refuses more
before touching a device; a stored HBM-traffic record is reported only for
the variant and the exact kernel sources it was measured on; the committed
records are well formed (per-launch bytes = scaled counters, ratio =
measured / algorithmic)."""
import glob
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_record_needs_matching_variant_and_sources(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    hashes = {v: bench.kernel_src_hash(v) for v in ("stream", "tile")}  # the repository's sources
    rec = {"variant": "tile", "kernel_src_sha": hashes["tile"], "hbm_bytes_per_launch": 123.0}
    (tmp_path / "profiles" / "traffic_gate_up_wl.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_src_hash", hashes.__getitem__)
    assert bench.traffic_for("gate_up", "wl", "tile") == 123.0
    assert bench.traffic_for("gate_up", "wl", "stream") is None      # other variant
    assert bench.traffic_for("gate_up", "other", "tile") is None     # no record
    rec["kernel_src_sha"] = "0" * 16                                 # sources changed since
    (tmp_path / "profiles" / "traffic_gate_up_wl.json").write_text(json.dumps(rec))
    assert bench.traffic_for("gate_up", "wl", "tile") is None


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json"))))
def test_committed_traffic_records_are_consistent(path):
    r = json.load(open(path))
    for key in ["kernel", "workload", "variant", "kernel_src_sha", "fetch_size_kib_per_dispatch",
                "write_size_kib_per_dispatch", "fetch_scale", "write_scale", "hbm_bytes_per_launch",
                "algorithmic_bytes_per_launch", "traffic_over_algorithmic", "commands"]:
        assert key in r, key
    assert r["variant"] in ("stream", "tile")
    assert os.path.basename(path) == f"traffic_gate_up_{r['workload']}.json"
    hbm = (r["fetch_size_kib_per_dispatch"] * r["fetch_scale"]
           + r["write_size_kib_per_dispatch"] * r["write_scale"]) * 1024
    assert abs(hbm - r["hbm_bytes_per_launch"]) <= 1e-6 * hbm
    assert abs(r["traffic_over_algorithmic"] - hbm / r["algorithmic_bytes_per_launch"]) < 1e-9
    assert all(c.startswith("rocprofv3 ") and "bench.py" in c for c in r["commands"])
