"""GPU test: the forward paths can be captured in a HIP graph by a caller.

Each path (streaming, tiled, single launch) is captured once on a side
stream, then replayed several times with eager work and synchronizations in
between (an eager forward on other output buffers, a fill of the outputs);
every replay must reproduce the eager result bit for bit on the valid rows,
and the single launch's queue state must be back to zero after each replay."""
import pytest
import torch

import mixture_experts_routed_grouped_amd as R
import workloads
from _gpu_run import fresh_outputs, prepare

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("path", ["stream", "tile", "single-launch"])
def test_forward_graph_replay(path):
    cfg = workloads.Config("graph", 300, 5, 2, 256, 384, routing="zipf", zipf_s=1.4, seed=1)
    d = fresh_outputs(prepare(workloads.make_inputs(cfg)))
    rows = d["prow"].long()
    tables = (d["gs"], d["go"], d["gpo"], d["gidx"])
    weights = (d["stacked"], d["wg"], d["wu"], d["wd"], d["w_compact"])
    sync = torch.zeros(R.fused_sync_words(d["c"]["num_blocks_m"]), dtype=torch.int32, device="cuda")

    def fwd(hid, out):
        if path == "single-launch":
            R.forward_fused(*weights, *tables, hid, out, sync=sync)
        else:
            R.forward(*weights, *tables, hid, out, variant=path)

    fwd(d["hid"], d["out"])
    torch.cuda.synchronize()
    want = d["out"][rows].clone()
    other_hid, other_out = torch.empty_like(d["hid"]), torch.empty_like(d["out"])
    print(f"[graph] {path}: capture", flush=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            fwd(d["hid"], d["out"])
    torch.cuda.synchronize()
    for i in range(4):
        d["out"].fill_(0.0)
        fwd(other_hid, other_out)          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d["out"][rows].view(torch.int16), want.view(torch.int16)), f"replay {i}"
        assert torch.equal(other_out[rows].view(torch.int16), want.view(torch.int16)), f"eager {i}"
        if path == "single-launch":
            assert not sync.cpu().numpy().any()
