"""A whole indexer trigger captured in a HIP graph and replayed.

The library allocates nothing and never synchronises inside a call, so the
five calls (and the kernels of a two-stage top-k) can be captured.  Each
replay is compared with the eager run; eager work and synchronisations run
between the replays."""
import numpy as np
import pytest
import torch

import lsa_inputs as gen
from gpu_util import DEV
from sparse_kv_cache_lsa_amd.pipeline import TriggerBuffers, run_trigger

pytestmark = pytest.mark.gpu

OUTS = ("q", "g", "mask", "cand_count", "surv_count", "topk_idx", "topk_count", "hot")


def _snapshot(buf):
    out = {n: getattr(buf, n).clone() for n in OUTS}
    for b in range(buf.surv_count.shape[0]):
        n = int(buf.surv_count[b])
        out[f"surv_idx{b}"] = buf.surv_idx[b, :n].clone()
        out[f"surv_z{b}"] = buf.surv_z[b, :n].clone()
    return out


@pytest.mark.parametrize("name", ["tiny", "ctx128k", "custom_long"])
def test_trigger_graph_replays_match_eager(name):
    if name == "custom_long":
        # long enough for the two-stage top-k (more than 16K survivors of capacity)
        w = gen.custom("graph", 93, B=2, L=3, N=40000, H=16, dI=64, D=512, k=512, row_elems=64)
        calib = None
    else:
        w = gen.WORKLOADS[name]
        calib = gen.load_calibration(w)
    if calib is None:
        u = np.ones((w.L, w.B, w.dI)) / np.sqrt(w.dI)
        calib = gen.Calibration(u=u, bias=np.full(w.L, -0.5, np.float32))
    inp = gen.indexer_inputs(w, calib)
    d = gen.to_device(inp, DEV)
    pool = gen.pool_tensor(w, DEV)
    buf = TriggerBuffers.allocate(w.L, w.B, w.N, w.H, w.dI, w.k, w.row_elems, device=DEV)

    def trigger():
        run_trigger(buf, d["h"], d["Wq"], d["Wg"], d["keys"], d["scale"], d["bias"], pool)

    trigger()
    torch.cuda.synchronize()
    want = _snapshot(buf)

    # scribble over every output, then capture
    for n in OUTS + ("surv_idx", "surv_z"):
        getattr(buf, n).view(torch.uint8).fill_(0xA5)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            trigger()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(3):
        for n in OUTS + ("surv_idx", "surv_z"):
            getattr(buf, n).view(torch.uint8).fill_(0x5A + rep)
        junk = torch.randn(1 << 20, device=DEV).sum()     # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(buf)
        for key, v in want.items():
            assert torch.equal(got[key], v), (name, rep, key)
        del junk
