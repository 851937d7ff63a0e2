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


def test_cold_fetch_graph_replays_match_eager():
    """Reset, two fetches from a pinned host cold pool and the resident
    gather, captured once; every replay equals the eager run."""
    import sparse_kv_cache_lsa_amd as lsa
    rng = np.random.default_rng(21)
    B, N, S, rb, k = 3, 5000, 1800, 64, 300
    cold = torch.from_numpy(rng.integers(0, 256, (B, N, rb), dtype=np.uint8)).pin_memory()
    sets = []
    for t in range(2):
        idx = np.full((B, N), -1, np.int32)
        cnt = np.zeros(B, np.int32)
        for b in range(B):
            x = np.sort(rng.choice(N, 1000 + 200 * b + 100 * t, replace=False)).astype(np.int32)
            idx[b, :x.size] = x
            cnt[b] = x.size
        sets.append((torch.from_numpy(idx).to(DEV), torch.from_numpy(cnt).to(DEV)))
    top = torch.from_numpy(np.sort(rng.choice(N, (B, k)), axis=1).astype(np.int32)).to(DEV)
    so = torch.empty((B, N), dtype=torch.int32, device=DEV)
    eo = torch.empty((B, S), dtype=torch.int32, device=DEV)
    rows = torch.zeros((B, S, rb), dtype=torch.uint8, device=DEV)
    fc = torch.empty((B,), dtype=torch.int32, device=DEV)
    hot = torch.empty((B, k, rb), dtype=torch.uint8, device=DEV)
    ws = torch.empty((lsa.lsa_fetch_workspace_bytes(B, N, N),), dtype=torch.uint8, device=DEV)
    outs = (so, eo, rows, fc, hot)

    def run():
        lsa.lsa_resident_reset(so, eo)
        for s in sets:
            lsa.lsa_fetch_survivors(cold, s[0], s[1], so, eo, rows, fc, ws)
        lsa.lsa_gather_resident(rows, so, top, hot)

    run()
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.view(torch.uint8).fill_(0x33 + rep)
        junk = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, t in enumerate(outs):
            if t is rows:        # slots left free keep whatever bytes they held
                occ = want[1] >= 0
                assert torch.equal(t[occ], want[i][occ]), rep
            else:
                assert torch.equal(t, want[i]), (rep, i)
        del junk


def test_graph_reads_the_current_bias():
    """The bias is a device array read when the kernels run: a graph captured
    once follows new bias values written between replays (each replay equals
    an eager trigger with the same bias)."""
    w = gen.WORKLOADS["tiny"]
    inp = gen.indexer_inputs(w, gen.load_calibration(w))
    d = gen.to_device(inp, DEV)
    pool = gen.pool_tensor(w, DEV)
    buf = TriggerBuffers.allocate(w.L, w.B, w.N, w.H, w.dI, w.k, w.row_elems, device=DEV)
    bias = d["bias"].clone()
    base = float(inp.bias[0])
    shifts = [0.0, 3.0, -2.0]
    want = []
    for sh in shifts:
        bias.fill_(base + sh)
        run_trigger(buf, d["h"], d["Wq"], d["Wg"], d["keys"], d["scale"], bias, pool)
        torch.cuda.synchronize()
        want.append(_snapshot(buf))
    # a larger bias selects more entries
    assert int(want[1]["surv_count"][0]) > int(want[0]["surv_count"][0]) > int(
        want[2]["surv_count"][0])
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            run_trigger(buf, d["h"], d["Wq"], d["Wg"], d["keys"], d["scale"], bias, pool)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(2):
        for i, sh in enumerate(shifts):
            bias.fill_(base + sh)
            junk = torch.randn(1 << 20, device=DEV).sum()
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            got = _snapshot(buf)
            for key, v in want[i].items():
                assert torch.equal(got[key], v), (rep, sh, key)
            del junk
