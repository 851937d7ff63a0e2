#!/usr/bin/env python3
"""Benchmark of the LSA indexer hot path on one MI355X.

One step = one indexer trigger over one batch: query projection, score +
threshold, three-layer OR + compaction, top-k, hot-pool gather (all five C
entry points).  Default workload: 1M-token context (262,144 compressed entries
per layer), 3 indexer layers, 32 concurrent requests, e4m3 keys with one fp32
scale per entry, top-k 2048, 1 KiB KV rows.

Prints ONE JSON line.  `value` is (request, layer, entry) triples scored and
selected per second of whole-step time; the `roofline` object is for the
dominant kernel, lsa_score, whose per-launch time comes from HIP events
recorded on the stream the kernels run on, inside the timed region.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "lsa_score_ctx1m_traffic.json")
PROFILE_TRAFFIC_LABELS = os.path.join(ROOT, "profiles", "lsa_label_vote_labels128k_traffic.json")


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "sparse_kv_cache_lsa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def score_source_hash() -> str:
    return source_hash(("lsa_score.hip", "lsa_device.h", "lsa_launch.h"))


def labels_source_hash() -> str:
    return source_hash(("lsa_labels.hip", "lsa_device.h", "lsa_dpp.h", "lsa_launch.h"))


def counter_traffic(path, source_hash_now, workload):
    """Counter-derived HBM bytes per launch from a committed profile summary,
    used only while the kernel sources hash the same; else None."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tr = json.load(f)
    if tr.get("kernel_source_hash") == source_hash_now and tr.get("workload") == workload:
        return tr.get("traffic_bytes_per_launch")
    return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="ctx1m")
    p.add_argument("--skip-cpu", action="store_true", help="do not time the CPU oracle")
    p.add_argument("--event-every", type=int, default=5,
                   help="bracket the roofline kernel with events in every n-th timed step")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="CPU oracle sample budget (whole requests until this much time)")
    p.add_argument("--copy-probe", type=int, default=0,
                   help="also run a plain device copy of this many MiB (counter calibration)")
    p.add_argument("--threads", type=int, default=16)
    p.add_argument("--rotate", type=int, default=1,
                   help="cycle the steps over this many copies of every input (keys, scales, "
                        "weights, hidden states, pool), so that small workloads stream from "
                        "HBM instead of the 256 MB Infinity Cache")
    p.add_argument("--no-cold-fetch", action="store_true",
                   help="skip the cold-pool fetch report")
    p.add_argument("--no-attention", action="store_true",
                   help="skip the core-attention report (attention over the hot rows)")
    p.add_argument("--no-stream", action="store_true",
                   help="skip the decode-session report (growing caches, 11 triggers) and the "
                        "survivor-growth sweep")
    p.add_argument("--no-stream-probe", action="store_true",
                   help="skip the plain streaming-read reference measurement")
    p.add_argument("--graph", action="store_true",
                   help="time the steps as replays of one captured HIP graph (per-kernel "
                        "times still come from an evented eager pass)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    torch.cuda.init()
    torch.empty(1, device="cuda")

    if args.workload == "labels128k":
        return bench_labels(args)

    import lsa_inputs as gen
    import sparse_kv_cache_lsa_amd as lsa
    from sparse_kv_cache_lsa_amd.pipeline import TriggerBuffers, pack_weights

    w = gen.WORKLOADS[args.workload]
    dev = "cuda"
    t0 = time.time()
    calib = gen.load_calibration(w)
    inp = gen.indexer_inputs(w, calib, threads=args.threads)
    d = gen.to_device(inp, dev)
    pool = gen.pool_tensor(w, dev)
    buf = TriggerBuffers.allocate(w.L, w.B, w.N, w.H, w.dI, w.k, w.row_elems, device=dev)
    torch.cuda.synchronize()
    print(f"# inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    # input copies the steps cycle over (one unless --rotate)
    def clone(v):
        if v is None:
            return None
        if isinstance(v, (list, tuple)):
            return [clone(x) for x in v]
        return v.clone() if isinstance(v, torch.Tensor) else v
    copies = [(d, pool)] + [(clone(d), pool.clone()) for _ in range(max(1, args.rotate) - 1)]
    # the query weights in their packed load-time layout (lsa_pack_query_weights),
    # made once per copy before any timing
    for dc, _ in copies:
        dc["Wp"] = pack_weights(dc["Wq"], dc["Wg"])
    rot_bytes = sum(t.numel() * t.element_size() for t in
                    [d["h"], pool] + list(d["Wp"]) + list(d["keys"]) +
                    [x for x in (d["scale"] or []) if x is not None]) * len(copies)
    torch.cuda.synchronize()
    it = [0]

    def step(marks=None):
        """One trigger; marks: {position: event} recorded on the stream before
        call 0..4 (position 5: after the last call)."""
        d, pool = copies[it[0] % len(copies)]
        it[0] += 1

        def mark(i):
            if marks is not None and i in marks:
                marks[i].record(stream)
        mark(0)
        lsa.lsa_project_query_packed(d["h"], d["Wp"], buf.q, buf.g, stream=stream)
        mark(1)
        lsa.lsa_score(d["keys"], d["scale"], buf.q, buf.g, d["bias"], buf.mask, buf.cand_idx,
                      buf.cand_z, buf.cand_count, stream=stream)
        mark(2)
        lsa.lsa_select_or_compact(buf.cand_idx, buf.cand_z, buf.cand_count, w.N, buf.surv_idx,
                                  buf.surv_z, buf.surv_count, stream=stream)
        mark(3)
        lsa.lsa_topk(buf.surv_idx, buf.surv_z, buf.surv_count, buf.topk_idx, buf.topk_count,
                     buf.ws_topk, stream=stream)
        mark(4)
        lsa.lsa_gather_hot(pool, buf.topk_idx, buf.hot, stream=stream)
        mark(5)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps between two synchronisations.  Two HIP events on
    # the kernels' stream bracket the score launch (the roofline kernel) of
    # every --event-every-th step.  Each recorded event costs the stream a few
    # microseconds between two kernels, so the sample keeps that overhead
    # small, and the per-call breakdown comes from a separate pass below.
    every = max(1, args.event_every)
    evs = [(ev(), ev()) if i % every == 0 else None for i in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for e in evs:
        step(None if e is None else {1: e[0], 2: e[1]})
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / max(args.steps, 1)
    sampled = [e for e in evs if e is not None]
    mean_score = float(np.mean([e[0].elapsed_time(e[1]) for e in sampled]))

    # per-call breakdown: K more steps (untimed) with an event between calls
    bd = [[ev() for _ in range(6)] for _ in range(args.steps)]
    for e in bd:
        step(dict(enumerate(e)))
    torch.cuda.synchronize()
    launch = "eager"
    if args.graph:
        # the same step captured once and replayed K times
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                lsa.lsa_project_query_packed(d["h"], d["Wp"], buf.q, buf.g)
                lsa.lsa_score(d["keys"], d["scale"], buf.q, buf.g, d["bias"], buf.mask,
                              buf.cand_idx, buf.cand_z, buf.cand_count)
                lsa.lsa_select_or_compact(buf.cand_idx, buf.cand_z, buf.cand_count, w.N,
                                          buf.surv_idx, buf.surv_z, buf.surv_count)
                lsa.lsa_topk(buf.surv_idx, buf.surv_z, buf.surv_count, buf.topk_idx,
                             buf.topk_count, buf.ws_topk)
                lsa.lsa_gather_hot(pool, buf.topk_idx, buf.hot)
        stream.wait_stream(side)
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t_start) * 1e3 / max(args.steps, 1)
        launch = "hip_graph"
    names = ["project", "score", "select", "topk", "gather"]
    per = {n: float(np.median([e[i].elapsed_time(e[i + 1]) for e in bd])) for i, n in enumerate(names)}
    pct = {n: [float(np.percentile([e[i].elapsed_time(e[i + 1]) for e in bd], q)) for q in (10, 90)]
           for i, n in enumerate(names)}
    score_select = float(np.median([e[1].elapsed_time(e[3]) for e in bd]))

    triples = w.triples
    key_bytes = triples * w.key_bytes_per_entry
    achieved = key_bytes / (mean_score * 1e-3) / 1e9
    ss_gbs = key_bytes / (score_select * 1e-3) / 1e9

    traffic = counter_traffic(PROFILE_TRAFFIC, score_source_hash(), w.name)

    counts = buf.surv_count.cpu().numpy()
    result = {
        "metric": "compressed entries scored+selected/sec at 1M ctx; % of peak HBM GB/s",
        "value": triples / (ms_per_step * 1e-3),
        "unit": "(request, layer, entry) triples/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "requests": w.B, "indexer_layers": w.L,
                   "entries_per_layer": w.N, "context_tokens": 4 * w.N, "heads": w.H,
                   "head_dim": w.dI, "hidden": w.D, "key_dtype": w.key_dtype, "top_k": w.k,
                   "kv_row_bytes": 2 * w.row_elems, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "lsa_score", "algorithmic_bytes_per_launch": key_bytes,
                     "mean_launch_ms": mean_score, "timed_launches_sampled": len(sampled)},
        "score_select": {"ms": score_select, "GB/s": ss_gbs, "frac_of_peak": ss_gbs / HBM_PEAK_GBS,
                         "triples_per_s": triples / (score_select * 1e-3),
                         "request_entries_per_s": w.B * w.N / (score_select * 1e-3)},
        "request_entries_per_s": w.B * w.N / (ms_per_step * 1e-3),
        "kernel_ms_median": per,
        "kernel_ms_p10_p90": pct,
        "survivor_fraction": float(counts.mean() / w.N),
        "launch": launch,
        "input_copies": {"count": len(copies), "bytes": rot_bytes},
    }

    if not args.no_stream_probe:
        # reference: a plain streaming read of the same byte count on this GPU
        # (row-wise max over an fp32 buffer, torch's own reduction kernel)
        nrow = max(1, key_bytes // 4096)
        x = torch.ones((nrow, 1024), dtype=torch.float32, device=dev)
        for _ in range(2):
            x.amax(dim=1)
        torch.cuda.synchronize()
        ts = []
        for _ in range(10):
            e0, e1 = ev(), ev()
            e0.record(stream)
            x.amax(dim=1)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        pms = float(np.median(ts))
        pgbs = x.numel() * 4 / (pms * 1e-3) / 1e9
        result["stream_probe"] = {"kernel": "torch amax over rows (plain streaming read)",
                                  "bytes": x.numel() * 4, "ms": pms, "GB/s": pgbs,
                                  "score_frac_of_probe": achieved / pgbs}
        del x

    if args.copy_probe:
        result["copy_probe"] = copy_probe(args.copy_probe, stream)

    if not args.no_attention and w.row_elems == 512:
        result["attention"] = attention_report(w, buf, stream, step, ms_per_step)
        result["fine_topk"] = fine_topk_report(w, buf, stream, args.threads)

    if not args.no_cold_fetch:
        result["cold_fetch"] = cold_fetch(w, d, pool, buf, stream, step, ms_per_step)

    if not args.no_stream and w.name == "ctx1m":
        result["decode_session"] = stream_report(w, d, pool, stream)
        result["survivor_growth"] = growth_report(args.threads)

    if not args.skip_cpu:
        result["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def fine_topk_report(w, buf, stream, threads, launches=20):
    """The top-k ranked by the fine-grained score inside the fetched set
    (lsa_lightning_score over the last trigger's survivors, then lsa_topk over
    those scores): 64 heads of 128 dims with their own e4m3 keys (+ fp32
    scale) per entry.  Mean of `launches` back-to-back pairs between two
    events; its own rooflines (each survivor's key row and scale read once)."""
    import numpy as np
    import torch
    import lsa_inputs as gen
    import sparse_kv_cache_lsa_amd as lsa

    li = gen.lightning_inputs(w, key_dtype="e4m3", threads=threads)
    dev = "cuda"
    keys = torch.from_numpy(li.keys).to(dev)
    scale = torch.from_numpy(li.scale).to(dev)
    q = torch.from_numpy(li.q.view(np.int16)).to(dev).view(torch.bfloat16)
    wt = torch.from_numpy(li.w).to(dev)
    score = torch.empty_like(buf.surv_z)
    ti, tc = torch.empty_like(buf.topk_idx), torch.empty_like(buf.topk_count)

    def run(which):
        if which & 1:
            lsa.lsa_lightning_score(keys, scale, q, wt, buf.surv_idx, buf.surv_count, score,
                                    stream=stream)
        if which & 2:
            lsa.lsa_topk(buf.surv_idx, score, buf.surv_count, ti, tc, buf.ws_topk, stream=stream)

    def timed(which):
        for _ in range(3):
            run(which)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(launches):
            run(which)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / launches

    both = timed(3)
    score_ms = timed(1)
    surv = int(buf.surv_count.sum().item())
    H, dI = li.q.shape[1], li.q.shape[2]
    nbytes = surv * (dI + 4 + 4 + 4) + w.B * H * (2 * dI + 4)   # key row + scale + index + score
    flops = 2.0 * H * dI * surv
    return {"kernel": "lsa_lightning_score", "heads": H, "head_dim": dI, "key_dtype": "e4m3",
            "survivors": surv, "score_ms": score_ms, "score_plus_topk_ms": both,
            "launches": launches, "algorithmic_bytes": nbytes,
            "GB/s": nbytes / (score_ms * 1e-3) / 1e9,
            "frac_hbm": nbytes / (score_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "TFLOP/s": flops / (score_ms * 1e-3) / 1e12,
            "frac_bf16_mfma": flops / (score_ms * 1e-3) / 1e12 / 2500.0}


def attention_report(w, buf, stream, step, ms_per_step, launches=20, tau=64):
    """Core attention of one decode step (lsa_sparse_attention) over the
    trigger's hot rows -- buf.hot, gathered by the last step, with the top-k
    counts -- plus a local window of recent rows, for ATT_HEADS heads: mean
    time of `launches` back-to-back launches between two events, its HBM and
    bf16 matrix-core rooflines, and one decode window of tau steps (one
    trigger, then tau attention steps) timed as a whole."""
    import numpy as np
    import torch
    import lsa_inputs as gen
    import sparse_kv_cache_lsa_amd as lsa

    B, k, D = w.B, w.k, gen.ATT_ROW
    H, W = gen.ATT_HEADS, gen.ATT_WINDOW
    a = gen.attention_inputs(B, H, 0, W, wid=59)
    dev = "cuda"
    q = torch.from_numpy(a.q.view(np.int16)).to(dev).view(torch.bfloat16)
    win = torch.from_numpy(a.win.view(np.int16)).to(dev).view(torch.bfloat16)
    hot = buf.hot.view(torch.bfloat16)
    out = torch.empty((B, H, D), dtype=torch.float32, device=dev)
    nws = lsa.lsa_sparse_attention_workspace_bytes(B, H, D, k, W)
    ws = torch.empty((max(nws, 1),), dtype=torch.uint8, device=dev)
    scale = gen.att_scale()

    def att():
        lsa.lsa_sparse_attention(q, hot, out, scale, hot_count=buf.topk_count, win=win,
                                 ws=ws, stream=stream)

    for _ in range(3):
        att()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(launches):
        att()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / launches
    rows = int(buf.topk_count.sum().item()) + B * W
    nbytes = rows * D * 2 + B * H * D * 2 + B * H * D * 4
    flops = 4.0 * H * rows * D
    # one decode window: a trigger, then tau attention steps
    wins = []
    for _ in range(3):
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        f0.record(stream)
        step()
        for _ in range(tau):
            att()
        f1.record(stream)
        torch.cuda.synchronize()
        wins.append(f0.elapsed_time(f1))
    wms = float(np.median(wins))
    return {"kernel": "lsa_sparse_attention", "heads": H, "row_elems": D,
            "selected_rows": k, "window_rows": W, "rows_attended": rows,
            "splits_workspace_bytes": nws, "ms": ms, "launches": launches,
            "algorithmic_bytes": nbytes, "GB/s": nbytes / (ms * 1e-3) / 1e9,
            "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "flops": flops, "TFLOP/s": flops / (ms * 1e-3) / 1e12,
            "frac_bf16_mfma": flops / (ms * 1e-3) / 1e12 / 2500.0,
            "decode_window": {"tau": tau, "ms": wms,
                              "decode_tokens_per_s": B * tau / (wms * 1e-3),
                              "trigger_ms": ms_per_step, "attention_ms_x_tau": ms * tau}}


def stream_report(w, d, pool, stream, triggers=11, tau=64, per_window=16):
    """A decode session over growing caches (pipeline.StreamingSession) on the
    workload's inputs: the caches start with all but the last
    per_window * (triggers - 1) entries, the host loop triggers every tau steps
    and appends each finished window's entries first; survivors are fetched
    from a pinned host copy of the pool into N/2 resident slots with reuse.
    Each trigger is timed with events (append + trigger + fetch + gather); the
    first trigger's fetch is cold, the later ones are deltas."""
    import numpy as np
    import torch
    import lsa_inputs as gen
    from sparse_kv_cache_lsa_amd.pipeline import StreamingSession

    N_cap, B = w.N, w.B
    N0 = N_cap - per_window * (triggers - 1)
    cold = torch.empty(pool.shape, dtype=pool.dtype, pin_memory=True)
    cold.copy_(pool)
    sess = StreamingSession(w.L, B, N_cap, w.H, w.dI, w.k, w.row_elems, N_cap // 2, cold,
                            key_dtype=w.key_dtype, tau=tau, per_window=per_window)
    sess.append([k[:, :N0].contiguous() for k in d["keys"]],
                None if d["scale"] is None else [s[:, :N0].contiguous() for s in d["scale"]],
                stream=stream)
    hs = gen.drift_hidden(w, triggers)
    hd = [torch.from_numpy(h.view(np.int16)).to("cuda").view(torch.bfloat16) for h in hs]
    win = []
    for i in range(1, triggers):
        lo, hi = N0 + per_window * (i - 1), N0 + per_window * i
        win.append(([k[:, lo:hi].contiguous() for k in d["keys"]],
                    None if d["scale"] is None else [s[:, lo:hi].contiguous() for s in d["scale"]]))
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    marks = []

    def window_source(i):
        e = ev()
        e.record(stream)
        marks.append(e)
        return win[i - 1]

    per = []

    def on_trigger(i, t):
        torch.cuda.synchronize()
        per.append({"step": t, "N": sess.N,
                    "survivors_mean": float(sess.surv_count.float().mean().item()),
                    "rows_fetched": int(sess.res.fetch_count.sum().item())})

    e0 = ev()
    e0.record(stream)
    marks.append(e0)
    ends = []

    def on_trigger_timed(i, t):
        e = ev()
        e.record(stream)
        ends.append(e)
        on_trigger(i, t)

    T = tau * (triggers - 1) + 1
    sess.decode(T, lambda i: hd[i], d["Wp"], d["bias"], window_source, on_trigger_timed,
                stream=stream)
    torch.cuda.synchronize()
    starts = [marks[0]] + marks[1:]
    ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    for r, m in zip(per, ms):
        r["ms"] = m
        r["survivor_fraction"] = r["survivors_mean"] / r["N"]
    delta = [r["ms"] for r in per[1:]]
    return {"requests": B, "triggers": triggers, "tau": tau, "entries_per_window": per_window,
            "N_first": N0, "N_last": sess.N,
            "cold_first_trigger_ms": per[0]["ms"],
            "delta_trigger_ms_median": float(np.median(delta)) if delta else None,
            "per_trigger": per}


def growth_report(threads, lengths=(16384, 32768, 65536, 131072, 262144)):
    """Survivors as the context grows around a fixed relevant set (workload
    growth1m: the planted entries lie in the first 16,384 of 262,144): one
    trigger over each prefix of the caches (lsa_score_strided), mean survivors
    per request and their fraction of N."""
    import numpy as np
    import torch
    import lsa_inputs as gen
    import sparse_kv_cache_lsa_amd as lsa
    from sparse_kv_cache_lsa_amd.pipeline import TriggerBuffers, pack_weights

    w = gen.WORKLOADS["growth1m"]
    inp = gen.indexer_inputs(w, gen.load_calibration(w), threads=threads)
    d = gen.to_device(inp, "cuda")
    wp = pack_weights(d["Wq"], d["Wg"])
    out = []
    for N in lengths:
        buf = TriggerBuffers.allocate(w.L, w.B, N, w.H, w.dI, w.k, w.row_elems)
        lsa.lsa_project_query_packed(d["h"], wp, buf.q, buf.g)
        lsa.lsa_score_strided(d["keys"], d["scale"], buf.q, buf.g, d["bias"], N, buf.mask,
                              buf.cand_idx, buf.cand_z, buf.cand_count)
        lsa.lsa_select_or_compact(buf.cand_idx, buf.cand_z, buf.cand_count, N, buf.surv_idx,
                                  buf.surv_z, buf.surv_count)
        torch.cuda.synchronize()
        m = float(buf.surv_count.float().mean().item())
        out.append({"N": N, "context_tokens": 4 * N, "survivors_mean": m,
                    "survivor_fraction": m / N})
    return {"workload": w.name, "relevant_within_first": w.plant_within, "requests": w.B,
            "points": out}


def cold_fetch(w, d, pool, buf, stream, step, ms_per_step):
    """The fetch of every survivor from a CPU cold pool into GPU memory, with
    reuse of rows already resident (lsa_fetch_survivors): the KV pool of the
    workload copied into pinned host memory, a resident set of N/2 slots per
    request.  Reported: a cold fetch (nothing resident), a delta fetch (the
    survivors of a second trigger whose hidden state is perturbed, after the
    first trigger's rows are resident), and the fetch on a side stream next to
    triggers on the main stream."""
    import numpy as np
    import torch
    import sparse_kv_cache_lsa_amd as lsa
    from sparse_kv_cache_lsa_amd.pipeline import ResidentSet

    ev = lambda: torch.cuda.Event(enable_timing=True)
    B, N = w.B, w.N
    rb = 2 * w.row_elems
    S = N // 2
    t0 = time.time()
    cold = torch.empty(pool.shape, dtype=pool.dtype, pin_memory=True)
    cold.copy_(pool)
    res = ResidentSet.allocate(B, N, S, w.row_elems, dtype=pool.dtype, stream=stream)

    def survivors(h):
        lsa.lsa_project_query_packed(h, d["Wp"], buf.q, buf.g, stream=stream)
        lsa.lsa_score(d["keys"], d["scale"], buf.q, buf.g, d["bias"], buf.mask, buf.cand_idx,
                      buf.cand_z, buf.cand_count, stream=stream)
        lsa.lsa_select_or_compact(buf.cand_idx, buf.cand_z, buf.cand_count, N, buf.surv_idx,
                                  buf.surv_z, buf.surv_count, stream=stream)
        return buf.surv_idx.clone(), buf.surv_count.clone()

    s1 = survivors(d["h"])
    g = torch.Generator(device="cuda")
    g.manual_seed(1)
    noise = torch.randn(d["h"].shape, generator=g, device="cuda")
    h2 = (0.97 * d["h"].float() + (1 - 0.97 ** 2) ** 0.5 * noise).to(d["h"].dtype)
    s2 = survivors(h2)
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    def fetch(s, st=stream):
        res.fetch(cold, s[0], s[1], stream=st)

    def timed(pre, s, reps=3):
        out = []
        for _ in range(reps + 1):            # the first run is a warm-up
            res.reset(stream)
            for p in pre:
                fetch(p)
            e0, e1 = ev(), ev()
            e0.record(stream)
            fetch(s)
            e1.record(stream)
            torch.cuda.synchronize()
            out.append((e0.elapsed_time(e1), int(res.fetch_count.sum())))
        out = out[1:]
        ms = float(np.median([o[0] for o in out]))
        return ms, out[-1][1]

    link_peak = 64.0   # PCIe 5.0 x16, one direction, GB/s
    cold_ms, cold_rows = timed([], s1)
    delta_ms, delta_rows = timed([s1], s2)
    surv2 = int(s2[1].sum())

    # overlap: the cold fetch on a side stream next to as many triggers on the
    # main stream as take about as long
    side = torch.cuda.Stream()
    n_trig = max(1, int(round(cold_ms / ms_per_step)))

    def wall(fn):
        torch.cuda.synchronize()
        t = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) * 1e3

    def triggers():
        for _ in range(n_trig):
            step()

    def reset_side():
        res.reset(side)
        torch.cuda.synchronize()

    reset_side()
    t_fetch = wall(lambda: fetch(s1, side))
    t_trig = wall(triggers)
    reset_side()
    t_both = wall(lambda: (fetch(s1, side), triggers()))
    gbs = lambda r, ms: r * rb / (ms * 1e-3) / 1e9
    return {
        "cold_pool": "pinned host memory [B][N][%d B], read in place by the GPU" % rb,
        "resident_slots_per_request": S,
        "cold": {"ms": cold_ms, "rows": cold_rows, "bytes": cold_rows * rb,
                 "GB/s": gbs(cold_rows, cold_ms), "frac_of_link": gbs(cold_rows, cold_ms) / link_peak},
        "delta": {"ms": delta_ms, "rows": delta_rows, "survivors": surv2,
                  "reused_fraction": 1.0 - delta_rows / max(surv2, 1),
                  "GB/s": gbs(delta_rows, delta_ms),
                  "second_trigger": "hidden state 0.97 h + 0.243 noise (cosine 0.97)"},
        "host_link_peak_GBs": link_peak,
        "overlap": {"triggers": n_trig, "triggers_alone_ms": t_trig, "fetch_alone_ms": t_fetch,
                    "together_ms": t_both},
        "setup_s": setup_s,
    }


def bench_labels(args):
    """Offline label workload: one step = golden labels by majority vote over
    the teacher layers (lsa_label_vote) followed by the student loss and its
    W_q gradient on those labels (lsa_focal_bce_grad)."""
    import numpy as np
    import torch

    import lsa_inputs as gen
    import sparse_kv_cache_lsa_amd as lsa

    w = gen.LABELS
    dev = "cuda"
    t0 = time.time()
    x = np.stack([gen.teacher_logits(w, q) for q in range(w.Q)])
    h, Wq, Wg, K, bias = gen.student(w)
    xd = torch.from_numpy(x).to(dev)
    hd = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).to(dev)
    Kd = torch.from_numpy(K.view(np.int16)).view(torch.bfloat16).to(dev)
    Wqd, Wgd = torch.from_numpy(Wq).to(dev), torch.from_numpy(Wg).to(dev)
    W = (w.N + 31) // 32
    mask = torch.empty((w.Q, w.L, W), dtype=torch.int32, device=dev)
    count = torch.empty((w.Q, w.N), dtype=torch.uint8, device=dev)
    label = torch.empty((w.Q, w.N), dtype=torch.uint8, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    dW = torch.empty((w.H * w.dI, w.D), dtype=torch.float32, device=dev)
    ws = torch.empty(lsa.lsa_focal_bce_grad_workspace_bytes(w.Q, w.N, w.D, w.H, w.dI),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    print(f"# inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()

    def step(e=None, n=3):
        """One step; e: events recorded before the vote, between the calls and
        after the loss/gradient (the first n of them)."""
        if e is not None and n > 0:
            e[0].record(stream)
        lsa.lsa_label_vote(xd, w.top_p, w.theta, count, label, layer_mask=mask, stream=stream)
        if e is not None and n > 1:
            e[1].record(stream)
        lsa.lsa_focal_bce_grad(hd, Wqd, Wgd, bias, Kd, label, w.gamma, loss, dW, ws, H=w.H,
                               dI=w.dI, stream=stream)
        if e is not None and n > 2:
            e[2].record(stream)

    ev = lambda: torch.cuda.Event(enable_timing=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: two events bracket the vote launch (the roofline kernel)
    # of every --event-every-th step; the loss/gradient time comes from a
    # separate pass
    every = max(1, args.event_every)
    evs = [[ev(), ev()] if i % every == 0 else None for i in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for e in evs:
        step(e, 2)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / max(args.steps, 1)
    vote_ms = [e[0].elapsed_time(e[1]) for e in evs if e is not None]
    bd = [[ev() for _ in range(3)] for _ in range(args.steps)]
    for e in bd:
        step(e)
    torch.cuda.synchronize()
    focal_ms = [e[1].elapsed_time(e[2]) for e in bd]
    logits = w.Q * w.L * w.N
    # algorithmic bytes: logits read once, masks + counts + labels written
    vote_bytes = logits * 4 + w.Q * w.L * W * 4 + 2 * w.Q * w.N
    # algorithmic flops of the student step: projection (q and gates), logits,
    # key gradient, dW_q -- each 2 flops per multiply-add
    HdI = w.H * w.dI
    focal_flops = 2.0 * w.Q * w.D * (HdI + w.H) + 2 * 2.0 * w.Q * w.N * w.dI + 2.0 * HdI * w.D * w.Q
    vote_mean = float(np.mean(vote_ms))
    focal_mean = float(np.mean(focal_ms))
    vote_gbs = vote_bytes / (vote_mean * 1e-3) / 1e9
    focal_tfs = focal_flops / (focal_mean * 1e-3) / 1e12
    result = {
        "metric": "teacher logits labelled per second (label vote + student loss/grad)",
        "value": logits / (ms_per_step * 1e-3),
        "unit": "(query, layer, entry) logits/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "queries": w.Q, "teacher_layers": w.L, "entries": w.N,
                   "top_p": w.top_p, "theta": w.theta, "gamma": w.gamma, "heads": w.H,
                   "head_dim": w.dI, "hidden": w.D, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": vote_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": vote_gbs / HBM_PEAK_GBS,
                     "traffic": counter_traffic(PROFILE_TRAFFIC_LABELS, labels_source_hash(), w.name),
                     "kernel": "lsa_label_vote",
                     "algorithmic_bytes_per_launch": vote_bytes, "mean_launch_ms": vote_mean,
                     "timed_launches_sampled": len(vote_ms)},
        "focal": {"bound": "mfma", "achieved": focal_tfs, "peak": 157.3, "unit": "TFLOP/s",
                  "frac": focal_tfs / 157.3, "kernel": "lsa_focal_bce_grad (fp32)",
                  "algorithmic_flops_per_launch": focal_flops, "mean_launch_ms": focal_mean},
        "kernel_ms_median": {"label_vote": float(np.median(vote_ms)),
                             "focal_bce_grad": float(np.median(focal_ms))},
        "loss": float(loss.item()),
        "positive_label_fraction": float(label.float().mean().item()),
    }
    if args.copy_probe:
        result["copy_probe"] = copy_probe(args.copy_probe, stream)
    if not args.skip_cpu:
        result["cpu_baseline"] = cpu_baseline_labels(w, x, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def copy_probe(mib, stream):
    """A plain copy of known size for hardware-counter calibration: the row
    gather with the identity index list reads and writes exactly rows * 1 KiB
    (plus the 4-byte indices)."""
    import torch
    import sparse_kv_cache_lsa_amd as lsa
    rows = (mib << 20) // 1024
    src = torch.zeros((1, rows, 512), dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    ident = torch.arange(rows, dtype=torch.int32, device="cuda").reshape(1, rows)
    lsa.lsa_gather_hot(src, ident, dst, stream=stream)
    torch.cuda.synchronize()
    return {"kernel": "gather_kernel (identity index list)",
            "read_bytes": rows * 1024 + rows * 4, "write_bytes": rows * 1024}


def cpu_baseline_labels(w, x, budget_s):
    """The CPU oracle's nucleus + vote on whole queries until the budget is
    used; throughput in teacher logits per second."""
    from oracle import oracle
    oracle._load()
    import numpy as np
    t0 = time.perf_counter()
    done = 0
    while done < w.Q and (time.perf_counter() - t0) < budget_s:
        sel = np.stack([oracle.nucleus(x[done, l], w.top_p)[0] for l in range(w.L)])
        oracle.vote(sel, w.theta)
        done += 1
    el = time.perf_counter() - t0
    return {"value": done * w.L * w.N / el, "unit": "(query, layer, entry) logits/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{done} of {w.Q} queries x {w.L} layers x {w.N} entries "
                      f"(softmax + nucleus + vote, no student step), {el:.1f}s"}


def cpu_baseline(w, inp, budget_s):
    """The CPU oracle as it stands, on whole requests of the same workload
    (all layers: projection, score, threshold, OR/compaction, top-k) until
    the time budget is used; throughput in triples/s."""
    import numpy as np
    from oracle import oracle
    oracle._load()
    t0 = time.perf_counter()
    done = 0
    b = 0
    while b < w.B and (time.perf_counter() - t0) < budget_s:
        zs = []
        for l in range(w.L):
            q, g = oracle.project(inp.h[b], inp.Wq[l], inp.Wg[l], w.H, w.dI)
            zs.append(oracle.score(inp.keys[l][b], None if inp.scale[l] is None else inp.scale[l][b],
                                   q, g, float(inp.bias[l])))
        z = np.stack(zs)
        surv, zstar, _ = oracle.merge_compact(oracle.threshold(z), z)
        oracle.topk(surv, zstar, w.k)
        done += 1
        b += 1
    el = time.perf_counter() - t0
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")),
                         "unknown")
    except OSError:
        pass
    return {"value": done * w.L * w.N / el, "unit": "(request, layer, entry) triples/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{done} of {w.B} requests x {w.L} layers x {w.N} entries "
                      f"(project+score+threshold+OR/compact+top-k), {el:.1f}s",
            "cpu_model": model, "nproc": os.cpu_count(),
            "single_thread_tiny": oracle_tiny_single_thread()}


_TINY_ORACLE = r"""
import json, sys, time
sys.path.insert(0, sys.argv[1]); sys.path.insert(0, sys.argv[1] + "/tests")
import lsa_inputs as gen
from oracle import oracle
w = gen.WORKLOADS["tiny"]
inp = gen.indexer_inputs(w, gen.load_calibration(w), threads=1)
oracle._load()
oracle.set_num_threads(1)
t0 = time.perf_counter(); reps = 0
while reps < 3 or time.perf_counter() - t0 < 1.0:
    for b in range(w.B):
        zs = []
        for l in range(w.L):
            q, g = oracle.project(inp.h[b], inp.Wq[l], inp.Wg[l], w.H, w.dI)
            zs.append(oracle.score(inp.keys[l][b], None if inp.scale[l] is None else inp.scale[l][b],
                                   q, g, float(inp.bias[l])))
        z = __import__("numpy").stack(zs)
        surv, zstar, _ = oracle.merge_compact(oracle.threshold(z), z)
        oracle.topk(surv, zstar, w.k)
    reps += 1
el = time.perf_counter() - t0
print(json.dumps({"value": reps * w.B * w.L * w.N / el, "unit": "(request, layer, entry) triples/s",
                  "threads": oracle.num_threads(), "repeats": reps, "seconds": el}))
"""


def oracle_tiny_single_thread():
    """The oracle on the tiny workload (1 request, 1 layer, 4096 entries) with
    one OpenMP thread, in a child process (the thread count is fixed when the
    OpenMP runtime starts)."""
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1")
    try:
        r = subprocess.run([sys.executable, "-c", _TINY_ORACLE, os.path.dirname(os.path.abspath(__file__))],
                           env=env, capture_output=True, text=True, timeout=120)
        return json.loads(r.stdout.strip().splitlines()[-1])
    except Exception as e:   # reported, never fatal for the GPU figures
        return {"error": str(e)[:200]}


if __name__ == "__main__":
    main()
