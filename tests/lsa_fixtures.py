"""Test-side input assembly: seeded draws from ``lsa_inputs`` plus the
planting direction and bias, calibrated with the CPU oracle.

Named workloads read their calibration from ``tests/golden/calibration.json``
(written by ``tests/golden/make_calibration.py``, which calls only the
oracle); ad-hoc workloads are calibrated here on the fly, again with the
oracle only.  Nothing here reads the GPU path.
"""
from __future__ import annotations

import numpy as np

import lsa_inputs as gen
from oracle import oracle


def oracle_queries(w: gen.Workload, h=None, Wq=None, Wg=None):
    """Oracle query encoder for every (layer, request): q uint16 [L][B][H][dI],
    g float32 [L][B][H]."""
    h = gen.hidden(w) if h is None else h
    q = np.empty((w.L, w.B, w.H, w.dI), np.uint16)
    g = np.empty((w.L, w.B, w.H), np.float32)
    for l in range(w.L):
        wq, wg = (gen.weights(w, l) if Wq is None else (Wq[l], Wg[l]))
        for b in range(w.B):
            q[l, b], g[l, b] = oracle.project(h[b], wq, wg, w.H, w.dI)
    return q, g


def calibrate(w: gen.Workload, q=None, g=None) -> gen.Calibration:
    """Planting direction u = q_eff / |q_eff| with q_eff the oracle's
    head-collapsed query, and a per-layer bias from the oracle's bias-free
    scores (pooled over requests, first ``calib_rows`` entries of each)."""
    if q is None:
        q, g = oracle_queries(w)
    u = np.empty((w.L, w.B, w.dI), np.float64)
    for l in range(w.L):
        for b in range(w.B):
            qe = oracle.query_collapse(q[l, b], g[l, b])
            u[l, b] = qe / np.linalg.norm(qe)
    rows = w.calib_rows or None
    plants = [gen.planted_sets(w, b) for b in range(w.B)]
    bias = np.empty(w.L, np.float32)
    for l in range(w.L):
        pooled = []
        for b in range(w.B):
            k, s = gen.keys(w, b, l, u[l, b], rows=rows, plant=plants[b])
            pooled.append(oracle.score(k, s, q[l, b], g[l, b], 0.0))
        bias[l] = gen.bias_from_sorted(np.concatenate(pooled), w.sel_frac[l])
    return gen.Calibration(u=u, bias=bias)


def named_calibration(name: str) -> gen.Calibration:
    return gen.load_calibration(gen.WORKLOADS[name])


def build(w: gen.Workload, calib: gen.Calibration | None = None, threads: int = 8):
    """Inputs plus the oracle queries for a workload."""
    q, g = oracle_queries(w)
    if calib is None:
        calib = calibrate(w, q, g) if w.name not in gen.WORKLOADS else named_calibration(w.name)
    inp = gen.indexer_inputs(w, calib, threads=threads)
    return inp, q, g
