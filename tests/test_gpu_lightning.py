"""Parity of lsa_lightning_score (the fine-grained score inside the fetched set:
per-query ReLU-gated heads with weights over each entry's own key) with the
oracle, through the C ABI, and of the top-k that ranks by it.

Tolerance, from the arithmetic: bf16 x bf16 products are exact (e4m3 keys
widen exactly), each head's dot product is an fp32 sum of dI = 64 or 128
terms, the weighted head sum another fp32 sum of H terms, then the scale:
|score_gpu - score_oracle| <= 2^-16 * sigma_s * sum_h w_h sum_d |q_hd k_sd|.
The top-k is compared under the usual k-th band widened by that bound."""
import numpy as np
import pytest
import torch

import lsa_inputs as gen
import parity
import sparse_kv_cache_lsa_amd as lsa
from gpu_util import DEV, dev, host
from oracle import oracle

pytestmark = pytest.mark.gpu


def _key_abs(keys, scale):
    if keys.dtype == np.uint16:
        return np.abs(gen.bf16_bits_to_f32(keys)).astype(np.float64)
    k = torch.from_numpy(np.ascontiguousarray(keys)).view(torch.float8_e4m3fn).double().numpy()
    return np.abs(k) * np.asarray(scale, np.float64)[:, None]


def _bound(keys, scale, q, w, idx):
    qa = np.abs(gen.bf16_bits_to_f32(q)).astype(np.float64)
    ka = _key_abs(keys, scale)[idx]
    return 2.0 ** -16 * (ka @ qa.T) @ np.asarray(w, np.float64) + 1e-30


def _run(li, surv, count, cap):
    B, N, dI = li.keys.shape
    kd = dev(li.keys)
    sd = None if li.scale is None else dev(li.scale)
    score = torch.full((B, cap), float("nan"), dtype=torch.float32, device=DEV)
    si, sc = dev(surv), dev(count)
    lsa.lsa_lightning_score(kd, sd, dev(li.q), dev(li.w), si, sc, score)
    k = 256
    ti = torch.empty((B, k), dtype=torch.int32, device=DEV)
    tc = torch.empty((B,), dtype=torch.int32, device=DEV)
    ws = torch.empty((max(1, lsa.lsa_topk_workspace_bytes(B, cap, k)),), dtype=torch.uint8,
                     device=DEV)
    lsa.lsa_topk(si, score, sc, ti, tc, ws)
    torch.cuda.synchronize()
    return host(score), host(ti), host(tc), k


def _lists(rng, B, N, cap, fracs):
    surv = np.full((B, cap), -1, np.int32)
    count = np.zeros(B, np.int32)
    for b in range(B):
        n = min(cap, int(fracs[b % len(fracs)] * N))
        s = np.sort(rng.choice(N, n, replace=False)).astype(np.int32)
        surv[b, :n] = s
        count[b] = n
    return surv, count


@pytest.mark.parametrize("kdt,H,dI,B,N", [("e4m3", 64, 128, 3, 40000), ("bf16", 64, 128, 2, 30000),
                                          ("bf16", 16, 64, 2, 5000), ("e4m3", 32, 64, 4, 777),
                                          ("e4m3", 48, 128, 3, 3333), ("bf16", 48, 64, 2, 65)])
def test_lightning_scores_and_topk_match_oracle(kdt, H, dI, B, N):
    w = gen.custom("light", 97 + H + dI, B=B, N=N, H=8, dI=64, D=256, key_dtype=kdt)
    li = gen.lightning_inputs(w, H=H, dI=dI)
    rng = np.random.default_rng(N + H)
    surv, count = _lists(rng, B, N, N, (0.25, 0.6, 0.01, 1.0))
    score, top, tcount, k = _run(li, surv, count, N)
    for b in range(B):
        n = int(count[b])
        sv = surv[b, :n]
        want = oracle.lightning(li.keys[b], None if li.scale is None else li.scale[b], li.q[b],
                                li.w[b], sv)
        tol = _bound(li.keys[b], None if li.scale is None else li.scale[b], li.q[b], li.w[b], sv)
        err = np.abs(score[b, :n].astype(np.float64) - want)
        assert (err <= tol).all(), f"request {b}: worst err/tol {(err / tol).max():.3g}"
        extra = np.zeros(N)
        extra[sv] = tol
        parity.check_topk(top[b], int(tcount[b]), sv, want, k, extra=extra)
        assert np.isnan(score[b, n:]).all()   # slots past the count are not written


def test_lightning_at_the_key_size_limit():
    # one request whose bf16 keys reach the documented limit: 2^23 - 1 rows of
    # 128 dims (2^31 - 256 bytes).  Only the survivors' rows are read, so only
    # they hold fresh N(0, 1/dI) keys; the survivors include the first and last
    # 100 rows (the largest offsets) and 20,000 rows in between.
    N, H, dI = (1 << 23) - 1, 64, 128
    rng = np.random.default_rng(2323)
    sv = np.unique(np.concatenate([np.arange(100), np.arange(N - 100, N),
                                   rng.choice(N, 20000, replace=False)])).astype(np.int32)
    keys = np.zeros((1, N, dI), np.uint16)
    keys[0, sv] = gen.to_bf16_bits((rng.standard_normal((sv.size, dI)) / np.sqrt(dI))
                                   .astype(np.float32))
    q = gen.to_bf16_bits(rng.standard_normal((1, H, dI)).astype(np.float32))
    wt = rng.uniform(0.0, 1.0, (1, H)).astype(np.float32)
    li = gen.LightningInputs(q=q, w=wt, keys=keys, scale=None)
    cap = sv.size
    score, top, tcount, k = _run(li, sv[None, :], np.array([cap], np.int32), cap)
    want = oracle.lightning(keys[0], None, q[0], wt[0], sv)
    tol = _bound(keys[0, sv], None, q[0], wt[0], np.arange(cap))
    err = np.abs(score[0].astype(np.float64) - want)
    assert (err <= tol).all(), f"worst err/tol {(err / tol).max():.3g}"
    extra = np.zeros(N)
    extra[sv] = tol
    parity.check_topk(top[0], int(tcount[0]), sv, want, k, extra=extra)


def test_lightning_empty_and_capped_lists():
    w = gen.custom("light0", 99, B=3, N=3000, H=8, dI=64, D=256, key_dtype="e4m3")
    li = gen.lightning_inputs(w)
    surv = np.tile(np.arange(1000, dtype=np.int32), (3, 1))
    count = np.array([0, 5000, 1000], np.int32)        # none; above the capacity; all
    score, top, tcount, k = _run(li, surv, count, 1000)
    assert np.isnan(score[0]).all() and tcount[0] == 0
    for b in (1, 2):          # a count above the capacity is clamped to it
        want = oracle.lightning(li.keys[b], li.scale[b], li.q[b], li.w[b], surv[b])
        tol = _bound(li.keys[b], li.scale[b], li.q[b], li.w[b], surv[b])
        assert (np.abs(score[b].astype(np.float64) - want) <= tol).all()
        assert tcount[b] == k


@pytest.mark.parametrize("name", ["ctx128k", "ctx1m"])
def test_lightning_top_k_after_a_trigger(name):
    # the GPU trigger's survivors ranked by the fine-grained score, against the
    # oracle's survivors ranked by the oracle's score: equal top-k sets except
    # the entries inside the threshold band (whose survivor status may
    # differ; widened by the query-rounding margin) and the k-th band
    from sparse_kv_cache_lsa_amd.pipeline import TriggerBuffers, pack_weights, run_trigger
    from test_gpu_chain import OracleQueries, _key_abs as chain_key_abs
    from gpu_util import bf16_host
    w = gen.WORKLOADS[name]
    inp = gen.indexer_inputs(w, gen.load_calibration(w), threads=16)
    li = gen.lightning_inputs(w, threads=16)
    d = gen.to_device(inp, DEV)
    buf = TriggerBuffers.allocate(w.L, w.B, w.N, w.H, w.dI, w.k, w.row_elems, device=DEV)
    run_trigger(buf, d["h"], d["Wq"], d["Wg"], d["keys"], d["scale"], d["bias"], None,
                packed=pack_weights(d["Wq"], d["Wg"]))
    score = torch.empty((w.B, w.N), dtype=torch.float32, device=DEV)
    lsa.lsa_lightning_score(dev(li.keys), None if li.scale is None else dev(li.scale),
                            dev(li.q), dev(li.w), buf.surv_idx, buf.surv_count, score)
    lsa.lsa_topk(buf.surv_idx, score, buf.surv_count, buf.topk_idx, buf.topk_count, buf.ws_topk)
    torch.cuda.synchronize()
    top, tcount = host(buf.topk_idx), host(buf.topk_count)
    qg = bf16_host(buf.q)
    # the pipeline's fine-grained option gives the same trigger
    buf2 = TriggerBuffers.allocate(w.L, w.B, w.N, w.H, w.dI, w.k, w.row_elems, device=DEV)
    score2 = torch.empty_like(score)
    run_trigger(buf2, d["h"], d["Wq"], d["Wg"], d["keys"], d["scale"], d["bias"], None,
                packed=pack_weights(d["Wq"], d["Wg"]),
                fine=(dev(li.keys), None if li.scale is None else dev(li.scale), dev(li.q),
                      dev(li.w), score2))
    torch.cuda.synchronize()
    assert torch.equal(buf2.topk_idx, buf.topk_idx) and torch.equal(buf2.topk_count, buf.topk_count)
    oq = OracleQueries(inp)
    for b in range(w.B):
        q_or, g_or, a, S = oq.request(b)
        E = np.zeros((w.L, w.N))
        for l in range(w.L):
            sig = None if inp.scale[l] is None else inp.scale[l][b]
            E[l], _ = parity.projection_flip_margin(q_or[l, b], qg[l, b], a[l], S[l], g_or[l, b],
                                                    chain_key_abs(inp, l, b), sig)
        z = np.stack([oracle.score(inp.keys[l][b], None if inp.scale[l] is None
                                   else inp.scale[l][b], q_or[l, b], g_or[l, b],
                                   float(inp.bias[l])) for l in range(w.L)])
        surv, _, _ = oracle.merge_compact(oracle.threshold(z), z)
        sc_b = None if li.scale is None else li.scale[b]
        want = oracle.lightning(li.keys[b], sc_b, li.q[b], li.w[b], surv)
        extra = np.zeros(w.N)
        extra[surv] = _bound(li.keys[b], sc_b, li.q[b], li.w[b], surv)
        unc = parity.uncertain_survivors(z, extra=E)
        nb = parity.check_topk(top[b], int(tcount[b]), surv, want, w.k, uncertain=unc,
                               extra=extra)
        print(name, b, "survivors", surv.size, "top-k band", nb, "uncertain", int(unc.sum()),
              flush=True)
