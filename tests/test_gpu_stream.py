"""A decode session over growing caches on the GPU (StreamingSession: the host
loop triggers at lsa_trigger_due(t, 64), appends the 16 entries of each
finished window with lsa_append_rows, scores the live prefix with
lsa_score_strided, fetches survivors into the resident set with reuse and
gathers the top-k rows), against the oracle's decode session, over 11
triggers.

Per trigger and request: the selections, survivors and top-k against the
oracle under the parity bands (with the margin for query elements the GPU
encoder rounded to the other bf16 neighbour); the resident set against the
GPU's own survivors (resident = survivors, rows copied = new survivors, hot
rows = cold rows of the top-k).  The fetch sequence is also replayed on the
GPU with the oracle's own survivor lists and compared with the oracle's slot
tables bit for bit.  Steps between triggers reuse the hot rows: the core
attention on them gives the same bits within a window."""
import numpy as np
import pytest
import torch

import lsa_inputs as gen
import lsa_fixtures as fx
import parity
import sparse_kv_cache_lsa_amd as lsa
from gpu_util import DEV, bf16_host, dev, host
from oracle import oracle
from sparse_kv_cache_lsa_amd.pipeline import ResidentSet, StreamingSession, pack_weights

pytestmark = pytest.mark.gpu

TAU, PER_WINDOW, N0, TRIGGERS = 64, 16, 32768, 11


def _workload():
    return gen.custom("stream128k", 95, B=2, L=3, N=N0 + PER_WINDOW * TRIGGERS, H=64, dI=128,
                      D=4096, k=2048, row_elems=512, planted=(0.10, 0.10, 0.10), core=0.05)


def test_decode_session_over_growing_caches():
    w = _workload()
    T = TAU * (TRIGGERS - 1) + 1          # steps [0, T): triggers at 0, 64, ..., 640
    inp = gen.indexer_inputs(w, fx.calibrate(w))
    hs = gen.drift_hidden(w, TRIGGERS)
    d = gen.to_device(inp, DEV)
    packed = pack_weights(d["Wq"], d["Wg"])
    pool = gen.pool_tensor(w, DEV)
    cold = torch.empty(pool.shape, dtype=pool.dtype, pin_memory=True)
    cold.copy_(pool)
    cold_np = cold.numpy().view(np.uint8).reshape(w.B, w.N, -1)
    S = w.N // 2
    sess = StreamingSession(w.L, w.B, w.N, w.H, w.dI, w.k, w.row_elems, S, cold, tau=TAU,
                            per_window=PER_WINDOW, device=DEV)
    sess.append([k[:, :N0].contiguous() for k in d["keys"]])
    torch.cuda.synchronize()

    def window(i):
        lo, hi = N0 + PER_WINDOW * (i - 1), N0 + PER_WINDOW * i
        return [k[:, lo:hi].contiguous() for k in d["keys"]], None

    # attention on the hot rows at a few steps of every window (one query)
    att = gen.attention_inputs(w.B, gen.ATT_HEADS, 0, gen.ATT_WINDOW, wid=96)
    aq, awin = dev(att.q), dev(att.win)
    aout = torch.empty((w.B, gen.ATT_HEADS, gen.ATT_ROW), dtype=torch.float32, device=DEV)
    nws = lsa.lsa_sparse_attention_workspace_bytes(w.B, gen.ATT_HEADS, gen.ATT_ROW, w.k,
                                                   gen.ATT_WINDOW)
    aws = torch.empty((max(1, nws),), dtype=torch.uint8, device=DEV)
    att_out = {}

    def on_step(t):
        if t % 32 == 5:
            lsa.lsa_sparse_attention(aq, sess.hot.view(torch.bfloat16), aout, gen.att_scale(),
                                     hot_count=sess.topk_count, win=awin, ws=aws)
            att_out[t] = aout.clone()

    snaps = []

    def on_trigger(i, t):
        torch.cuda.synchronize()
        snaps.append({"step": t, "N": sess.N, "q": bf16_host(sess.q), "g": host(sess.g),
                      "mask": host(sess._views()[0]),
                      "count": host(sess.surv_count),
                      "surv": [host(sess.surv_idx[b, :int(sess.surv_count[b])])
                               for b in range(w.B)],
                      "zs": [host(sess.surv_z[b, :int(sess.surv_count[b])]) for b in range(w.B)],
                      "topk": host(sess.topk_idx), "kcount": host(sess.topk_count),
                      "slot_of": host(sess.res.slot_of), "fetched": host(sess.res.fetch_count),
                      "hot": host(sess.hot)})

    n = sess.decode(T, lambda i: dev(hs[i]), packed, d["bias"], window, on_trigger, on_step)
    torch.cuda.synchronize()
    assert n == TRIGGERS == len(snaps)
    assert [s["step"] for s in snaps] == [TAU * i for i in range(TRIGGERS)]
    assert [s["N"] for s in snaps] == [N0 + PER_WINDOW * i for i in range(TRIGGERS)]
    # the hot rows are reused between triggers: the same attention output
    # within a window
    for t in att_out:
        t2 = t + 32
        if t2 in att_out and t // TAU == t2 // TAU:
            assert torch.equal(att_out[t], att_out[t2]), t

    wabs = [np.abs(gen.bf16_bits_to_f32(W)) for W in inp.Wq]
    for b in range(w.B):
        habs = [np.abs(gen.bf16_bits_to_f32(h[b])) for h in hs]
        proj = [[oracle.project(hs[i][b], inp.Wq[l], inp.Wg[l], w.H, w.dI, want_a=True)
                 for l in range(w.L)] for i in range(TRIGGERS)]
        rec = oracle.stream_session(
            [inp.keys[l][b] for l in range(w.L)], None,
            lambda i: (np.stack([p[0] for p in proj[i]]), np.stack([p[1] for p in proj[i]])),
            inp.bias, N0, TAU, T, PER_WINDOW, w.k, cold=cold_np[b], S=S)
        assert len(rec) == TRIGGERS
        prev = set()
        for i, (s, r) in enumerate(zip(snaps, rec)):
            N = r["N"]
            E = np.zeros((w.L, N))
            for l in range(w.L):
                q_or, g_or, a = proj[i][l]
                Sabs = (wabs[l] @ habs[i]).astype(np.float64).reshape(w.H, w.dI)
                E[l], _ = parity.projection_flip_margin(
                    q_or, s["q"][l, b], a, Sabs, g_or,
                    np.abs(gen.bf16_bits_to_f32(inp.keys[l][b][:N])))
                np.testing.assert_allclose(s["g"][l, b], g_or, rtol=1e-5, atol=1e-7)
                parity.check_selection(parity.unpack_mask(s["mask"][l, b], N), r["z"][l],
                                       extra=E[l])
            cnt = int(s["count"][b])
            unc = parity.check_survivors(s["surv"][b], cnt, r["z"], extra=E)
            parity.check_merged_scores(s["surv"][b], s["zs"][b], r["z"], extra=E)
            kc = int(s["kcount"][b])
            nb = parity.check_topk(s["topk"][b], kc, r["survivors"], r["zstar"], w.k,
                                   uncertain=parity.uncertain_survivors(r["z"], extra=E),
                                   extra=E.max(axis=0))
            # the resident set follows the GPU's own survivors
            surv = set(s["surv"][b].tolist())
            assert set(np.nonzero(s["slot_of"][b] >= 0)[0].tolist()) == surv
            assert int(s["fetched"][b]) == len(surv - prev)
            top = s["topk"][b][:kc]
            assert np.array_equal(s["hot"][b][:kc].view(np.uint8).reshape(kc, -1),
                                  cold_np[b][top])
            prev = surv
            print(f"request {b} trigger {i}: N {N}, survivors {cnt} ({cnt / N:.4f} of N), "
                  f"uncertain {unc}, top-k band {nb}, rows fetched {int(s['fetched'][b])}",
                  flush=True)
        _replay_fetch_with_oracle_survivors(w, b, rec, cold, cold_np, S)


def _replay_fetch_with_oracle_survivors(w, b, rec, cold, cold_np, S):
    """The oracle session's survivor lists, trigger after trigger, fetched on
    the GPU into a fresh resident set: slot tables and resident rows equal the
    oracle's after every trigger."""
    res = ResidentSet.allocate(1, w.N, S, w.row_elems, dtype=cold.dtype, device=DEV)
    res.rows.zero_()
    cold_b = cold[b:b + 1]
    o_rows = np.zeros((S, cold_np.shape[2]), np.uint8)
    o_slot = np.full(w.N, -1, np.int32)
    o_entry = np.full(S, -1, np.int32)
    for r in rec:
        surv = r["survivors"]
        idx = np.full((1, w.N), -1, np.int32)
        idx[0, :surv.size] = surv
        res.fetch(cold_b, dev(idx), dev(np.array([surv.size], np.int32)))
        torch.cuda.synchronize()
        assert int(host(res.fetch_count)[0]) == oracle.fetch(cold_np[b], surv, o_slot, o_entry,
                                                             o_rows)
        assert np.array_equal(host(res.slot_of)[0], o_slot)
        assert np.array_equal(host(res.entry_of)[0], o_entry)
        assert np.array_equal(host(res.rows)[0].view(np.uint8).reshape(S, -1), o_rows)
        assert np.array_equal(o_slot, r["slot_of"]) and np.array_equal(o_entry, r["entry_of"])


def test_append_rows_and_strided_score_prefix():
    # appending in pieces builds the same cache as one copy; scoring the
    # first N of a larger cache equals lsa_score on exactly those N entries
    rng = np.random.default_rng(12)
    L, B, N_cap, N, H, dI = 2, 3, 10000, 7777, 8, 64
    keys = [rng.integers(0, 1 << 16, (B, N_cap, dI), dtype=np.uint16) & 0xBFFF for _ in range(L)]
    cache = [torch.zeros((B, N_cap, dI), dtype=torch.bfloat16, device=DEV) for _ in range(L)]
    start = 0
    for piece in (5000, 1, 2000, 776):
        for l in range(L):
            lsa.lsa_append_rows(dev(keys[l][:, start:start + piece]), cache[l], start)
        start += piece
    torch.cuda.synchronize()
    for l in range(L):
        assert np.array_equal(bf16_host(cache[l])[:, :N], keys[l][:, :N])
        assert not bf16_host(cache[l])[:, N:].any()
    # e4m3 keys with their fp32 scales (4-byte rows)
    sc = rng.random((B, 300)).astype(np.float32)
    sdev = torch.zeros((B, 1000), dtype=torch.float32, device=DEV)
    lsa.lsa_append_rows(dev(sc), sdev, 17)
    torch.cuda.synchronize()
    assert np.array_equal(host(sdev)[:, 17:317], sc) and not host(sdev)[:, :17].any()
    q = torch.from_numpy(rng.standard_normal((L, B, H, dI)).astype(np.float32)).to(DEV).to(torch.bfloat16)
    g = torch.from_numpy(rng.uniform(0.1, 1, (L, B, H)).astype(np.float32)).to(DEV)
    bias = torch.tensor([-0.5, 0.25], device=DEV)
    from sparse_kv_cache_lsa_amd.pipeline import TriggerBuffers
    b1 = TriggerBuffers.allocate(L, B, N, H, dI, 16, device=DEV)
    b2 = TriggerBuffers.allocate(L, B, N, H, dI, 16, device=DEV)
    z1 = torch.empty((L, B, N), dtype=torch.float32, device=DEV)
    z2 = torch.empty_like(z1)
    lsa.lsa_score_strided(cache, None, q, g, bias, N, b1.mask, b1.cand_idx, b1.cand_z,
                          b1.cand_count, z1)
    lsa.lsa_score([c[:, :N].contiguous() for c in cache], None, q, g, bias, b2.mask,
                  b2.cand_idx, b2.cand_z, b2.cand_count, z2)
    torch.cuda.synchronize()
    assert torch.equal(z1, z2) and torch.equal(b1.mask, b2.mask)
    assert torch.equal(b1.cand_count, b2.cand_count)
