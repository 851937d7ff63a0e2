"""Pins of the oracle's decode session over a growing key cache: a
hand-worked session, closed forms of the trigger cadence and cache growth,
and the invariants the reuse of resident rows fixes."""
import math

import numpy as np
import pytest

import lsa_inputs as gen


def _bf(x):
    return gen.to_bf16_bits(np.asarray(x, np.float32))


def test_hand_worked_session(oracle):
    # one layer, one head, dI = 2, g = 1, bias -0.5: z = q . k - 0.5.
    # Entries (k0, k1): 0:(1,0) 1:(-1,0) 2:(2,0) 3:(0,1) 4:(3,0) 5:(-2,0)
    keys = [_bf([[1, 0], [-1, 0], [2, 0], [0, 1], [3, 0], [-2, 0]])]
    qs = [_bf([[[1, 0]]]), _bf([[[1, 0]]]), _bf([[[0, 1]]])]
    g = np.ones((1, 1), np.float32)
    rows = np.arange(6 * 16, dtype=np.uint8).reshape(6, 16)
    # tau 8, one entry per window, 3 entries at step 0, steps [0, 17):
    # triggers at 0, 8, 16 over 3, 4 and 5 entries
    rec = oracle.stream_session(keys, None, lambda i: (qs[i], g), [-0.5], N0=3, tau=8, T=17,
                                per_window=1, k=1, cold=rows, S=3)
    assert [r["step"] for r in rec] == [0, 8, 16]
    assert [r["N"] for r in rec] == [3, 4, 5]
    # trigger 0 over entries 0..2 with q=(1,0): z = 0.5, -1.5, 1.5
    r = rec[0]
    assert r["survivors"].tolist() == [0, 2] and r["zstar"].tolist() == [0.5, 1.5]
    assert r["topk"].tolist() == [2] and r["fetched"] == 2
    assert r["entry_of"].tolist() == [0, 2, -1]
    assert np.array_equal(r["hot"], rows[[2]])
    # trigger 1 over entries 0..3: entry 3 has z = -0.5, nothing new survives
    r = rec[1]
    assert r["survivors"].tolist() == [0, 2] and r["fetched"] == 0
    # trigger 2 over entries 0..4 with q=(0,1): only entry 3 (z = 0.5)
    r = rec[2]
    assert r["survivors"].tolist() == [3] and r["topk"].tolist() == [3]
    assert r["fetched"] == 1 and r["entry_of"].tolist() == [3, -1, -1]
    assert r["slot_of"].tolist() == [-1, -1, -1, 0, -1, -1]
    assert np.array_equal(r["hot"], rows[[3]])


@pytest.mark.parametrize("tau,T,per_window", [(64, 704, 16), (64, 1, 16), (64, 65, 16),
                                              (16, 100, 4)])
def test_cadence_and_growth_closed_forms(oracle, tau, T, per_window):
    rng = np.random.default_rng(tau + T)
    N0, dI, H = 40, 8, 2
    n_trig = math.ceil(T / tau)
    N_cap = N0 + per_window * n_trig
    keys = [_bf(rng.standard_normal((N_cap, dI)))]
    qg = (_bf(rng.standard_normal((1, H, dI))), rng.uniform(0.2, 1, (1, H)).astype(np.float32))
    rec = oracle.stream_session(keys, None, lambda i: qg, [0.0], N0=N0, tau=tau, T=T,
                                per_window=per_window, k=5)
    assert len(rec) == n_trig
    assert [r["step"] for r in rec] == [tau * i for i in range(n_trig)]
    assert [r["N"] for r in rec] == [N0 + per_window * i for i in range(n_trig)]
    for r in rec:
        assert r["survivors"].size == 0 or r["survivors"].max() < r["N"]


def test_resident_set_follows_the_survivors(oracle):
    # every trigger leaves exactly its survivors resident, copies only the
    # survivors the previous trigger did not have, and its hot rows are the
    # cold-pool rows of its top-k
    rng = np.random.default_rng(11)
    N0, dI, H, L, per_window, tau, T = 300, 16, 4, 2, 16, 64, 64 * 12
    N_cap = N0 + per_window * 12
    keys = [_bf(rng.standard_normal((N_cap, dI))) for _ in range(L)]
    cold = rng.integers(0, 256, (N_cap, 32), dtype=np.uint8)
    qs = [(_bf(rng.standard_normal((L, H, dI))), rng.uniform(0.2, 1, (L, H)).astype(np.float32))
          for _ in range(12)]
    rec = oracle.stream_session(keys, None, lambda i: qs[i], [-0.3, -0.2], N0=N0, tau=tau, T=T,
                                per_window=per_window, k=20, cold=cold, S=N_cap)
    prev = set()
    for r in rec:
        surv = set(r["survivors"].tolist())
        assert set(np.nonzero(r["slot_of"] >= 0)[0].tolist()) == surv
        assert r["fetched"] == len(surv - prev)
        assert np.array_equal(r["hot"], cold[r["topk"][:r["kcount"]]])
        prev = surv
    # a trigger is the single-trigger chain on the cache prefix
    r = rec[7]
    z = np.stack([oracle.score(keys[l][:r["N"]], None, qs[7][0][l], qs[7][1][l], b)
                  for l, b in zip(range(L), (-0.3, -0.2))])
    assert np.array_equal(z, r["z"])
