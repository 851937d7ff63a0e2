"""Parity of lsa_topk and lsa_gather_hot with the oracle (bit-exact: both
rank the same fp32 values, and the gather is a byte copy)."""
import numpy as np
import pytest
import torch

import sparse_kv_cache_lsa_amd as lsa
from gpu_util import DEV, dev, host
from oracle import oracle

pytestmark = pytest.mark.gpu


def _survivors(rng, B, cap, ns, N=None, ties=False):
    N = max(300_000, 2 * cap) if N is None else N
    idx = np.full((B, cap), -9, np.int32)
    z = np.full((B, cap), np.nan, np.float32)
    for b, n in enumerate(ns):
        n = min(n, cap)
        idx[b, :n] = np.sort(rng.choice(N, n, replace=False))
        v = rng.standard_normal(n) * 20 + 30
        if ties:
            v = np.round(v)          # many exact ties
        z[b, :n] = v.astype(np.float32)
    return idx, z


def _topk(idx, z, counts, k):
    B, cap = idx.shape
    out = torch.full((B, max(k, 1)), -5, dtype=torch.int32, device=DEV)
    oc = torch.full((B,), -5, dtype=torch.int32, device=DEV)
    o = out[:, :k].contiguous() if k else torch.empty((B, 0), dtype=torch.int32, device=DEV)
    nws = lsa.lsa_topk_workspace_bytes(B, cap, k)
    # stale workspace contents must not matter: fill it with garbage first
    ws = torch.full((max(nws, 1),), 0x5A, dtype=torch.uint8, device=DEV) if nws else None
    lsa.lsa_topk(dev(idx), dev(z), dev(np.asarray(counts, np.int32)), o, oc, ws)
    torch.cuda.synchronize()
    return host(o), host(oc)


@pytest.mark.parametrize("ns,k", [
    ([0, 1, 5], 4),
    ([100, 2048, 2049], 2048),
    ([10000, 63000, 4097], 2048),
    ([70000, 3, 2], 256),
    ([81920, 81921, 40001], 2048),
    ([100000, 5, 9], 512),
    ([17000, 3], 20000),
    ([16384, 16385, 16383], 1000),
    ([530000, 10], 2048),
    ([500, 600, 700], 1),
    ([5000, 5000, 5000], 0),
    ([1 << 24, 7], 2048),   # a request as long as the score call allows (4,096 slices)
])
@pytest.mark.parametrize("ties", [False, True])
def test_topk_matches_oracle(ns, k, ties):
    rng = np.random.default_rng(sum(ns) + k + ties)
    cap = max(max(ns), 1)
    idx, z = _survivors(rng, len(ns), cap, ns, ties=ties)
    out, oc = _topk(idx, z, ns, k)
    for b, n in enumerate(ns):
        want, cnt = oracle.topk(idx[b, :n], z[b, :n].astype(np.float64), k)
        assert oc[b] == cnt
        assert np.array_equal(out[b], want), f"request {b}"


@pytest.mark.parametrize("cap", [3000, 30000])
def test_topk_count_above_capacity_uses_capacity(cap):
    rng = np.random.default_rng(5)
    idx, z = _survivors(rng, 2, cap, [cap, cap])
    out, oc = _topk(idx, z, [99999, cap], 1000)
    for b in range(2):
        want, cnt = oracle.topk(idx[b], z[b].astype(np.float64), 1000)
        assert np.array_equal(out[b], want) and oc[b] == cnt


def test_topk_signed_zero_ties_and_equal_scores():
    idx = np.arange(10, 30, dtype=np.int32).reshape(1, 20) * 3
    z = np.zeros((1, 20), np.float32)
    z[0, ::2] = -0.0
    out, oc = _topk(idx, z, [20], 7)
    assert out[0].tolist() == idx[0, :7].tolist()      # all equal: lowest indices
    z2 = np.full((1, 20), 5.0, np.float32)
    z2[0, 13] = 6.0
    out, _ = _topk(idx, z2, [20], 3)
    assert out[0].tolist() == sorted([idx[0, 13], idx[0, 0], idx[0, 1]])


# Long lists are cut into slices of 4096 survivors that keep their best 256
# when k is larger; the final stage must notice when a slice may have lost
# members of the top-k (all its kept entries made the top-k) and redo the
# select over the whole list.  Each case makes that happen for some request.
@pytest.mark.parametrize("pattern", ["clustered", "equal", "exact256", "dense512", "short"])
def test_topk_truncated_slices_stay_exact(pattern):
    rng = np.random.default_rng(77)
    B, cap, k = 3, 63000, 2048
    ns = [63000, 40000, 20001]
    idx, z = _survivors(rng, B, cap, ns)
    for b, n in enumerate(ns):
        if pattern == "clustered":      # the best entries all in one slice
            lo = 4096 * b
            z[b, lo:lo + 3000] = (1000.0 - np.arange(3000)).astype(np.float32)
        elif pattern == "equal":        # one score everywhere: the first k positions win
            z[b, :n] = 7.0
        elif pattern in ("exact256", "dense512"):   # slice 1 holds 256 / 512 of the top-k
            m = 256 if pattern == "exact256" else 512
            z[b, :n] = rng.uniform(0, 1, n).astype(np.float32)
            top = np.concatenate([4096 + rng.choice(4096, m, replace=False),
                                  rng.choice(np.arange(8192, n), k - m, replace=False)])
            z[b, top] = (10.0 + rng.uniform(0, 1, k)).astype(np.float32)
        else:                           # the slices keep fewer than k entries in total
            ns[b] = [5000, 4097, 9000][b]
    out, oc = _topk(idx, z, ns, k)
    for b, n in enumerate(ns):
        want, cnt = oracle.topk(idx[b, :n], z[b, :n].astype(np.float64), k)
        assert oc[b] == cnt
        assert np.array_equal(out[b], want), f"{pattern}: request {b}"


@pytest.mark.parametrize("row_bytes", [1024, 48, 16])
def test_gather_matches_oracle(row_bytes):
    rng = np.random.default_rng(row_bytes)
    B, N, k = 3, 5000, 700
    pool = rng.integers(0, 256, (B, N, row_bytes), dtype=np.uint8)
    idx = rng.integers(-3, N + 3, (B, k)).astype(np.int32)
    idx[:, :5] = [-1, 0, N - 1, N, 2 * N]
    hot = torch.full((B, k, row_bytes), 0xAB, dtype=torch.uint8, device=DEV)
    lsa.lsa_gather_hot(dev(pool), dev(idx), hot)
    torch.cuda.synchronize()
    got = host(hot)
    for b in range(B):
        assert np.array_equal(got[b], oracle.gather(pool[b], idx[b]))


def test_gather_from_a_pool_past_4_gib():
    # two requests of 2^22 rows of 1 KiB: request 1's rows start at 4 GiB
    # from the pool base, so every row offset needs 64-bit arithmetic; the
    # rows read are random bytes (the rest of the pool is zero), the list
    # includes the first and last rows and indices outside [0, N)
    B, N, k, rb = 2, 1 << 22, 3000, 1024
    rng = np.random.default_rng(4096)
    idx = rng.integers(0, N, (B, k)).astype(np.int32)
    idx[:, :6] = [0, N - 1, N - 2, -1, N, 1]
    pool = np.zeros((B, N, rb), np.uint8)
    for b in range(B):
        rows = np.unique(idx[b][(idx[b] >= 0) & (idx[b] < N)])
        pool[b, rows] = rng.integers(0, 256, (rows.size, rb), dtype=np.uint8)
    hot = torch.full((B, k, rb), 0xAB, dtype=torch.uint8, device=DEV)
    lsa.lsa_gather_hot(dev(pool), dev(idx), hot)
    torch.cuda.synchronize()
    got = host(hot)
    for b in range(B):
        assert np.array_equal(got[b], oracle.gather(pool[b], idx[b])), f"request {b}"
