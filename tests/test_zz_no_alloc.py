"""lsa_topk_noalloc (the top-k that uses the library's own scratch array
instead of a caller workspace) against lsa_topk with a workspace, through the
C ABI: two calls in a row, the second on a smaller input, each bit-exact
against the workspace call and the oracle's top-k."""
import numpy as np
import pytest
import torch

import sparse_kv_cache_lsa_amd as lsa
from gpu_util import DEV, dev, host
from oracle import oracle

pytestmark = pytest.mark.gpu


def _lists(rng, B, cap, fill):
    """Ascending survivor lists of about fill * cap entries per request, with
    repeated logits (ties) mixed in."""
    idx = np.full((B, cap), -1, np.int32)
    z = np.full((B, cap), np.nan, np.float32)
    cnt = np.zeros(B, np.int32)
    for b in range(B):
        n = int(cap * fill) - 37 * b
        s = np.sort(rng.choice(4 * cap, n, replace=False)).astype(np.int32)
        v = rng.standard_normal(n).astype(np.float32) * 8
        v[rng.random(n) < 0.1] = 1.5                 # ties, broken by lower index
        idx[b, :n], z[b, :n], cnt[b] = s, v, n
    return idx, z, cnt


def _both(idx, z, cnt, k):
    B, cap = idx.shape
    si, sz, sc = dev(idx), dev(z), dev(cnt)
    t1 = torch.full((B, k), -9, dtype=torch.int32, device=DEV)
    c1 = torch.full((B,), -9, dtype=torch.int32, device=DEV)
    t2 = torch.full((B, k), -9, dtype=torch.int32, device=DEV)
    c2 = torch.full((B,), -9, dtype=torch.int32, device=DEV)
    ws = torch.empty((max(1, lsa.lsa_topk_workspace_bytes(B, cap, k)),), dtype=torch.uint8,
                     device=DEV)
    lsa.lsa_topk(si, sz, sc, t1, c1, ws)
    lsa.lsa_topk_noalloc(si, sz, sc, t2, c2)
    torch.cuda.synchronize()
    return host(t1), host(c1), host(t2), host(c2)


def test_noalloc_topk_matches_workspace_topk_twice():
    rng = np.random.default_rng(77)
    for B, cap, fill, k in [(8, 100_000, 0.6, 2048), (3, 40_000, 0.9, 512)]:
        idx, z, cnt = _lists(rng, B, cap, fill)
        assert lsa.lsa_topk_workspace_bytes(B, cap, k) > 0     # the two-stage path
        assert lsa.lsa_topk_workspace_bytes(B, cap, k) <= lsa.LSA_TOPK_NOALLOC_MAX_BYTES
        t1, c1, t2, c2 = _both(idx, z, cnt, k)
        assert np.array_equal(t1, t2) and np.array_equal(c1, c2)
        for b in range(B):
            n = int(cnt[b])
            want, wc = oracle.topk(idx[b, :n], z[b, :n].astype(np.float64), k)
            assert c2[b] == wc and np.array_equal(t2[b, :wc], want)
            assert (t2[b, wc:] == -1).all()
        print(f"B={B} cap={cap} k={k}: equal to lsa_topk and the oracle")


def test_noalloc_topk_short_lists_need_no_scratch():
    rng = np.random.default_rng(78)
    idx, z, cnt = _lists(rng, 4, 3000, 0.5)
    assert lsa.lsa_topk_workspace_bytes(4, 3000, 256) == 0
    t1, c1, t2, c2 = _both(idx, z, cnt, 256)
    assert np.array_equal(t1, t2) and np.array_equal(c1, c2)
