"""Parity of lsa_select_or_compact (concatenation of the per-chunk candidate
lists into one ascending survivor list) with the oracle's OR merge and
compaction.  Integer work: bit-exact, including the fp32 merged logits."""
import numpy as np
import pytest
import torch

import sparse_kv_cache_lsa_amd as lsa
from gpu_util import DEV, dev, host
from oracle import oracle

pytestmark = pytest.mark.gpu
CH = lsa.LSA_CAND_CHUNK


def _chunk_lists(sel, z):
    """Test-side input construction: the candidate lists lsa_score defines
    for a request -- per chunk the ascending entries some layer selects, and
    the max of z over the selecting layers."""
    L, N = sel.shape
    nch = (N + CH - 1) // CH
    ci = np.full((nch, CH), -1, np.int32)
    cz = np.full((nch, CH), np.nan, np.float32)
    cc = np.zeros(nch, np.int32)
    any_sel = sel.any(axis=0)
    zm = np.where(sel, z, -np.inf).max(axis=0).astype(np.float32)
    for c in range(nch):
        e = np.nonzero(any_sel[c * CH:(c + 1) * CH])[0] + c * CH
        ci[c, :e.size] = e
        cz[c, :e.size] = zm[e]
        cc[c] = e.size
    return ci, cz, cc


def _run(sel, z, cap):
    L, B, N = sel.shape
    lists = [_chunk_lists(sel[:, b], z[:, b]) for b in range(B)]
    ci = np.stack([x[0] for x in lists]).reshape(B, -1, CH)
    cz = np.stack([x[1] for x in lists]).reshape(B, -1, CH)
    cc = np.stack([x[2] for x in lists]).reshape(B, -1)
    si = torch.full((B, cap), -7, dtype=torch.int32, device=DEV)
    sz = torch.full((B, cap), -7.0, dtype=torch.float32, device=DEV)
    sc = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    lsa.lsa_select_or_compact(dev(ci), dev(cz), dev(cc), N, si, sz, sc)
    torch.cuda.synchronize()
    return host(si), host(sz), host(sc)


@pytest.mark.parametrize("L,B,N", [(3, 4, 1), (3, 4, 31), (3, 4, 4096), (3, 2, 1000),
                                   (3, 2, 8192), (3, 2, 8193), (3, 3, 40000), (1, 1, 70000),
                                   (5, 2, 12345)])
def test_select_matches_oracle(L, B, N):
    rng = np.random.default_rng(N * 7 + L)
    z = (rng.standard_normal((L, B, N)) * 3 - 2.5).astype(np.float32)
    sel = z >= 0
    si, sz, sc = _run(sel, z, N)
    for b in range(B):
        idx, zs, count = oracle.merge_compact(sel[:, b].astype(np.uint8), z[:, b].astype(np.float64))
        assert sc[b] == count
        assert np.array_equal(si[b, :count], idx)
        assert np.array_equal(sz[b, :count].astype(np.float64), zs)


def test_select_capacity_overflow_reports_true_count():
    rng = np.random.default_rng(3)
    L, B, N, cap = 3, 2, 20000, 1000
    z = rng.standard_normal((L, B, N)).astype(np.float32)
    sel = z >= 0
    si, sz, sc = _run(sel, z, cap)
    for b in range(B):
        idx, zs, count = oracle.merge_compact(sel[:, b].astype(np.uint8),
                                              z[:, b].astype(np.float64), cap=cap)
        assert sc[b] == count > cap
        assert np.array_equal(si[b], idx)
        assert np.array_equal(sz[b].astype(np.float64), zs)


def test_select_empty_chunks_and_no_survivors():
    L, B, N = 3, 2, 3 * CH + 5
    z = np.full((L, B, N), -1.0, np.float32)
    z[1, 0, 2 * CH + 3] = 4.0           # one survivor in the third chunk of request 0
    si, sz, sc = _run(z >= 0, z, 16)
    assert sc.tolist() == [1, 0] and si[0, 0] == 2 * CH + 3 and sz[0, 0] == 4.0


def test_select_n_zero_sets_zero_counts():
    sc = torch.full((4,), 9, dtype=torch.int32, device=DEV)
    e = lambda *sh: torch.empty(sh, dtype=torch.int32, device=DEV)
    lsa.lsa_select_or_compact(e(4, 0, CH), torch.empty((4, 0, CH), device=DEV), e(4, 0), 0,
                              e(4, 0), torch.empty((4, 0), device=DEV), sc)
    torch.cuda.synchronize()
    assert host(sc).tolist() == [0, 0, 0, 0]
