"""Parity of lsa_select_or_compact (OR merge + ascending compaction) with
the oracle.  Integer work: bit-exact, including the merged fp32 maxima."""
import numpy as np
import pytest
import torch

import sparse_kv_cache_lsa_amd as lsa
import parity
from gpu_util import DEV, dev, host
from oracle import oracle

pytestmark = pytest.mark.gpu


def _pack(sel):
    """bool [..., N] -> int32 words [..., ceil(N/32)] (bit s%32 of word s//32)."""
    N = sel.shape[-1]
    W = (N + 31) // 32
    pad = np.zeros(sel.shape[:-1] + (W * 32,), bool)
    pad[..., :N] = sel
    b = np.packbits(pad.reshape(*sel.shape[:-1], W, 32), axis=-1, bitorder="little")
    return np.ascontiguousarray(b).view(np.int32).reshape(*sel.shape[:-1], W)


def _run(mask, z, cap):
    L, B, N = z.shape
    si = torch.full((B, max(cap, 1)), -7, dtype=torch.int32, device=DEV)
    sz = torch.full((B, max(cap, 1)), -7.0, dtype=torch.float32, device=DEV)
    sc = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    ws = torch.empty((max(1, lsa.lsa_select_or_compact_workspace_bytes(L, B, N)),),
                     dtype=torch.uint8, device=DEV)
    lsa.lsa_select_or_compact(dev(mask), dev(z), si[:, :cap] if cap else si[:, :0].contiguous(),
                              sz[:, :cap] if cap else sz[:, :0].contiguous(), sc, ws)
    torch.cuda.synchronize()
    return host(si), host(sz), host(sc)


@pytest.mark.parametrize("L,B,N", [(3, 4, 1), (3, 4, 31), (3, 4, 32), (3, 2, 1000),
                                   (3, 2, 8192), (3, 2, 8193), (3, 3, 40000), (1, 1, 70000),
                                   (5, 2, 12345)])
@pytest.mark.parametrize("consistent", [True, False])
def test_select_matches_oracle(L, B, N, consistent):
    rng = np.random.default_rng(N * 7 + L)
    z = (rng.standard_normal((L, B, N)) * 3 - 2.5).astype(np.float32)
    sel = (z >= 0) if consistent else (rng.random((L, B, N)) < 0.15)
    si, sz, sc = _run(_pack(sel), z, N)
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
    si = torch.full((B, cap + 5), -7, dtype=torch.int32, device=DEV)
    sz = torch.full((B, cap + 5), -7.0, dtype=torch.float32, device=DEV)
    sc = torch.empty((B,), dtype=torch.int32, device=DEV)
    ws = torch.empty((lsa.lsa_select_or_compact_workspace_bytes(L, B, N),), dtype=torch.uint8,
                     device=DEV)
    # the output rows are cap wide: pass views of the first cap columns of a
    # wider buffer would not be contiguous, so use separate exact-size tensors
    si_c = si[:, :cap].contiguous()
    sz_c = sz[:, :cap].contiguous()
    lsa.lsa_select_or_compact(dev(_pack(sel)), dev(z), si_c, sz_c, sc, ws)
    torch.cuda.synchronize()
    for b in range(B):
        idx, zs, count = oracle.merge_compact(sel[:, b].astype(np.uint8), z[:, b].astype(np.float64),
                                              cap=cap)
        assert host(sc)[b] == count > cap
        assert np.array_equal(host(si_c)[b], idx)
        assert np.array_equal(host(sz_c)[b].astype(np.float64), zs)


def test_select_nan_layer_is_ignored_in_the_max():
    z = np.array([[[np.nan, 1.0, -1.0]], [[2.0, np.nan, np.nan]]], np.float32)
    sel = np.array([[[0, 1, 0]], [[1, 0, 0]]], bool)
    si, sz, sc = _run(_pack(sel), z, 3)
    assert sc[0] == 2 and si[0, :2].tolist() == [0, 1] and sz[0, :2].tolist() == [2.0, 1.0]


def test_select_n_zero_sets_zero_counts():
    z = np.zeros((3, 4, 0), np.float32)
    sc = torch.full((4,), 9, dtype=torch.int32, device=DEV)
    lsa.lsa_select_or_compact(torch.zeros((3, 4, 0), dtype=torch.int32, device=DEV), dev(z),
                              torch.empty((4, 0), dtype=torch.int32, device=DEV),
                              torch.empty((4, 0), dtype=torch.float32, device=DEV), sc,
                              torch.empty((1,), dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    assert host(sc).tolist() == [0, 0, 0, 0]
