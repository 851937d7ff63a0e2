"""Pins of the oracle's OR-merge/compaction (O5), top-k (O6) and gather (O7)
against brute force, library routines and the invariants the method fixes."""
import itertools

import numpy as np
import pytest
import torch


# ------------------------------------------------------------- OR + compact

def test_merge_matches_numpy_union(oracle):
    rng = np.random.default_rng(20)
    L, N = 3, 500
    z = rng.standard_normal((L, N)) * 3 - 2
    sel = oracle.threshold(z)
    idx, zs, count = oracle.merge_compact(sel, z)
    want = np.nonzero(sel.any(axis=0))[0]
    assert count == want.size
    assert np.array_equal(idx, want)
    np.testing.assert_array_equal(zs, z[:, want].max(axis=0))
    # union = {s : max_l z_l >= 0}, every layer's selection inside it
    assert np.array_equal(idx, np.nonzero(z.max(axis=0) >= 0)[0])
    for l in range(L):
        assert set(np.nonzero(sel[l])[0]) <= set(idx.tolist())
    assert (np.diff(idx) > 0).all()


def test_merge_special_cases(oracle):
    rng = np.random.default_rng(21)
    N = 300
    z1 = rng.standard_normal((1, N))
    s1 = oracle.threshold(z1)
    idx, _, c = oracle.merge_compact(s1, z1)
    assert np.array_equal(idx, np.nonzero(s1[0])[0]) and c == s1.sum()   # L=1: identity
    z3 = np.repeat(z1, 3, axis=0)
    idx3, zs3, c3 = oracle.merge_compact(oracle.threshold(z3), z3)
    assert np.array_equal(idx3, idx) and c3 == c                         # identical layers
    zb = z1 + 1e6
    assert oracle.merge_compact(oracle.threshold(zb), zb)[2] == N         # bias -> +inf
    zb = z1 - 1e6
    assert oracle.merge_compact(oracle.threshold(zb), zb)[2] == 0         # bias -> -inf


def test_merge_capacity_overflow_reports_true_count(oracle):
    z = np.ones((2, 50))
    idx, zs, count = oracle.merge_compact(oracle.threshold(z), z, cap=7)
    assert count == 50 and idx.tolist() == list(range(7))


def test_merge_nan_layer_ignored_in_max(oracle):
    z = np.array([[np.nan, 1.0], [2.0, np.nan]])
    sel = oracle.threshold(z)
    idx, zs, count = oracle.merge_compact(sel, z)
    assert idx.tolist() == [0, 1] and zs.tolist() == [2.0, 1.0]


# -------------------------------------------------------------------- top-k

def _brute_topk(idx, z, k):
    """Enumerate all k-subsets; return the one whose members all rank ahead
    of all non-members under (z desc, index asc)."""
    n = len(idx)
    if k >= n:
        return sorted(idx)
    ahead = lambda a, b: z[a] > z[b] or (z[a] == z[b] and idx[a] < idx[b])
    found = []
    for comb in itertools.combinations(range(n), k):
        inside = set(comb)
        if all(ahead(a, b) for a in inside for b in range(n) if b not in inside):
            found.append(sorted(idx[a] for a in comb))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_small(oracle, seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 13))
    idx = np.sort(rng.choice(1000, n, replace=False)).astype(np.int32)
    z = rng.integers(0, 4, n).astype(np.float64)        # many ties on purpose
    for k in range(0, n + 2):
        out, cnt = oracle.topk(idx, z, k)
        want = _brute_topk(list(idx), list(z), k)
        assert cnt == min(k, n)
        assert out[:cnt].tolist() == want
        assert (out[cnt:] == -1).all()


def test_topk_matches_torch_stable_sort(oracle):
    rng = np.random.default_rng(30)
    n, k = 5000, 300
    idx = np.sort(rng.choice(100_000, n, replace=False)).astype(np.int32)
    z = np.round(rng.standard_normal(n) * 4, 1)            # ties
    out, cnt = oracle.topk(idx, z, k)
    order = torch.sort(torch.from_numpy(z), descending=True, stable=True).indices[:k].numpy()
    assert out.tolist() == sorted(idx[order].tolist())
    assert set(out.tolist()) <= set(idx.tolist())


def test_topk_all_equal_takes_lowest_indices(oracle):
    idx = np.arange(10, 110, 2, dtype=np.int32)
    out, cnt = oracle.topk(idx, np.full(idx.size, 3.5), 7)
    assert out.tolist() == idx[:7].tolist() and cnt == 7


def test_topk_empty_and_k_above_n(oracle):
    out, cnt = oracle.topk(np.zeros(0, np.int32), np.zeros(0), 4)
    assert cnt == 0 and out.tolist() == [-1] * 4
    out, cnt = oracle.topk(np.array([5, 9], np.int32), np.array([1.0, 2.0]), 4)
    assert cnt == 2 and out.tolist() == [5, 9, -1, -1]


# ------------------------------------------------------------------- gather

def test_gather_matches_numpy_indexing(oracle):
    rng = np.random.default_rng(40)
    pool = rng.integers(0, 256, (64, 48), dtype=np.uint8)
    idx = np.array([3, -1, 63, 0, 3], np.int32)
    hot = oracle.gather(pool, idx)
    want = pool[np.maximum(idx, 0)].copy()
    want[idx < 0] = 0
    assert np.array_equal(hot, want)
    # gather is composable: gathering a gathered pool by positions gives the
    # rows the composed index picks
    pos = np.array([4, 0, 2], np.int32)
    assert np.array_equal(oracle.gather(hot, pos), oracle.gather(pool, idx[pos]))
