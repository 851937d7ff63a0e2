"""Parity of lsa_label_vote (softmax -> per-layer nucleus -> majority vote)
with the oracle, through the C ABI.

Per-layer selections are bit-exact except entries whose oracle mass ahead
lies within TOPP_BAND of top_p (the GPU sums mass in 64-bit fixed point, the
oracle in fp64); vote counts are bit-exact where no layer of the entry is in
that band; labels are bit-exact where the band cannot change the outcome.
The GPU's own count and label must always agree with its own masks."""
import numpy as np
import pytest
import torch

import lsa_inputs as gen
import parity
import sparse_kv_cache_lsa_amd as lsa
from gpu_util import DEV, dev, host
from oracle import oracle

pytestmark = pytest.mark.gpu


def _gpu(x, top_p, theta, with_mask=True):
    Q, L, N = x.shape
    W = (N + 31) // 32
    count = torch.full((Q, N), 0xEE, dtype=torch.uint8, device=DEV)
    label = torch.full((Q, N), 0xEE, dtype=torch.uint8, device=DEV)
    mask = torch.empty((Q, L, W), dtype=torch.int32, device=DEV) if with_mask else None
    ws = None
    if not with_mask:
        ws = torch.empty(lsa.lsa_label_vote_workspace_bytes(Q, L, N), dtype=torch.uint8, device=DEV)
    lsa.lsa_label_vote(dev(x), top_p, theta, count, label, layer_mask=mask, ws=ws)
    torch.cuda.synchronize()
    return (host(mask) if with_mask else None), host(count), host(label)


def _check(x, top_p, theta, mask, count, label):
    """Compare one GPU result with the oracle; returns the excluded counts."""
    Q, L, N = x.shape
    p = float(np.float32(top_p))     # the value the kernel receives
    n_band = 0
    for q in range(Q):
        sel_or = np.empty((L, N), np.uint8)
        band = np.zeros((L, N), bool)
        sel_gpu = parity.unpack_mask(mask[q], N) if mask is not None else None
        for l in range(L):
            s, _, A = oracle.nucleus(x[q, l], p, want_mass=True)
            sel_or[l] = s
            band[l] = np.abs(A - p) <= parity.TOPP_BAND
            if sel_gpu is not None:
                bad = (sel_gpu[l] != s.astype(bool)) & ~band[l]
                assert not bad.any(), (q, l, np.nonzero(bad)[0][:10])
        n_band += int(band.sum())
        if sel_gpu is not None:
            own = sel_gpu.sum(0)
            assert np.array_equal(count[q], own)
        assert np.array_equal(label[q], (count[q].astype(np.int64) >= theta).astype(np.uint8))
        c_or, y_or = oracle.vote(sel_or, theta)
        free = ~band.any(0)
        assert np.array_equal(count[q][free], c_or[free])
        certain_in = (sel_or.astype(bool) & ~band).sum(0)
        nb = band.sum(0)
        decided = (certain_in >= theta) | (certain_in + nb < theta)
        assert np.array_equal(label[q][decided], y_or[decided])
    return n_band


def test_labels_full_workload():
    w = gen.LABELS
    x = np.stack([gen.teacher_logits(w, q) for q in range(w.Q)])
    mask, count, label = _gpu(x, w.top_p, w.theta)
    nb = _check(x, w.top_p, w.theta, mask, count, label)
    frac = label.mean()
    print(f"labels: positive fraction {frac:.4f}, band entries {nb}")
    assert 0.01 < frac < 0.2
    # same result through the workspace path, and deterministic
    _, count2, label2 = _gpu(x, w.top_p, w.theta, with_mask=False)
    assert np.array_equal(count2, count) and np.array_equal(label2, label)


@pytest.mark.parametrize("Q,L,N", [(2, 1, 1), (2, 3, 31), (1, 3, 32), (3, 5, 1000),
                                   (2, 3, 4097), (2, 3, 16384), (1, 3, 16385), (2, 2, 30001),
                                   (1, 2, 32773), (1, 2, 65536)])
def test_labels_ragged_sizes(Q, L, N):
    rng = np.random.default_rng(N + 10 * L)
    x = rng.standard_normal((Q, L, N)).astype(np.float32) * 2
    mask, count, label = _gpu(x, 0.6, min(3, L))
    _check(x, 0.6, min(3, L), mask, count, label)


@pytest.mark.parametrize("N", [5000, 20000])
@pytest.mark.parametrize("top_p", [1e-6, 0.05, 0.6, 0.999, 1.0])
def test_labels_top_p_extremes(top_p, N):
    # top_p near 1 puts the crossing in the last value bin, where the padding
    # of a ragged row's last thread also falls (weight 0, never kept)
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, 4, N)).astype(np.float32) * 3
    mask, count, label = _gpu(x, top_p, 2)
    _check(x, top_p, 2, mask, count, label)


def test_labels_constant_logits_closed_form():
    # every entry has mass 1/N: the layer keeps exactly the lowest ceil(pN) indices
    N = 32768
    x = np.full((1, 3, N), 0.25, np.float32)
    mask, count, label = _gpu(x, 0.6, 3)
    sel = parity.unpack_mask(mask[0], N)
    n_keep = int(np.ceil(float(np.float32(0.6)) * N))
    assert n_keep == 19661
    for l in range(3):
        assert sel[l, :n_keep].all() and not sel[l, n_keep:].any()
    assert np.array_equal(count[0], np.where(np.arange(N) < n_keep, 3, 0))


@pytest.mark.parametrize("N", [9000, 20000, 50000])
def test_labels_heavy_ties_and_signed_zeros(N):
    # few distinct values: the crossing bin holds thousands of entries and
    # takes the radix path (32 entries a thread up to 16K, 64 above)
    rng = np.random.default_rng(11)
    x = (np.round(rng.standard_normal((2, 3, N)) * 2) / 2).astype(np.float32)
    z = rng.random(x.shape) < 0.1
    x[z] = np.where(rng.random(z.sum()) < 0.5, np.float32(0.0), np.float32(-0.0))
    for theta in (0, 1, 3):
        mask, count, label = _gpu(x, 0.6, theta)
        _check(x, 0.6, theta, mask, count, label)
        if theta == 0:
            assert label.all()


@pytest.mark.parametrize("N", [32768, 5000, 65536])
def test_labels_large_offsets(N):
    # rows whose values are large against their spread (3e5 + N(0,1), 1e6 + ...):
    # the value bins come from max * inv rounded before the subtraction, so
    # the largest entries' bin value can fall below 0 and must be clamped
    rng = np.random.default_rng(N + 5)
    offs = np.array([0.0, 1e3, 3e5, 1e6, -1e6, 2e7], np.float64)
    x = np.stack([np.stack([offs[(q * 3 + l) % len(offs)] + rng.standard_normal(N) * (1 + l)
                            for l in range(3)]) for q in range(2)]).astype(np.float32)
    for top_p in (0.05, 0.6, 0.999):
        mask, count, label = _gpu(x, top_p, 2)
        _check(x, top_p, 2, mask, count, label)
