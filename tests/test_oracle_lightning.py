"""Pins of the oracle's fine-grained score inside the fetched set (the
Lightning-Indexer form: ReLU-gated heads with per-query weights over the
entry's own key): a library evaluation, exact small-integer arithmetic, the
ReLU's effect, the key scale, and the top-k it feeds."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import lsa_inputs as gen


def _bf(x):
    return gen.to_bf16_bits(np.asarray(x, np.float32))


@pytest.mark.parametrize("e4m3", [False, True])
def test_lightning_matches_torch_relu_form(oracle, e4m3):
    rng = np.random.default_rng(31 + e4m3)
    N, H, dI = 500, 16, 64
    x = (rng.standard_normal((N, dI)) / 8).astype(np.float32)
    if e4m3:
        keys, scale = gen.to_e4m3_rows(x)
        kf = torch.from_numpy(keys).view(torch.float8_e4m3fn).double() * torch.from_numpy(
            scale).double()[:, None]
    else:
        keys, scale = _bf(x), None
        kf = torch.from_numpy(gen.bf16_bits_to_f32(keys)).double()
    q = _bf(rng.standard_normal((H, dI)))
    w = rng.uniform(0, 1, H).astype(np.float32)
    idx = np.sort(rng.choice(N, 200, replace=False)).astype(np.int32)
    out = oracle.lightning(keys, scale, q, w, idx)
    Q = torch.from_numpy(gen.bf16_bits_to_f32(q)).double()
    ref = (torch.relu(kf[idx] @ Q.T) * torch.from_numpy(w).double()).sum(1)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_lightning_exact_small_integers(oracle):
    rng = np.random.default_rng(32)
    N, H, dI = 12, 3, 5
    kk = rng.integers(-3, 4, (N, dI))
    qq = rng.integers(-3, 4, (H, dI))
    ww = rng.integers(0, 4, H)
    out = oracle.lightning(_bf(kk), None, _bf(qq), ww.astype(np.float32), np.arange(N, dtype=np.int32))
    for s in range(N):
        want = sum(Fraction(int(ww[h])) * max(Fraction(0), sum(Fraction(int(qq[h, d] * kk[s, d]))
                                                           for d in range(dI)))
                   for h in range(H))
        assert out[s] == float(want)


def test_lightning_relu_and_scale(oracle):
    dI = 4
    keys = _bf([[1, 0, 0, 0], [-1, 0, 0, 0], [2, 1, 0, 0]])
    q = _bf([[1, 0, 0, 0], [-1, 0, 0, 0]])
    w = np.array([1.0, 10.0], np.float32)
    out = oracle.lightning(keys, None, q, w, np.array([0, 1, 2], np.int32))
    # entry 0: head 0 sees +1, head 1 sees -1 (cut); entry 1: only head 1
    # (+1 x 10); entry 2: head 0 +2
    assert out.tolist() == [1.0, 10.0, 2.0]
    # a positive per-entry scale multiplies the score (relu(s x) = s relu(x))
    codes, sc = gen.to_e4m3_rows(np.array([[1, 0, 0, 0], [-1, 0, 0, 0]], np.float32))
    o1 = oracle.lightning(codes, sc, q, w, np.array([0, 1], np.int32))
    o2 = oracle.lightning(codes, sc * 4, q, w, np.array([0, 1], np.int32))
    np.testing.assert_array_equal(o2, 4 * o1)
    # one head, weight 1, every dot positive: the plain dot product
    assert oracle.lightning(keys, None, q[:1], np.ones(1, np.float32),
                            np.array([2], np.int32)).tolist() == [2.0]


def test_lightning_feeds_the_top_k(oracle):
    # the top-k over the survivors ranks by this score; entries are scored by
    # index, so a permuted index list gives the permuted scores
    rng = np.random.default_rng(33)
    N, H, dI = 300, 8, 32
    keys = _bf(rng.standard_normal((N, dI)) / 6)
    q = _bf(rng.standard_normal((H, dI)))
    w = rng.uniform(0, 1, H).astype(np.float32)
    surv = np.sort(rng.choice(N, 120, replace=False)).astype(np.int32)
    sc = oracle.lightning(keys, None, q, w, surv)
    perm = rng.permutation(surv.size)
    np.testing.assert_array_equal(oracle.lightning(keys, None, q, w, surv[perm]), sc[perm])
    top, kc = oracle.topk(surv, sc, 10)
    order = np.lexsort((surv, -sc))
    assert kc == 10 and top.tolist() == sorted(surv[order[:10]].tolist())
