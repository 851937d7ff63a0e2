"""Pins of the oracle's golden-label rule (O8: softmax, nucleus top-p, vote)
and of the student loss/gradient (O9)."""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import lsa_inputs as gen


# ------------------------------------------------------------------ nucleus

def test_nucleus_mass_matches_torch_softmax_sort_cumsum(oracle):
    rng = np.random.default_rng(50)
    x = np.round(rng.standard_normal(4000), 2).astype(np.float32)   # ties
    sel, n, mass = oracle.nucleus(x, 0.6, want_mass=True)
    pi = torch.softmax(torch.from_numpy(x.astype(np.float64)), 0)
    order = torch.sort(torch.from_numpy(x), descending=True, stable=True).indices
    ahead = torch.zeros_like(pi)
    ahead[order] = torch.cumsum(pi[order], 0) - pi[order]
    np.testing.assert_allclose(mass, ahead.numpy(), atol=1e-12)
    assert pi.sum().item() == pytest.approx(1.0, abs=1e-12)
    want = ahead.numpy() < 0.6
    band = np.abs(ahead.numpy() - 0.6) < 1e-12
    assert np.array_equal(sel.astype(bool)[~band], want[~band])
    assert n == sel.sum()


@pytest.mark.parametrize("N", [8, 1024, 32768])
def test_nucleus_constant_logits_closed_form(oracle, N):
    # equal logits: the order is by index, the mass ahead of entry j is j/N
    # (exact for N a power of two), so the nucleus is the lowest ceil(0.6 N)
    sel, n, mass = oracle.nucleus(np.full(N, 0.25, np.float32), 0.6, want_mass=True)
    want = math.ceil(0.6 * N)
    assert n == want and sel[:want].all() and not sel[want:].any()
    assert np.array_equal(mass, np.arange(N) / N)
    if N == 32768:
        assert n == 19661


@pytest.mark.parametrize("seed", range(5))
def test_nucleus_is_minimum_cardinality_set(oracle, seed):
    # brute force: the nucleus size is the smallest number of entries whose
    # probability mass reaches p, and the nucleus is such a set
    rng = np.random.default_rng(60 + seed)
    n = int(rng.integers(2, 15))
    x = (rng.standard_normal(n) * 2).astype(np.float32)
    p = float(rng.uniform(0.2, 0.95))
    sel, size = oracle.nucleus(x, p)
    pi = np.exp(x.astype(np.float64) - x.max())
    pi /= pi.sum()
    best = None
    for r in range(1, n + 1):
        if any(pi[list(c)].sum() >= p for c in itertools.combinations(range(n), r)):
            best = r
            break
    assert size == best
    assert pi[sel.astype(bool)].sum() >= p - 1e-12


def test_nucleus_exact_boundary(oracle):
    # equal logits, N = 8, p = 0.5: four entries carry exactly 0.5, so the
    # smallest set reaching p has four entries; the fifth has mass ahead = p
    sel, n = oracle.nucleus(np.full(8, -1.5, np.float32), 0.5)
    assert n == 4 and sel.tolist() == [1, 1, 1, 1, 0, 0, 0, 0]


def test_nucleus_crossing_entry_included(oracle):
    # masses 0.5, 0.3, 0.2: the second entry crosses 0.6 and is included
    x = np.log(np.array([0.5, 0.3, 0.2])).astype(np.float32)
    sel, n = oracle.nucleus(x, 0.6)
    assert sel.tolist() == [1, 1, 0]


# --------------------------------------------------------------------- vote

def test_vote_special_cases(oracle):
    rng = np.random.default_rng(70)
    L, N = 6, 400
    sel = (rng.random((L, N)) < 0.3).astype(np.uint8)
    c, y = oracle.vote(sel, 1)
    assert np.array_equal(y.astype(bool), sel.any(axis=0))                  # theta=1: union
    c, y = oracle.vote(sel, L)
    assert np.array_equal(y.astype(bool), sel.all(axis=0))                  # theta=L: intersection
    assert np.array_equal(c, sel.sum(axis=0))
    same = np.repeat(sel[:1], L, axis=0)
    c, _ = oracle.vote(same, 3)
    assert set(np.unique(c).tolist()) <= {0, L}                             # identical layers


def test_single_layer_noise_is_filtered(oracle):
    # The vote exists to drop what one layer alone asks for: an entry that
    # only layer 7 keeps (a large boost there, a very low logit in every other
    # layer) is counted once and is not a golden label at theta = 3, while an
    # entry that exactly theta layers keep is.
    rng = np.random.default_rng(71)
    L, N = 20, 2048
    x = rng.standard_normal((L, N)).astype(np.float32)
    x[:, 100] = -40.0
    x[7, 100] = 40.0
    x[:, 200] = -40.0
    x[[2, 9, 15], 200] = 40.0
    x[:, 300] = -40.0
    x[[4, 11], 300] = 40.0
    sel = np.stack([oracle.nucleus(x[l], 0.6)[0] for l in range(L)])
    c, y = oracle.vote(sel, 3)
    assert sel[:, 100].tolist() == [int(l == 7) for l in range(L)]
    assert c[100] == 1 and y[100] == 0
    assert c[300] == 2 and y[300] == 0
    assert c[200] == 3 and y[200] == 1


# --------------------------------------------------------------------- loss

def _tiny_student(rng, Q=2, N=8, D=4, H=2, dI=3):
    h = gen.to_bf16_bits(rng.standard_normal((Q, D)).astype(np.float32))
    Wq = (rng.standard_normal((H * dI, D)) / 2).astype(np.float32)
    Wg = (rng.standard_normal((H, D)) / 2).astype(np.float32)
    K = gen.to_bf16_bits(rng.standard_normal((N, dI)).astype(np.float32))
    y = (rng.random((Q, N)) < 0.4).astype(np.uint8)
    return h, Wq, Wg, K, y


@pytest.mark.parametrize("gamma", [0.0, 2.0])
def test_loss_gradient_matches_finite_differences(oracle, gamma):
    rng = np.random.default_rng(80)
    H, dI = 2, 3
    h, Wq, Wg, K, y = _tiny_student(rng, H=H, dI=dI)
    loss, dW, _ = oracle.focal_bce_grad(h, Wq, Wg, 0.3, K, y, gamma, H, dI)
    hf, Kf = gen.bf16_bits_to_f32(h).astype(np.float64), gen.bf16_bits_to_f32(K).astype(np.float64)
    W64 = Wq.astype(np.float64)
    assert loss == pytest.approx(oracle.focal_bce_loss64(hf, W64, Wg, 0.3, Kf, y, gamma, H, dI), rel=1e-14)
    eps = 1e-6
    for j in range(H * dI):
        for c in range(h.shape[1]):
            Wp, Wm = W64.copy(), W64.copy()
            Wp[j, c] += eps
            Wm[j, c] -= eps
            fd = (oracle.focal_bce_loss64(hf, Wp, Wg, 0.3, Kf, y, gamma, H, dI)
                  - oracle.focal_bce_loss64(hf, Wm, Wg, 0.3, Kf, y, gamma, H, dI)) / (2 * eps)
            assert dW[j, c] == pytest.approx(fd, rel=1e-6, abs=1e-9)


def test_loss_terms_against_torch_bce_and_textbook_focal(oracle):
    rng = np.random.default_rng(81)
    H, dI = 2, 3
    h, Wq, Wg, K, y = _tiny_student(rng, Q=3, N=20, H=H, dI=dI)
    loss0, _, z = oracle.focal_bce_grad(h, Wq, Wg, -0.2, K, y, 0.0, H, dI, want_grad=False, want_z=True)
    zt, yt = torch.from_numpy(z), torch.from_numpy(y.astype(np.float64))
    bce = F.binary_cross_entropy_with_logits(zt, yt).item()
    assert loss0 == pytest.approx(2 * bce, rel=1e-13)          # gamma=0: FL == BCE
    loss2, _, _ = oracle.focal_bce_grad(h, Wq, Wg, -0.2, K, y, 2.0, H, dI, want_grad=False)
    p = torch.sigmoid(zt)
    pt = torch.where(yt > 0, p, 1 - p)
    fl = (-(1 - pt) ** 2 * torch.log(pt)).mean().item()
    assert loss2 == pytest.approx(bce + fl, rel=1e-12)


def test_loss_logits_match_library_contraction(oracle):
    rng = np.random.default_rng(82)
    H, dI = 3, 4
    h, Wq, Wg, K, y = _tiny_student(rng, Q=2, N=10, D=6, H=H, dI=dI)
    _, _, z = oracle.focal_bce_grad(h, Wq, Wg, 0.125, K, y, 2.0, H, dI, want_grad=False, want_z=True)
    hf = gen.bf16_bits_to_f32(h).astype(np.float64)
    Kf = gen.bf16_bits_to_f32(K).astype(np.float64)
    q = (hf @ Wq.astype(np.float64).T).reshape(2, H, dI)
    g = np.log1p(np.exp(hf @ Wg.astype(np.float64).T))
    z_ref = np.einsum("th,thd,sd->ts", g, q, Kf) + 0.125
    np.testing.assert_allclose(z, z_ref, rtol=1e-12, atol=1e-12)


def test_loss_at_zero_logits_closed_form(oracle):
    # Wq = 0 -> every logit equals the bias 0: BCE = ln 2, FL = 0.5^gamma ln 2
    rng = np.random.default_rng(83)
    H, dI = 2, 3
    h, Wq, Wg, K, y = _tiny_student(rng, H=H, dI=dI)
    loss, _, _ = oracle.focal_bce_grad(h, np.zeros_like(Wq), Wg, 0.0, K, y, 2.0, H, dI, want_grad=False)
    assert loss == pytest.approx(1.25 * math.log(2.0), rel=1e-15)
