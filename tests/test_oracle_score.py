"""Pins of the oracle's query encoder (O1) and lookahead score (O2/O3)
against library routines, closed forms, exact arithmetic and invariants."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import lsa_inputs as gen


def _bf16(x):
    return gen.to_bf16_bits(np.asarray(x, np.float32))


def _f(bits):
    return gen.bf16_bits_to_f32(bits).astype(np.float64)


# ---------------------------------------------------------------- projection

def test_project_matches_numpy_matmul_and_torch_cast(oracle):
    rng = np.random.default_rng(3)
    D, H, dI = 96, 4, 16
    h = _bf16(rng.standard_normal(D))
    Wq = _bf16(rng.standard_normal((H * dI, D)) / math.sqrt(D))
    Wg = _bf16(rng.standard_normal((H, D)) / math.sqrt(D))
    q, g, a = oracle.project(h, Wq, Wg, H, dI, want_a=True)
    a_ref = _f(Wq) @ _f(h)
    np.testing.assert_allclose(a.ravel(), a_ref, rtol=1e-12, atol=1e-14)
    q_ref = torch.from_numpy(a_ref).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (q.ravel() == q_ref).all()
    g_ref = np.log1p(np.exp(_f(Wg) @ _f(h)))
    np.testing.assert_allclose(g, g_ref, rtol=1e-6)
    assert g.dtype == np.float32


def test_project_one_hot_hidden_reads_a_column(oracle):
    rng = np.random.default_rng(4)
    D, H, dI = 32, 2, 8
    Wq = _bf16(rng.standard_normal((H * dI, D)))
    Wg = _bf16(rng.standard_normal((H, D)))
    for j in (0, 7, 31):
        h = np.zeros(D, np.float32)
        h[j] = 1.0
        q, g = oracle.project(_bf16(h), Wq, Wg, H, dI)
        assert (q.ravel() == Wq[:, j]).all()       # column j, exactly
        for hh in range(H):
            x = float(_f(Wg[hh, j]))
            assert g[hh] == np.float32(math.log1p(math.exp(x)))


# --------------------------------------------------------------------- score

def _random_case(rng, N=40, H=3, dI=16, e4m3=False):
    q = _bf16(rng.standard_normal((H, dI)))
    g = rng.uniform(0.1, 2.0, H).astype(np.float32)
    x = rng.standard_normal((N, dI)).astype(np.float32) / 4
    if e4m3:
        keys, scale = gen.to_e4m3_rows(x)
    else:
        keys, scale = _bf16(x), None
    return q, g, keys, scale


def _decode_keys(oracle, keys, scale):
    if keys.dtype == np.uint16:
        return _f(keys)
    return oracle.e4m3_to_double(keys) * scale.astype(np.float64)[:, None]


@pytest.mark.parametrize("e4m3", [False, True])
def test_score_matches_library_contraction(oracle, e4m3):
    # z = K Q^T g + b written with numpy's matmul (a different evaluation:
    # the contraction over d first for every head, then the gate-weighted sum)
    rng = np.random.default_rng(5)
    q, g, keys, scale = _random_case(rng, e4m3=e4m3)
    z = oracle.score(keys, scale, q, g, 0.75)
    K = _decode_keys(oracle, keys, scale)
    z_ref = (K @ _f(q).T) @ g.astype(np.float64) + 0.75
    np.testing.assert_allclose(z, z_ref, rtol=1e-12, atol=1e-12)


def test_score_collapse_identity(oracle):
    # sum_h g_h (q_h . k) == (sum_h g_h q_h) . k
    rng = np.random.default_rng(6)
    q, g, keys, scale = _random_case(rng, N=64, H=8, dI=32)
    q_eff = oracle.query_collapse(q, g)
    np.testing.assert_allclose(q_eff, _f(q).T @ g.astype(np.float64), rtol=1e-13)
    z = oracle.score(keys, scale, q, g, -1.25)
    np.testing.assert_allclose(z, _f(keys) @ q_eff - 1.25, rtol=1e-12, atol=1e-12)


def test_score_exact_small_integers(oracle):
    # small integers and dyadic gates: every intermediate is exact in fp64,
    # so the oracle must reproduce the rational value exactly
    rng = np.random.default_rng(7)
    N, H, dI = 12, 3, 5
    qi = rng.integers(-8, 9, (H, dI))
    ki = rng.integers(-8, 9, (N, dI))
    gi = rng.integers(1, 16, H) / 4.0
    b = -3.5
    z = oracle.score(_bf16(ki), None, _bf16(qi), gi.astype(np.float32), b)
    for s in range(N):
        exact = sum(Fraction(gi[h]) * sum(Fraction(int(qi[h, d]) * int(ki[s, d])) for d in range(dI))
                    for h in range(H)) + Fraction(b)
        assert z[s] == float(exact)


def test_score_e4m3_scale_is_a_factor(oracle):
    rng = np.random.default_rng(8)
    q, g, keys, scale = _random_case(rng, N=32, e4m3=True)
    z_scaled = oracle.score(keys, scale, q, g, 0.0)
    z_unit = oracle.score(keys, np.ones_like(scale), q, g, 0.0)
    np.testing.assert_allclose(z_scaled, z_unit * scale.astype(np.float64), rtol=1e-13)


def test_score_identity_keys(oracle):
    # k_s = e_s: z_s = sum_h g_h q_{h,s} + b
    rng = np.random.default_rng(9)
    H, dI = 4, 16
    q = _bf16(rng.standard_normal((H, dI)))
    g = rng.uniform(0.5, 1.5, H).astype(np.float32)
    keys = _bf16(np.eye(dI))
    z = oracle.score(keys, None, q, g, 0.5)
    want = np.array([sum(float(g[h]) * _f(q[h, s]) for h in range(H)) + 0.5 for s in range(dI)])
    np.testing.assert_allclose(z, want, rtol=1e-14)


def test_score_single_head_is_a_dot_product(oracle):
    rng = np.random.default_rng(10)
    q, _, keys, _ = _random_case(rng, N=50, H=1, dI=24)
    z = oracle.score(keys, None, q, np.ones(1, np.float32), 2.0)
    np.testing.assert_allclose(z, np.dot(_f(keys), _f(q[0])) + 2.0, rtol=1e-13)


def test_score_permutation_invariance(oracle):
    # permuting heads (q rows with their gates) or the key dimension (q and k
    # columns together) must leave every score unchanged
    rng = np.random.default_rng(11)
    q, g, keys, _ = _random_case(rng, N=30, H=5, dI=12)
    z = oracle.score(keys, None, q, g, 0.0)
    ph = rng.permutation(5)
    np.testing.assert_allclose(oracle.score(keys, None, q[ph], g[ph], 0.0), z, rtol=1e-12)
    pd = rng.permutation(12)
    np.testing.assert_allclose(oracle.score(np.ascontiguousarray(keys[:, pd]), None,
                                            np.ascontiguousarray(q[:, pd]), g, 0.0), z, rtol=1e-12)
    # and a genuine change of one key element must change that score
    k2 = keys.copy()
    k2[3, 4] = _bf16(np.float32(_f(k2[3, 4]) + 1.0).reshape(1))[0]
    z2 = oracle.score(k2, None, q, g, 0.0)
    assert z2[3] != z[3] and np.array_equal(np.delete(z2, 3), np.delete(z, 3))


def test_score_index_list_matches_full(oracle):
    rng = np.random.default_rng(12)
    q, g, keys, scale = _random_case(rng, N=70, e4m3=True)
    full = oracle.score(keys, scale, q, g, 0.1)
    idx = np.array([69, 0, 5, 5, 33], np.int64)
    np.testing.assert_array_equal(oracle.score(keys, scale, q, g, 0.1, idx=idx), full[idx])


def test_threshold_is_inclusive_at_half(oracle):
    # z = 0 exactly <=> I = 0.5 exactly: selected; NaN never selected
    z = np.array([0.0, -0.0, -1e-300, 1e-300, np.nan, -np.inf, np.inf])
    assert oracle.threshold(z).tolist() == [1, 1, 0, 1, 0, 0, 1]
    assert oracle.sigmoid(0.0) == 0.5
    rng = np.random.default_rng(13)
    qi = rng.integers(-4, 5, (2, 4))
    ki = rng.integers(-4, 5, (6, 4))
    z0 = oracle.score(_bf16(ki), None, _bf16(qi), np.ones(2, np.float32), 0.0)
    z = oracle.score(_bf16(ki), None, _bf16(qi), np.ones(2, np.float32), -z0[2])
    assert z[2] == 0.0 and oracle.threshold(z)[2] == 1
