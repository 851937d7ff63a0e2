"""Pins of the oracle's core attention over the selected rows (each row both
key and value, shared by all heads; gist.science technical summary, 2.1,
hierarchical-selection bullet): a library attention, closed forms, the
large-score limit and invariants."""
import math

import numpy as np
import pytest
import torch

import lsa_inputs as gen


def _bf16(rng, *shape, s=1.0):
    return gen.to_bf16_bits((rng.standard_normal(shape) * s).astype(np.float32))


def _f64(bits):
    return gen.bf16_bits_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("n,H,D,scale", [(1, 1, 8, 0.5), (7, 3, 8, 1.0), (300, 4, 64, 0.125),
                                         (2176, 2, 512, 1 / math.sqrt(512)), (33, 16, 128, 2.0)])
def test_attention_matches_torch_softmax_attention(oracle, n, H, D, scale):
    rng = np.random.default_rng(n + H + D)
    q, rows = _bf16(rng, H, D), _bf16(rng, n, D)
    out = oracle.attention(q, rows, scale)
    Q, R = torch.from_numpy(_f64(q)), torch.from_numpy(_f64(rows))
    ref = torch.softmax(scale * Q @ R.T, dim=-1) @ R
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_attention_closed_forms(oracle):
    rng = np.random.default_rng(5)
    D = 16
    rows = _bf16(rng, 9, D)
    q = _bf16(rng, 2, D)
    # one row: the output is that row (weight exactly 1)
    assert np.array_equal(oracle.attention(q, rows[:1], 0.7), np.repeat(_f64(rows[:1]), 2, 0))
    # equal scores (zero query, or zero scale): the mean of the rows
    np.testing.assert_allclose(oracle.attention(np.zeros((1, D), np.uint16), rows, 1.0)[0],
                               _f64(rows).mean(0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(oracle.attention(q, rows, 0.0), np.repeat(_f64(rows).mean(0)[None], 2, 0),
                               rtol=0, atol=1e-15)
    # two rows whose scores differ by delta: weights sigmoid(delta), 1 - sigmoid(delta)
    e0 = np.zeros(D, np.float32)
    e0[0] = 1.0
    q1 = gen.to_bf16_bits(e0[None])
    two = gen.to_bf16_bits(np.stack([np.r_[1.5, np.ones(D - 1)], np.r_[-0.5, -np.ones(D - 1)]])
                           .astype(np.float32))
    scale = 0.8
    delta = scale * (1.5 - (-0.5))
    w0 = 1 / (1 + math.exp(-delta))
    np.testing.assert_allclose(oracle.attention(q1, two, scale)[0],
                               w0 * _f64(two[0]) + (1 - w0) * _f64(two[1]), rtol=1e-14, atol=1e-15)
    # no rows: zeros
    assert not oracle.attention(q, np.zeros((0, D), np.uint16), 1.0).any()


def test_attention_large_scores_stay_finite(oracle):
    # scores of order 1e4 (no overflow: the weights are shifted by the
    # maximum); with gaps that large the output is the best row
    rng = np.random.default_rng(6)
    D = 32
    rows = _bf16(rng, 50, D)
    q = _bf16(rng, 3, D)
    out = oracle.attention(q, rows, 1e4)
    assert np.isfinite(out).all()
    best = np.argmax(_f64(q) @ _f64(rows).T, axis=1)
    np.testing.assert_allclose(out, _f64(rows)[best], rtol=0, atol=1e-12)


def test_attention_invariants(oracle):
    rng = np.random.default_rng(7)
    n, H, D = 120, 5, 24
    q, rows = _bf16(rng, H, D), _bf16(rng, n, D)
    out, wabs = oracle.attention(q, rows, 0.3, want_wabs=True)
    # the set of rows, not their order, decides the output
    perm = rng.permutation(n)
    np.testing.assert_allclose(oracle.attention(q, rows[perm], 0.3), out, rtol=1e-12, atol=1e-13)
    # heads are independent
    np.testing.assert_allclose(oracle.attention(q[2:3], rows, 0.3), out[2:3], rtol=0, atol=0)
    # the output is a convex combination of the rows
    lo, hi = _f64(rows).min(0), _f64(rows).max(0)
    assert (out >= lo - 1e-12).all() and (out <= hi + 1e-12).all()
    # weighted |v| bounds |out|, and equals it for non-negative rows
    assert (wabs >= np.abs(out) - 1e-12).all()
    pos = gen.to_bf16_bits(np.abs(gen.bf16_bits_to_f32(rows)))
    o2, w2 = oracle.attention(q, pos, 0.3, want_wabs=True)
    np.testing.assert_allclose(w2, o2, rtol=1e-13, atol=0)
    # every row twice: each weight halves, the output stays
    dup = np.concatenate([rows, rows])
    np.testing.assert_allclose(oracle.attention(q, dup, 0.3), out, rtol=1e-12, atol=1e-13)
