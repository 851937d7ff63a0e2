"""The comparison rules themselves (tests/parity.py), checked on the CPU with
the oracle: the margin that covers GPU query-encoder rounding decisions must
bound the logit change that such decisions cause."""
import numpy as np
import pytest

import lsa_inputs as gen
import parity


@pytest.mark.parametrize("name", ["tiny", "ctx128k"])
def test_flip_margin_bounds_every_rounding_flip(oracle, name):
    w = gen.WORKLOADS[name]
    inp = gen.indexer_inputs(w, gen.load_calibration(w))
    for l in range(w.L):
        q, g, a = oracle.project(inp.h[0], inp.Wq[l], inp.Wg[l], w.H, w.dI, want_a=True)
        kabs = np.abs(gen.bf16_bits_to_f32(inp.keys[l][0]))
        sig = None if inp.scale[l] is None else inp.scale[l][0]
        z = oracle.score(inp.keys[l][0], sig, q, g, float(inp.bias[l]))
        other = parity.other_bf16_neighbour(q, a)
        huge = np.full(a.shape, 1e12)       # puts every element in the band
        rng = np.random.default_rng(l)
        for frac in (1.0, 0.5, 0.01):
            pick = rng.random(q.shape) < frac
            q2 = np.where(pick, other, q)
            E, n = parity.projection_flip_margin(q, q2, a, huge, g, kabs, sig)
            assert n == pick.sum()
            z2 = oracle.score(inp.keys[l][0], sig, q2, g, float(inp.bias[l]))
            assert (np.abs(z2 - z) <= E).all()
        # no difference: no margin
        E, n = parity.projection_flip_margin(q, q, a, huge, g, kabs, sig)
        assert n == 0 and not E.any()


def test_flip_margin_refuses_differences_outside_the_band(oracle):
    w = gen.WORKLOADS["tiny"]
    inp = gen.indexer_inputs(w, gen.load_calibration(w))
    q, g, a = oracle.project(inp.h[0], inp.Wq[0], inp.Wg[0], w.H, w.dI, want_a=True)
    kabs = np.abs(gen.bf16_bits_to_f32(inp.keys[0][0]))
    S = (np.abs(gen.bf16_bits_to_f32(inp.Wq[0])).astype(np.float64) @ np.abs(
        gen.bf16_bits_to_f32(inp.h[0])).astype(np.float64)).reshape(a.shape)
    d = parity.bf16_boundary_distance(a)
    far = np.unravel_index(np.argmax(d / S), a.shape)      # farthest from a midpoint
    q2 = q.copy()
    q2[far] = parity.other_bf16_neighbour(q, a)[far]
    with pytest.raises(AssertionError, match="outside the band"):
        parity.projection_flip_margin(q, q2, a, S, g, kabs)
    # an element inside the band whose GPU value is far from any rounding of
    # a value within the band's error
    near = np.unravel_index(np.argmin(d / S), a.shape)
    q3 = q.copy()
    q3[near] ^= 0x0100
    with pytest.raises(AssertionError, match="not roundings"):
        parity.projection_flip_margin(q, q3, a, S, g, kabs)


def test_boundary_distance_closed_form():
    # 1 + 2^-8 is a bf16 midpoint (between 1 and 1 + 2^-7); 1.5 is representable
    d = parity.bf16_boundary_distance(np.array([1 + 2.0 ** -8, 1.5, -(1 + 2.0 ** -8), 3.0]))
    assert d[0] == 0 and d[2] == 0
    assert d[1] == pytest.approx(2.0 ** -8) and d[3] == pytest.approx(2.0 ** -7)
