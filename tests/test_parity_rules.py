"""The comparison rules themselves (tests/parity.py), checked on the CPU with
the oracle: the margin that covers GPU query-encoder rounding decisions must
bound the logit change that such decisions cause."""
import numpy as np
import pytest

import lsa_inputs as gen
import parity


def _other_neighbour(q_bits, a):
    """The bf16 neighbour of a that q_bits (its RNE rounding) is not."""
    qv = gen.bf16_bits_to_f32(q_bits).astype(np.float64)
    away = np.abs(qv) > np.abs(a)                # rounded away from zero
    step = np.where(away, -1, 1).astype(np.int32)
    return (q_bits.astype(np.int32) + step).astype(np.uint16)


@pytest.mark.parametrize("name", ["tiny", "ctx128k"])
def test_flip_margin_bounds_every_rounding_flip(oracle, name):
    w = gen.WORKLOADS[name]
    inp = gen.indexer_inputs(w, gen.load_calibration(w))
    for l in range(w.L):
        q, g, a = oracle.project(inp.h[0], inp.Wq[l], inp.Wg[l], w.H, w.dI, want_a=True)
        kabs = np.abs(gen.bf16_bits_to_f32(inp.keys[l][0]))
        sig = None if inp.scale[l] is None else inp.scale[l][0]
        z = oracle.score(inp.keys[l][0], sig, q, g, float(inp.bias[l]))
        # an S this large puts every element in the band: flip them all
        E, band = parity.projection_flip_margin(a, np.full(a.shape, 1e12), g, kabs, sig)
        assert band.all()
        q2 = _other_neighbour(q, a)
        z2 = oracle.score(inp.keys[l][0], sig, q2, g, float(inp.bias[l]))
        assert (np.abs(z2 - z) <= E).all()
        # and half of them: the bound still holds (it is a sum over the band)
        rng = np.random.default_rng(l)
        pick = rng.random(q.shape) < 0.5
        z3 = oracle.score(inp.keys[l][0], sig, np.where(pick, q2, q), g, float(inp.bias[l]))
        assert (np.abs(z3 - z) <= E).all()
        # the real band (1e-6 sum |W||h|) holds a small fraction of the elements
        S = np.abs(gen.bf16_bits_to_f32(inp.Wq[l])).astype(np.float64) @ np.abs(
            gen.bf16_bits_to_f32(inp.h[0])).astype(np.float64)
        _, band_real = parity.projection_flip_margin(a, S.reshape(a.shape), g, kabs, sig)
        assert band_real.mean() < 0.1


def test_boundary_distance_closed_form():
    # 1 + 2^-8 is a bf16 midpoint (between 1 and 1 + 2^-7); 1.5 is representable
    d = parity.bf16_boundary_distance(np.array([1 + 2.0 ** -8, 1.5, -(1 + 2.0 ** -8), 3.0]))
    assert d[0] == 0 and d[2] == 0
    assert d[1] == pytest.approx(2.0 ** -8) and d[3] == pytest.approx(2.0 ** -7)
