"""Pins of the oracle's storage formats and scalar functions against library
routines and closed forms (no GPU)."""
import math

import numpy as np
import pytest
import torch


def test_bf16_decode_matches_torch(oracle):
    bits = np.arange(0, 1 << 16, 97, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_to_double(bits)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_bf16_round_matches_torch_on_binary32_values(oracle):
    # On values that binary32 holds exactly, torch's fp32->bf16 cast is a
    # single nearest-even rounding, so it must agree with the oracle.
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200_000) * np.exp2(rng.integers(-140, 120, 200_000))).astype(np.float32)
    x = np.concatenate([x, np.float32([0.0, -0.0, 1.0, -2.5, 3.4e38, -3.4e38, 1e-40, -1e-42])])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_from_double(x.astype(np.float64))
    assert (got == ref).all()


@pytest.mark.parametrize("value,bits", [
    (1.0 + 2.0 ** -8, 0x3F80),               # tie -> even mantissa (down)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),           # tie -> even mantissa (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),  # just above the tie: up (a two-step fp32 rounding gives 0x3F80)
    (-(1.0 + 2.0 ** -8 + 2.0 ** -30), 0xBF81),
    (2.0 ** -133, 0x0001),                   # smallest subnormal
    (2.0 ** -134, 0x0000),                   # tie between 0 and 2^-133 -> even (0)
    (3 * 2.0 ** -134, 0x0002),               # tie between 1 and 2 ulps -> even (2)
    ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),  # largest finite
    ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),  # tie at the top rounds to even = infinity
    (1e300, 0x7F80),
])
def test_bf16_round_closed_forms(oracle, value, bits):
    assert int(oracle.bf16_from_double(value)) == bits


def test_e4m3_decode_all_codes_match_torch(oracle):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_to_double(codes)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_softplus_and_sigmoid(oracle):
    assert oracle.softplus(0.0) == pytest.approx(math.log(2.0), abs=1e-16)
    for x in np.linspace(-30, 30, 121):
        assert oracle.softplus(x) == pytest.approx(math.log1p(math.exp(x)), rel=1e-14)
        assert oracle.sigmoid(x) == pytest.approx(1.0 / (1.0 + math.exp(-x)), rel=1e-14)
    assert oracle.softplus(800.0) == 800.0
    assert oracle.softplus(-800.0) == 0.0
    assert oracle.sigmoid(0.0) == 0.5


def test_trigger_cadence(oracle):
    tau = 64
    due = [t for t in range(1000) if oracle.trigger_due(t, tau)]
    assert due[:4] == [0, 64, 128, 192]
    for T in (1, 63, 64, 65, 640, 999):
        assert sum(oracle.trigger_due(t, tau) for t in range(T)) == math.ceil(T / tau)
    assert not oracle.trigger_due(-64, tau)
