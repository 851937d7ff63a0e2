"""Parity of lsa_project_query (MFMA query encoder) with the oracle.

q is bf16: bit-exact except where the oracle's fp64 pre-rounding value lies
within 1e-6 * sum_d |W h| of a bf16 rounding boundary (the GPU accumulates in
fp32, whose error on these sums is far below that).  g is fp32: relative
1e-5."""
import numpy as np
import pytest
import torch

import lsa_inputs as gen
import sparse_kv_cache_lsa_amd as lsa
from gpu_util import DEV, bf16_dev, bf16_host, dev, host
from oracle import oracle
from sparse_kv_cache_lsa_amd.pipeline import pack_weights

pytestmark = pytest.mark.gpu


def _bf16_boundary_distance(a):
    """Distance of each fp64 value to the nearest bf16 rounding midpoint."""
    a = np.asarray(a, np.float64)
    m = np.abs(a)
    e = np.floor(np.log2(np.maximum(m, 1e-300)))
    ulp = np.exp2(e - 7)
    frac = m / ulp - np.floor(m / ulp)
    return np.abs(frac - 0.5) * ulp


def _run_and_check(w: gen.Workload, h=None, stride=0, packed=False):
    h = gen.hidden(w) if h is None else h
    Wq, Wg = zip(*[gen.weights(w, l) for l in range(w.L)])
    q = torch.empty((w.L, w.B, w.H, w.dI), dtype=torch.bfloat16, device=DEV)
    g = torch.empty((w.L, w.B, w.H), dtype=torch.float32, device=DEV)
    wq, wg = [bf16_dev(x) for x in Wq], [bf16_dev(x) for x in Wg]
    lsa.lsa_project_query(bf16_dev(h), wq, wg, q, g, h_layer_stride=stride)
    if packed:
        # packed weights: the same q and g bit for bit (then checked below)
        wp = pack_weights(wq, wg)
        qp = torch.full_like(q, 7.0)
        gp = torch.full_like(g, float("nan"))
        lsa.lsa_project_query_packed(bf16_dev(h), wp, qp, gp, h_layer_stride=stride)
        torch.cuda.synchronize()
        assert torch.equal(qp.view(torch.int16), q.view(torch.int16))
        assert torch.equal(gp, g)
        q, g = qp, gp
    torch.cuda.synchronize()
    qg, gg = bf16_host(q), host(g)
    excluded = 0
    for l in range(w.L):
        for b in range(w.B):
            hb = h[l * (stride // w.D) + b] if stride else h[b]
            qo, go, a = oracle.project(hb, Wq[l], Wg[l], w.H, w.dI, want_a=True)
            S = np.abs(gen.bf16_bits_to_f32(Wq[l]).astype(np.float64)) @ np.abs(
                gen.bf16_bits_to_f32(hb).astype(np.float64))
            band = _bf16_boundary_distance(a.ravel()) <= 1e-6 * S
            diff = qg[l, b].ravel() != qo.ravel()
            assert not (diff & ~band).any(), f"layer {l} request {b}: {(diff & ~band).sum()} q mismatches"
            excluded += int(band.sum())
            np.testing.assert_allclose(gg[l, b], go, rtol=1e-5, atol=1e-7)
    return excluded


@pytest.mark.parametrize("name", ["tiny", "ctx128k"])
def test_project_named_workloads(name):
    print("excluded", _run_and_check(gen.WORKLOADS[name]))


@pytest.mark.parametrize("B,D,H", [(5, 768, 40), (33, 768, 40), (3, 256, 3), (2, 64, 4), (7, 320, 5)])
def test_project_request_groups(B, D, H):
    w = gen.custom("proj", 91, B=B, L=2, H=H, dI=64, D=D, N=64)
    _run_and_check(w)


# Launch regimes of the tile split (R = H*dI + H rows in 16-row tiles, about
# one block per compute unit per (layer, request group), at most 8 tiles a
# block): one tile per block; 3-4 tiles per block; more tiles than
# 8 x blocks, so extra blocks; ten request groups.
@pytest.mark.parametrize("B,L,D,H,dI", [(65, 1, 512, 7, 64), (40, 2, 1024, 24, 128),
                                        (32, 4, 768, 64, 128), (300, 3, 256, 64, 128),
                                        (2, 1, 65536, 64, 128)])   # the largest hidden size
def test_project_tile_split(B, L, D, H, dI):
    w = gen.custom("proj3", 93, B=B, L=L, H=H, dI=dI, D=D, N=64)
    _run_and_check(w)


def test_project_per_layer_hidden_states():
    w = gen.custom("proj2", 92, B=3, L=2, H=8, dI=128, D=512, N=64)
    rng = np.random.default_rng(3)
    h = gen.to_bf16_bits(rng.standard_normal((w.L * w.B, w.D)).astype(np.float32))
    _run_and_check(w, h=h, stride=w.B * w.D)


# Packed weights (lsa_pack_query_weights): one tile, gate tiles, a ragged last
# tile (H*dI + H not a multiple of 16), several request groups, per-layer
# hidden states, the largest tile count.
@pytest.mark.parametrize("B,L,D,H,dI", [(1, 1, 64, 1, 64), (5, 2, 768, 40, 64), (7, 1, 320, 5, 64),
                                        (40, 2, 1024, 24, 128), (65, 1, 512, 7, 64),
                                        (32, 3, 4096, 64, 128),
                                        (2, 1, 65536, 64, 128)])   # the largest hidden size
def test_project_packed_weights(B, L, D, H, dI):
    w = gen.custom("projp", 94, B=B, L=L, H=H, dI=dI, D=D, N=64)
    _run_and_check(w, packed=True)


def test_project_packed_per_layer_hidden_states():
    w = gen.custom("projp2", 95, B=3, L=2, H=8, dI=128, D=512, N=64)
    rng = np.random.default_rng(4)
    h = gen.to_bf16_bits(rng.standard_normal((w.L * w.B, w.D)).astype(np.float32))
    _run_and_check(w, h=h, stride=w.B * w.D, packed=True)


def test_pack_layout_is_the_documented_one():
    # the packed buffer against its definition, element by element
    H, dI, D = 3, 64, 192
    rng = np.random.default_rng(6)
    Wq = rng.integers(0, 1 << 16, (H * dI, D), dtype=np.uint16)
    Wg = rng.integers(0, 1 << 16, (H, D), dtype=np.uint16)
    n = lsa.lsa_query_weights_packed_bytes(H, dI, D)
    R = H * dI + H
    T = (R + 15) // 16
    assert n == T * (D // 64) * 2048
    p = torch.full((n,), 0xA5, dtype=torch.uint8, device=DEV)
    lsa.lsa_pack_query_weights(dev(Wq.view(np.int16)), dev(Wg.view(np.int16)), p)
    torch.cuda.synchronize()
    got = host(p).view(np.uint16).reshape(T, D // 64, 2, 64, 8)
    W = np.zeros((16 * T, D), np.uint16)
    W[:H * dI] = Wq
    W[H * dI:R] = Wg
    l = np.arange(64)
    for t in range(T):
        for u in range(D // 64):
            for st in range(2):
                rows = 16 * t + l % 16
                cols = 64 * u + 32 * st + 8 * (l // 16)
                want = np.stack([W[rows, cols + e] for e in range(8)], axis=1)
                assert np.array_equal(got[t, u, st], want), (t, u, st)
