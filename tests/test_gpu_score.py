"""Parity of lsa_score (collapsed-head dot products + fused epilogue) with the oracle."""
import numpy as np
import pytest
import torch

import lsa_inputs as gen
import sparse_kv_cache_lsa_amd as lsa
import parity
from gpu_util import DEV, bf16_dev, dev, host
from oracle import oracle

pytestmark = pytest.mark.gpu


def _case(seed, L, B, N, H, dI, e4m3):
    rng = np.random.default_rng(seed)
    q = gen.to_bf16_bits(rng.standard_normal((L, B, H, dI)).astype(np.float32))
    g = rng.uniform(0.1, 1.5, (L, B, H)).astype(np.float32)
    keys, scales = [], []
    for l in range(L):
        x = (rng.standard_normal((B, N, dI)) / np.sqrt(dI)).astype(np.float32)
        if e4m3:
            c, s = gen.to_e4m3_rows(x.reshape(-1, dI))
            keys.append(c.reshape(B, N, dI))
            scales.append(s.reshape(B, N))
        else:
            keys.append(gen.to_bf16_bits(x))
            scales.append(None)
    bias = rng.uniform(-1.0, 1.0, L).astype(np.float32)
    return q, g, keys, scales, bias


CH = lsa.LSA_CAND_CHUNK


def _run(q, g, keys, scales, bias, want_I=True, want_z=True):
    L, B, H, dI = q.shape
    N = keys[0].shape[1]
    W = (N + 31) // 32
    nch = (N + CH - 1) // CH
    z = torch.full((L, B, N), float("nan"), dtype=torch.float32, device=DEV) if want_z else None
    I = torch.full((L, B, N), float("nan"), dtype=torch.float32, device=DEV) if want_I else None
    mask = torch.full((L, B, max(W, 1)), -1, dtype=torch.int32, device=DEV)
    ci = torch.full((B, max(nch, 1), CH), -3, dtype=torch.int32, device=DEV)
    cz = torch.full((B, max(nch, 1), CH), float("nan"), dtype=torch.float32, device=DEV)
    cc = torch.full((B, max(nch, 1)), -3, dtype=torch.int32, device=DEV)
    lsa.lsa_score([dev(k) for k in keys], None if scales[0] is None else [dev(s) for s in scales],
                  bf16_dev(q), dev(g), bias, mask[..., :W] if W else mask, ci, cz, cc, z, I)
    torch.cuda.synchronize()
    return ((host(z) if want_z else None), (host(I) if want_I else None), host(mask),
            (host(ci), host(cz), host(cc)))


def _check(q, g, keys, scales, bias, z, I, mask, cand):
    L, B, H, dI = q.shape
    N = keys[0].shape[1]
    W = (N + 31) // 32
    worst = 0.0
    ci, cz, cc = cand
    for b in range(B):
        z_or = np.stack([oracle.score(keys[l][b], None if scales[l] is None else scales[l][b],
                                      q[l, b], g[l, b], float(bias[l])) for l in range(L)])
        for l in range(L):
            if z is not None:
                d = parity.check_scores(z[l, b], z_or[l], None if I is None else I[l, b])
                worst = max(worst, d["max_dz"])
            sel = parity.unpack_mask(mask[l, b, :W], W * 32)
            parity.check_selection(sel[:N], z_or[l])
            assert not sel[N:].any(), "selection bits set past N"
        # the chunk lists: each chunk ascending, inside its chunk, OR of the
        # layers' selections, merged logit = max over selecting layers
        for c in range((N + CH - 1) // CH):
            lst = ci[b, c, :cc[b, c]]
            assert ((lst >= c * CH) & (lst < min(N, (c + 1) * CH))).all()
        idx, zs = parity.flatten_candidates(ci[b], cz[b], cc[b])
        parity.check_survivors(idx, idx.size, z_or)
        worst = max(worst, parity.check_merged_scores(idx, zs, z_or))
    return worst


CASES = [
    # (L, B, N, H, dI, e4m3)
    (1, 1, 4096, 8, 64, False),
    (1, 1, 1000, 64, 128, False),
    (1, 1, 1000, 64, 128, True),
    (1, 1, 4129, 33, 64, True),
    (1, 1, 31, 1, 128, False),
    (1, 1, 1, 64, 128, True),
    (1, 2, 257, 64, 64, False),
    (3, 2, 5000, 64, 128, False),
    (3, 2, 5000, 64, 128, True),
    (2, 3, 8192 + 33, 17, 128, True),
    # enough (chunk, request) blocks for the 4-wavefront launch, ragged last chunk
    (1, 128, 4 * 4096 + 1, 8, 64, True),
    # two chunks a block (enough requests for three such blocks per compute
    # unit): a full chunk and a ragged one; a single short chunk
    (1, 768, 4096 + 33, 8, 64, True),
    (2, 768, 300, 8, 64, False),
    # two-chunk blocks for the first pairs of every request, one-chunk blocks
    # for the rest (768 // 400 = 1 pair a request on 256 compute units)
    (1, 400, 3 * 4096 + 7, 8, 64, True),
]


@pytest.mark.parametrize("L,B,N,H,dI,e4m3", CASES)
def test_score_matches_oracle(L, B, N, H, dI, e4m3):
    q, g, keys, scales, bias = _case(1000 + N + H, L, B, N, H, dI, e4m3)
    z, I, mask, cand = _run(q, g, keys, scales, bias)
    worst = _check(q, g, keys, scales, bias, z, I, mask, cand)
    print(f"max |dz| = {worst:.3g}")


def test_score_at_the_key_size_limit():
    # one (layer, request) at the documented limit: 2^24 - 1 e4m3 entries of
    # 128 dims, 2^31 - 128 bytes of keys, so the last rows sit just below the
    # 32-bit signed offset limit (4,096 chunks: two-chunk and one-chunk blocks).
    # The bulk repeats one random block of 2^20 entries; the first 2^16 and the
    # last 2^18 entries are fresh, so a row read from a wrong offset there
    # changes the result.  The oracle scores those two regions entry by entry.
    N, H, dI, M = (1 << 24) - 1, 8, 128, 1 << 20
    rng = np.random.default_rng(4242)
    q = gen.to_bf16_bits(rng.standard_normal((1, 1, H, dI)).astype(np.float32))
    g = rng.uniform(0.1, 1.5, (1, 1, H)).astype(np.float32)
    bias = np.array([0.3], np.float32)

    def block(n):
        c, sc = gen.to_e4m3_rows((rng.standard_normal((n, dI)) / np.sqrt(dI)).astype(np.float32))
        return c, sc

    kb, sb = block(M)
    keys = np.empty((1, N, dI), np.uint8)
    scl = np.empty((1, N), np.float32)
    for i in range(0, N, M):
        e = min(N, i + M)
        keys[0, i:e] = kb[:e - i]
        scl[0, i:e] = sb[:e - i]
    regions = [(0, 1 << 16), (N - (1 << 18), N)]
    for lo, hi in regions:
        keys[0, lo:hi], scl[0, lo:hi] = block(hi - lo)
    z, I, mask, (ci, cz, cc) = _run(q, g, [keys], [scl], bias)
    W = (N + 31) // 32
    sel = parity.unpack_mask(mask[0, 0, :W], W * 32)
    assert not sel[N:].any(), "selection bits set past N"
    for lo, hi in regions:
        z_or = oracle.score(keys[0, lo:hi], scl[0, lo:hi], q[0, 0], g[0, 0], float(bias[0]))
        d = parity.check_scores(z[0, 0, lo:hi], z_or, I[0, 0, lo:hi])
        parity.check_selection(sel[lo:hi], z_or)
        # one layer: each chunk's list is exactly its set bits, with the layer's logits
        for c in range(-(-lo // CH), hi // CH):
            want = c * CH + np.flatnonzero(sel[c * CH:(c + 1) * CH])
            got = ci[0, c, :cc[0, c]]
            assert np.array_equal(got, want), f"chunk {c}"
            assert np.array_equal(cz[0, c, :cc[0, c]].view(np.uint32), z[0, 0, want].view(np.uint32))
        print(f"entries {lo}..{hi}: max |dz| = {d['max_dz']:.3g}")
    assert cc[0, -1] == np.count_nonzero(sel[(N // CH) * CH:N])


@pytest.mark.parametrize("want_z,want_I", [(False, False), (False, True), (True, False)])
def test_score_optional_outputs(want_z, want_I):
    # the hot path writes only masks + merged logits; optional per-layer
    # outputs must not change them
    q, g, keys, scales, bias = _case(7, 3, 2, 3000, 64, 128, True)
    z, I, mask, cand = _run(q, g, keys, scales, bias, want_I=want_I, want_z=want_z)
    _check(q, g, keys, scales, bias, z, I, mask, cand)


def test_score_n_zero_launches_nothing():
    q, g, keys, scales, bias = _case(8, 1, 1, 0, 8, 64, False)
    e = lambda *sh: torch.empty(sh, dtype=torch.int32, device=DEV)
    lsa.lsa_score([dev(keys[0])], None, bf16_dev(q), dev(g), bias, e(1, 1, 0), e(1, 0, CH),
                  torch.empty((1, 0, CH), device=DEV), e(1, 0))


def test_score_deterministic():
    q, g, keys, scales, bias = _case(9, 2, 2, 20000, 64, 128, True)
    a = _run(q, g, keys, scales, bias)
    b = _run(q, g, keys, scales, bias)
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(np.asarray(x).view(np.uint32), np.asarray(y).view(np.uint32))
    for bb in range(2):
        ia, za = parity.flatten_candidates(a[3][0][bb], a[3][1][bb], a[3][2][bb])
        ib, zb = parity.flatten_candidates(b[3][0][bb], b[3][1][bb], b[3][2][bb])
        assert np.array_equal(ia, ib) and np.array_equal(za.view(np.uint32), zb.view(np.uint32))


@pytest.mark.parametrize("dI", [64, 128])
def test_e4m3_widening_is_exact(dI):
    # every finite e4m3 code, each in its own entry at key dimension
    # (entry % dI) -- so every lane position of a key row is used -- with all
    # query elements 1 and one head of gate 1: z must equal the decoded code
    # exactly (the other dimensions are zero)
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]                       # drop the two NaNs
    codes = np.concatenate([codes, codes[::-1]])                # each code at two dimensions
    N = codes.size
    keys = np.zeros((1, N, dI), np.uint8)
    keys[0, np.arange(N), np.arange(N) % dI] = codes
    scale = np.ones((1, N), np.float32)
    q = gen.to_bf16_bits(np.ones((1, 1, 1, dI), np.float32))
    g = np.ones((1, 1, 1), np.float32)
    z, _, _, _ = _run(q, g, [keys], [scale], np.zeros(1, np.float32))
    want = oracle.e4m3_to_double(codes)
    assert np.array_equal(z[0, 0].astype(np.float64), want)
