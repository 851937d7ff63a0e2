"""Parity of lsa_select_or_compact (concatenation of the per-chunk candidate
lists into one ascending survivor list) with the oracle's OR merge and
compaction.  Integer work: bit-exact, including the fp32 merged logits."""
import numpy as np
import pytest
import torch

import sparse_kv_cache_lsa_amd as lsa
from gpu_util import DEV, dev, host
from oracle import oracle

pytestmark = pytest.mark.gpu
CH = lsa.LSA_CAND_CHUNK


def _chunk_lists(sel, z):
    """Test-side input construction: the candidate lists lsa_score defines
    for a request -- per chunk the ascending entries some layer selects, and
    the max of z over the selecting layers."""
    L, N = sel.shape
    nch = (N + CH - 1) // CH
    ci = np.full((nch, CH), -1, np.int32)
    cz = np.full((nch, CH), np.nan, np.float32)
    cc = np.zeros(nch, np.int32)
    any_sel = sel.any(axis=0)
    zm = np.where(sel, z, -np.inf).max(axis=0).astype(np.float32)
    for c in range(nch):
        e = np.nonzero(any_sel[c * CH:(c + 1) * CH])[0] + c * CH
        ci[c, :e.size] = e
        cz[c, :e.size] = zm[e]
        cc[c] = e.size
    return ci, cz, cc


def _run(sel, z, cap):
    L, B, N = sel.shape
    lists = [_chunk_lists(sel[:, b], z[:, b]) for b in range(B)]
    ci = np.stack([x[0] for x in lists]).reshape(B, -1, CH)
    cz = np.stack([x[1] for x in lists]).reshape(B, -1, CH)
    cc = np.stack([x[2] for x in lists]).reshape(B, -1)
    si = torch.full((B, cap), -7, dtype=torch.int32, device=DEV)
    sz = torch.full((B, cap), -7.0, dtype=torch.float32, device=DEV)
    sc = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    lsa.lsa_select_or_compact(dev(ci), dev(cz), dev(cc), N, si, sz, sc)
    torch.cuda.synchronize()
    return host(si), host(sz), host(sc)


@pytest.mark.parametrize("L,B,N", [(3, 4, 1), (3, 4, 31), (3, 4, 4096), (3, 2, 1000),
                                   (3, 2, 8192), (3, 2, 8193), (3, 3, 40000), (1, 1, 70000),
                                   (5, 2, 12345), (2, 1, 1 << 24)])   # the largest N: 4,096 chunks
def test_select_matches_oracle(L, B, N):
    rng = np.random.default_rng(N * 7 + L)
    z = (rng.standard_normal((L, B, N)) * 3 - 2.5).astype(np.float32)
    sel = z >= 0
    si, sz, sc = _run(sel, z, N)
    for b in range(B):
        idx, zs, count = oracle.merge_compact(sel[:, b].astype(np.uint8), z[:, b].astype(np.float64))
        assert sc[b] == count
        assert np.array_equal(si[b, :count], idx)
        assert np.array_equal(sz[b, :count].astype(np.float64), zs)


def test_select_capacity_overflow_reports_true_count():
    rng = np.random.default_rng(3)
    L, B, N, cap = 3, 2, 20000, 1000
    z = rng.standard_normal((L, B, N)).astype(np.float32)
    sel = z >= 0
    si, sz, sc = _run(sel, z, cap)
    for b in range(B):
        idx, zs, count = oracle.merge_compact(sel[:, b].astype(np.uint8),
                                              z[:, b].astype(np.float64), cap=cap)
        assert sc[b] == count > cap
        assert np.array_equal(si[b], idx)
        assert np.array_equal(sz[b].astype(np.float64), zs)


def test_select_empty_chunks_and_no_survivors():
    L, B, N = 3, 2, 3 * CH + 5
    z = np.full((L, B, N), -1.0, np.float32)
    z[1, 0, 2 * CH + 3] = 4.0           # one survivor in the third chunk of request 0
    si, sz, sc = _run(z >= 0, z, 16)
    assert sc.tolist() == [1, 0] and si[0, 0] == 2 * CH + 3 and sz[0, 0] == 4.0


def test_select_n_zero_sets_zero_counts():
    sc = torch.full((4,), 9, dtype=torch.int32, device=DEV)
    e = lambda *sh: torch.empty(sh, dtype=torch.int32, device=DEV)
    lsa.lsa_select_or_compact(e(4, 0, CH), torch.empty((4, 0, CH), device=DEV), e(4, 0), 0,
                              e(4, 0), torch.empty((4, 0), device=DEV), sc)
    torch.cuda.synchronize()
    assert host(sc).tolist() == [0, 0, 0, 0]


# ---------------------------------------------------------------- dense masks
# lsa_select_or_compact_masks: per-layer masks and logits from any source.


def _pack_bits(sel, junk_rng=None):
    """bool [..., N] -> uint32 words [..., ceil(N/32)] (bit s%32 of word s//32);
    with junk_rng, the bits at or past N are set at random (they must be
    ignored)."""
    N = sel.shape[-1]
    W = (N + 31) // 32
    pad = np.zeros(sel.shape[:-1] + (W * 32,), bool)
    pad[..., :N] = sel
    if junk_rng is not None:
        pad[..., N:] = junk_rng.random(pad[..., N:].shape) < 0.5
    bits = pad.reshape(sel.shape[:-1] + (W, 32)).astype(np.uint64)
    words = (bits << np.arange(32, dtype=np.uint64)).sum(axis=-1)
    return words.astype(np.uint32)


def _run_masks(sel, z, cap, junk=True, seed=0):
    L, B, N = sel.shape
    rng = np.random.default_rng(seed)
    words = _pack_bits(sel, rng if junk else None)
    si = torch.full((B, cap), -7, dtype=torch.int32, device=DEV)
    sz = torch.full((B, cap), -7.0, dtype=torch.float32, device=DEV)
    sc = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    ws = torch.empty((max(1, lsa.lsa_select_or_compact_masks_workspace_bytes(B, N)),),
                     dtype=torch.uint8, device=DEV)
    lsa.lsa_select_or_compact_masks(dev(words.view(np.int32)), dev(z), si, sz, sc, ws)
    torch.cuda.synchronize()
    return host(si), host(sz), host(sc)


def test_pack_bits_layout():
    sel = np.zeros((1, 70), bool)
    sel[0, [0, 5, 31, 32, 69]] = True
    w = _pack_bits(sel)
    assert w.tolist() == [[(1 << 0) | (1 << 5) | (1 << 31), 1, 1 << 5]]


@pytest.mark.parametrize("L,B,N", [(3, 4, 1), (3, 4, 31), (2, 3, 33), (3, 4, 4096), (3, 2, 8193),
                                   (3, 3, 40000), (1, 1, 70000), (8, 2, 12345),
                                   (2, 1, 1 << 24)])   # the largest N
def test_select_masks_matches_oracle(L, B, N):
    # masks independent of z (any producer), NaN and signed zeros among the
    # logits: survivors are the OR of the masks, merged logit the max over
    # all layers ignoring NaN
    rng = np.random.default_rng(N * 11 + L)
    z = (rng.standard_normal((L, B, N)) * 3).astype(np.float32)
    z[rng.random(z.shape) < 0.05] = np.nan
    z[rng.random(z.shape) < 0.01] = -0.0
    sel = rng.random((L, B, N)) < 0.2
    si, sz, sc = _run_masks(sel, z, N, seed=N)
    for b in range(B):
        idx, zs, count = oracle.merge_compact(sel[:, b].astype(np.uint8), z[:, b].astype(np.float64))
        assert sc[b] == count
        assert np.array_equal(si[b, :count], idx)
        np.testing.assert_array_equal(sz[b, :count].astype(np.float64), zs)


def test_select_masks_capacity_overflow_and_empty():
    rng = np.random.default_rng(5)
    L, B, N, cap = 3, 3, 20000, 700
    z = rng.standard_normal((L, B, N)).astype(np.float32)
    sel = z >= 0
    sel[:, 2] = False                      # request 2 has no survivor
    si, sz, sc = _run_masks(sel, z, cap)
    for b in range(B):
        idx, zs, count = oracle.merge_compact(sel[:, b].astype(np.uint8),
                                              z[:, b].astype(np.float64), cap=cap)
        assert sc[b] == count
        assert np.array_equal(si[b, :min(count, cap)], idx)
        assert np.array_equal(sz[b, :min(count, cap)].astype(np.float64), zs)
    assert sc[0] > cap and sc[2] == 0
    assert (si[2] == -7).all()             # nothing written for an empty request


def test_select_masks_n_zero_and_cap_zero():
    sc = torch.full((3,), 9, dtype=torch.int32, device=DEV)
    lsa.lsa_select_or_compact_masks(torch.empty((2, 3, 0), dtype=torch.int32, device=DEV),
                                    torch.empty((2, 3, 0), device=DEV),
                                    torch.empty((3, 0), dtype=torch.int32, device=DEV),
                                    torch.empty((3, 0), device=DEV), sc)
    torch.cuda.synchronize()
    assert host(sc).tolist() == [0, 0, 0]
    z = np.ones((2, 3, 100), np.float32)
    si, sz, sc = _run_masks(z >= 0, z, 0)
    assert sc.tolist() == [100, 100, 100]


def test_select_masks_equals_fused_path_on_a_trigger():
    # the dense path on lsa_score's own masks and logits gives the fused
    # path's survivors and merged logits bit for bit
    from sparse_kv_cache_lsa_amd.pipeline import TriggerBuffers
    rng = np.random.default_rng(9)
    L, B, N, H, dI = 3, 2, 3 * CH + 77, 8, 64
    q = rng.standard_normal((L, B, H, dI)).astype(np.float32)
    g = rng.uniform(0.1, 1.0, (L, B, H)).astype(np.float32)
    keys = [rng.standard_normal((B, N, dI)).astype(np.float32) / 8 for _ in range(L)]
    qd = torch.from_numpy(q).to(DEV).to(torch.bfloat16)
    kd = [torch.from_numpy(k).to(DEV).to(torch.bfloat16) for k in keys]
    buf = TriggerBuffers.allocate(L, B, N, H, dI, 16, device=DEV)
    zl = torch.empty((L, B, N), dtype=torch.float32, device=DEV)
    bias = torch.tensor([-0.5, -1.0, -0.25], device=DEV)
    lsa.lsa_score(kd, None, qd, dev(g), bias, buf.mask, buf.cand_idx, buf.cand_z, buf.cand_count,
                  zl)
    lsa.lsa_select_or_compact(buf.cand_idx, buf.cand_z, buf.cand_count, N, buf.surv_idx,
                              buf.surv_z, buf.surv_count)
    si = torch.full((B, N), -7, dtype=torch.int32, device=DEV)
    sz = torch.full((B, N), -7.0, device=DEV)
    sc = torch.empty((B,), dtype=torch.int32, device=DEV)
    ws = torch.empty((lsa.lsa_select_or_compact_masks_workspace_bytes(B, N),), dtype=torch.uint8,
                     device=DEV)
    lsa.lsa_select_or_compact_masks(buf.mask, zl, si, sz, sc, ws)
    torch.cuda.synchronize()
    assert torch.equal(sc, buf.surv_count) and int(sc.min()) > 0
    for b in range(B):
        n = int(sc[b])
        assert torch.equal(si[b, :n], buf.surv_idx[b, :n])
        assert torch.equal(sz[b, :n], buf.surv_z[b, :n])
