"""Parity of lsa_fetch_survivors and lsa_gather_resident with the oracle's
cold-pool fetch, bit-exact: per trigger the copy counts, both slot tables and
every byte of the resident rows (slots that were never written included) must
equal the oracle's after the same sequence of survivor sets."""
import numpy as np
import pytest
import torch

import sparse_kv_cache_lsa_amd as lsa
from gpu_util import DEV, dev, host
from oracle import oracle

pytestmark = pytest.mark.gpu


def _sets(rng, N, steps, frac, keep):
    """A sequence of ascending survivor sets: each keeps about `keep` of the
    previous one and adds fresh entries up to about frac * N."""
    out, cur = [], np.zeros(0, np.int64)
    for _ in range(steps):
        kept = cur[rng.random(cur.size) < keep]
        add = rng.choice(N, max(0, int(frac * N) - kept.size), replace=False) if N else cur[:0]
        cur = np.unique(np.concatenate([kept, add])).astype(np.int64)
        out.append(cur.astype(np.int32))
    return out


class Pair:
    """The GPU resident set and the oracle's, driven with the same calls."""

    def __init__(self, cold, S, cap, pinned):
        B, N, rb = cold.shape
        self.B, self.N, self.S, self.cap, self.rb = B, N, S, cap, rb
        t = torch.from_numpy(cold)
        self.cold = t.pin_memory() if pinned else t.to(DEV)
        if pinned:
            assert self.cold.is_pinned()
        self.cold_np = cold
        self.so = torch.full((B, N), 77, dtype=torch.int32, device=DEV)
        self.eo = torch.full((B, S), 77, dtype=torch.int32, device=DEV)
        lsa.lsa_resident_reset(self.so, self.eo)
        self.rows = torch.zeros((B, S, rb), dtype=torch.uint8, device=DEV)
        nws = lsa.lsa_fetch_workspace_bytes(B, N, cap)
        # stale workspace contents must not matter
        self.ws = torch.full((max(nws, 16),), 0x5A, dtype=torch.uint8, device=DEV)
        self.fc = torch.full((B,), -7, dtype=torch.int32, device=DEV)
        self.o = [(np.full(N, -1, np.int32), np.full(S, -1, np.int32),
                   np.zeros((S, rb), np.uint8)) for _ in range(B)]

    def step(self, sets, counts=None):
        B, cap = self.B, self.cap
        idx = np.full((B, max(cap, 1)), -9, np.int32)[:, :cap].copy()
        cnt = np.zeros(B, np.int32)
        for b, s in enumerate(sets):
            m = min(s.size, cap)
            idx[b, :m] = s[:m]
            cnt[b] = s.size if counts is None else counts[b]
        lsa.lsa_fetch_survivors(self.cold, dev(idx), dev(cnt), self.so, self.eo, self.rows,
                                self.fc, self.ws)
        torch.cuda.synchronize()
        want = []
        for b in range(B):
            n = min(int(cnt[b]), cap)
            so, eo, rows = self.o[b]
            want.append(oracle.fetch(self.cold_np[b], idx[b, :n], so, eo, rows))
        return host(self.fc), np.array(want)

    def check(self):
        so, eo, rows = host(self.so), host(self.eo), host(self.rows)
        for b in range(self.B):
            o_so, o_eo, o_rows = self.o[b]
            assert np.array_equal(so[b], o_so), f"slot_of differs for request {b}"
            assert np.array_equal(eo[b], o_eo), f"entry_of differs for request {b}"
            assert np.array_equal(rows[b], o_rows), f"resident rows differ for request {b}"


@pytest.mark.parametrize("pinned", [True, False])
@pytest.mark.parametrize("rb", [1024, 16, 48])
def test_fetch_sequence_matches_oracle(pinned, rb):
    rng = np.random.default_rng(rb + pinned)
    B, N = 3, 4999                      # N not a multiple of 32
    cold = rng.integers(0, 256, (B, N, rb), dtype=np.uint8)
    seqs = [_sets(rng, N, 6, f, 0.7) for f in (0.25, 0.1, 0.4)]
    S = 2100
    p = Pair(cold, S, N, pinned)
    for t in range(6):
        sets = [seqs[b][t] for b in range(B)]
        if t == 3:
            sets[1] = np.zeros(0, np.int32)           # a request with no survivors
        got, want = p.step(sets)
        assert np.array_equal(got, want), (t, got, want)
        assert (want >= 0).all()
        p.check()


def test_capacity_shortfall_leaves_request_untouched():
    rng = np.random.default_rng(11)
    B, N, rb, S = 2, 3000, 64, 500
    cold = rng.integers(0, 256, (B, N, rb), dtype=np.uint8)
    p = Pair(cold, S, N, pinned=True)
    a = np.sort(rng.choice(N, 400, replace=False)).astype(np.int32)
    got, want = p.step([a, a])
    assert np.array_equal(got, want) and (got == 400).all()
    big = np.sort(rng.choice(N, 700, replace=False)).astype(np.int32)
    # request 0 overflows (700 > 500 slots), request 1 fits exactly
    exact = np.sort(rng.choice(N, 500, replace=False)).astype(np.int32)
    got, want = p.step([big, exact])
    assert got[0] == -1 and want[0] == -1 and got[1] == want[1]
    p.check()
    got, want = p.step([a, a])                     # back to a set that fits
    assert np.array_equal(got, want)
    p.check()


def test_truncated_survivor_lists_and_spare_slots():
    rng = np.random.default_rng(12)
    B, N, rb, cap = 3, 20000, 32, 1500
    cold = rng.integers(0, 256, (B, N, rb), dtype=np.uint8)
    p = Pair(cold, cap + 333, cap, pinned=False)
    for t in range(4):
        sets = [np.sort(rng.choice(N, n, replace=False)).astype(np.int32)
                for n in (2500, 1500, 700 + 100 * t)]
        got, want = p.step(sets)             # surv_count above cap for request 0
        assert np.array_equal(got, want)
        p.check()


def test_every_entry_survives_then_none():
    rng = np.random.default_rng(13)
    B, N, rb = 2, 4096 + 77, 16
    cold = rng.integers(0, 256, (B, N, rb), dtype=np.uint8)
    p = Pair(cold, N, N, pinned=True)
    full = np.arange(N, dtype=np.int32)
    for sets in ([full, full[::3].copy()], [full, full], [full[:0], full[1::2].copy()]):
        got, want = p.step(sets)
        assert np.array_equal(got, want)
        p.check()


def test_one_request_carries_every_row():
    """Copies are spread over all requests' rows: one request with many new
    rows next to requests with none, or with a capacity shortfall."""
    rng = np.random.default_rng(16)
    B, N, rb, S = 5, 30000, 1024, 9000
    cold = rng.integers(0, 256, (B, N, rb), dtype=np.uint8)
    p = Pair(cold, S, N, pinned=True)
    none = np.zeros(0, np.int32)
    many = np.sort(rng.choice(N, 8500, replace=False)).astype(np.int32)
    over = np.sort(rng.choice(N, 9500, replace=False)).astype(np.int32)
    few = np.sort(rng.choice(N, 3, replace=False)).astype(np.int32)
    for sets in ([none, none, many, none, none], [over, few, many, none, many],
                 [none, many, over, few, none]):
        got, want = p.step(sets)
        assert np.array_equal(got, want)
        p.check()


def test_gather_resident_matches_oracle():
    rng = np.random.default_rng(14)
    B, N, rb, S, k = 3, 6000, 1024, 2000, 700
    cold = rng.integers(0, 256, (B, N, rb), dtype=np.uint8)
    p = Pair(cold, S, N, pinned=True)
    seqs = [_sets(rng, N, 3, 0.2, 0.6) for _ in range(B)]
    for t in range(3):
        p.step([seqs[b][t] for b in range(B)])
        idx = np.full((B, k), -1, np.int32)
        for b in range(B):
            s = seqs[b][t]
            m = min(k - 20, s.size)
            idx[b, :m] = np.sort(rng.choice(s, m, replace=False))
            idx[b, m:m + 10] = rng.integers(0, N, 10)      # mostly not resident
        hot = torch.full((B, k, rb), 0xEE, dtype=torch.uint8, device=DEV)
        lsa.lsa_gather_resident(p.rows, p.so, dev(idx), hot)
        torch.cuda.synchronize()
        hot = host(hot)
        for b in range(B):
            so, _, rows = p.o[b]
            assert np.array_equal(hot[b], oracle.gather_resident(rows, so, idx[b]))
            m = min(k - 20, seqs[b][t].size)
            assert np.array_equal(hot[b, :m], cold[b, idx[b, :m]])


def test_fetch_at_1m_context_rows():
    """Four requests of the 1M-context shape (N = 262,144 entries, 1 KiB KV
    rows, a pinned 1 GiB cold pool), ~24% survivors; the second trigger keeps
    ~80% of them.  Resident set of N/2 slots."""
    rng = np.random.default_rng(15)
    B, N, rb = 4, 262144, 1024
    cold = np.empty((B, N, rb), np.uint8)
    for b in range(B):
        cold[b] = rng.integers(0, 256, (N, rb), dtype=np.uint8)
    p = Pair(cold, N // 2, N, pinned=True)
    seqs = [_sets(rng, N, 2, 0.24, 0.8) for _ in range(B)]
    for t in range(2):
        got, want = p.step([seqs[b][t] for b in range(B)])
        assert np.array_equal(got, want)
        p.check()


def test_pageable_cold_pool_is_refused():
    """A cold pool in ordinary (pageable) host memory is refused before any
    launch.  No request has survivors, so nothing would be read even if the
    check let it through."""
    import ctypes as C
    from sparse_kv_cache_lsa_amd import _abi
    B, N, S, rb = 1, 64, 8, 1024
    buf = np.zeros(N * rb + 16, np.uint8)
    addr = (buf.ctypes.data + 15) & ~15
    so = torch.full((B, N), -1, dtype=torch.int32, device=DEV)
    eo = torch.full((B, S), -1, dtype=torch.int32, device=DEV)
    rows = torch.zeros((B, S, rb), dtype=torch.uint8, device=DEV)
    idx = torch.zeros((B, 4), dtype=torch.int32, device=DEV)
    cnt = torch.zeros((B,), dtype=torch.int32, device=DEV)
    fc = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    nws = lsa.lsa_fetch_workspace_bytes(B, N, 4)
    ws = torch.zeros((nws,), dtype=torch.uint8, device=DEV)
    lib = _abi.load()
    st = lib.lsa_fetch_survivors(B, N, S, rb, C.c_void_p(addr), 4, idx.data_ptr(),
                                 cnt.data_ptr(), so.data_ptr(), eo.data_ptr(), rows.data_ptr(),
                                 fc.data_ptr(), ws.data_ptr(), nws,
                                 torch.cuda.current_stream().cuda_stream)
    assert st == _abi.LSA_E_ARG and b"cold pool" in lib.lsa_last_error()
    torch.cuda.synchronize()
    assert host(fc).tolist() == [-7]
    with pytest.raises(ValueError):
        lsa.lsa_fetch_survivors(torch.zeros((B, N, rb), dtype=torch.uint8), idx, cnt, so, eo,
                                rows, fc, ws)


def test_many_requests():
    """More requests than one planning block covers (the per-request copy
    offsets are summed in several passes), some of them over capacity."""
    rng = np.random.default_rng(17)
    B, N, rb, S = 1100, 256, 16, 60
    cold = rng.integers(0, 256, (B, N, rb), dtype=np.uint8)
    p = Pair(cold, S, N, pinned=True)
    for t in range(3):
        sizes = rng.integers(0, 70, B)                 # sizes above 60 do not fit
        sets = [np.sort(rng.choice(N, n, replace=False)).astype(np.int32) for n in sizes]
        got, want = p.step(sets)
        assert np.array_equal(got, want)
        assert (got == -1).any() and (got > 0).any()
        p.check()
