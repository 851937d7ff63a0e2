"""Comparison rules between the HIP path and the oracle.

Floating point decides three integer outcomes on this path: the I >= 0.5
threshold, the top-k boundary and the top-p boundary.  The GPU takes them in
fp32, the oracle in fp64, so entries whose oracle value lies inside a band
around the boundary are excluded from the exact comparison (and counted);
everything else must match exactly.

Band widths:
  * threshold: |I_oracle - 0.5| <= 1e-3, i.e. |z_oracle| <= Z_BAND, where
    Z_BAND = logit(0.501) = 4.0e-3 (every GPU z must also be within
    Z_TOL < Z_BAND of the oracle, which the score tests assert first);
  * top-k: |z*_oracle - z*_oracle(k-th)| <= 1e-3;
  * top-p: |mass_ahead_oracle - p| <= 1e-4.
"""
from __future__ import annotations

import math

import numpy as np

I_TOL = 1e-3                       # |I_gpu - I_oracle|
Z_BAND = math.log(0.501 / 0.499)   # 4.0e-3: |I - 0.5| <= 1e-3 <=> |z| <= Z_BAND
Z_TOL = 2e-3                       # asserted |z_gpu - z_oracle| (half the band)
TOPK_BAND = 1e-3
TOPP_BAND = 1e-4


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-np.asarray(z, np.float64)))


def unpack_mask(words, N):
    """uint32 words [..., W] -> bool [..., N] (bit s%32 of word s//32)."""
    w = np.ascontiguousarray(np.asarray(words).view(np.uint32))
    bits = np.unpackbits(w.view(np.uint8).reshape(*w.shape, 4), axis=-1, bitorder="little")
    return bits.reshape(*w.shape[:-1], w.shape[-1] * 32)[..., :N].astype(bool)


def check_scores(z_gpu, z_or, I_gpu=None):
    """Returns diagnostics; raises AssertionError on a violation."""
    z_gpu = np.asarray(z_gpu, np.float64)
    z_or = np.asarray(z_or, np.float64)
    dz = np.abs(z_gpu - z_or)
    dI = np.abs(sigmoid(z_gpu) - sigmoid(z_or))
    assert np.isfinite(z_gpu).all(), "non-finite GPU score"
    assert dz.max(initial=0) <= Z_TOL, f"max |dz| = {dz.max():.3g} > {Z_TOL}"
    assert dI.max(initial=0) <= I_TOL, f"max |dI| = {dI.max():.3g}"
    if I_gpu is not None:
        dI2 = np.abs(np.asarray(I_gpu, np.float64) - sigmoid(z_or))
        assert dI2.max(initial=0) <= I_TOL, f"max |I_gpu - I| = {dI2.max():.3g}"
    return {"max_dz": float(dz.max(initial=0)), "max_dI": float(dI.max(initial=0))}


def check_selection(sel_gpu, z_or):
    """Per-layer threshold: exact outside the band."""
    sel_gpu = np.asarray(sel_gpu, bool)
    z_or = np.asarray(z_or, np.float64)
    want = z_or >= 0
    band = np.abs(z_or) <= Z_BAND
    bad = (sel_gpu != want) & ~band
    assert not bad.any(), f"{bad.sum()} selection mismatches outside the band"
    return int(band.sum())


def flatten_candidates(cand_idx, cand_z, cand_count):
    """Chunk candidate lists of one request -> (entries, merged logits)."""
    cnt = np.asarray(cand_count)
    idx = np.concatenate([np.asarray(cand_idx)[c, :cnt[c]] for c in range(cnt.size)]) if cnt.size else np.zeros(0, np.int32)
    z = np.concatenate([np.asarray(cand_z)[c, :cnt[c]] for c in range(cnt.size)]) if cnt.size else np.zeros(0, np.float32)
    return idx, z


def check_merged_scores(idx_gpu, z_gpu, z_or_layers):
    """Merged logit of each listed entry: the max over the layers selecting
    it, compared where every layer's selection is outside the band."""
    z = np.asarray(z_or_layers, np.float64)
    idx = np.asarray(idx_gpu, np.int64)
    zg = np.asarray(z_gpu, np.float64)
    sel = z >= 0
    want = np.where(sel, z, -np.inf).max(axis=0)[idx]
    certain = (np.abs(z) > Z_BAND).all(axis=0)[idx]
    assert np.isfinite(zg).all(), "non-finite merged logit in a survivor list"
    d = np.abs(zg[certain] - want[certain])
    assert d.max(initial=0) <= Z_TOL, f"merged logit max |dz| = {d.max():.3g}"
    return float(d.max(initial=0))


def check_survivors(idx_gpu, count_gpu, z_or_layers, cap=None):
    """z_or_layers: fp64 [L][N].  idx_gpu: the GPU survivor list (first
    min(count, cap) entries)."""
    z = np.asarray(z_or_layers, np.float64)
    N = z.shape[1]
    idx = np.asarray(idx_gpu, np.int64)
    assert (np.diff(idx) > 0).all(), "survivor list not strictly ascending"
    assert idx.size == 0 or (idx[0] >= 0 and idx[-1] < N)
    certain_in = (z >= Z_BAND).any(axis=0)
    certain_out = (z < -Z_BAND).all(axis=0)
    uncertain = ~certain_in & ~certain_out
    n_cap = idx.size
    in_gpu = np.zeros(N, bool)
    in_gpu[idx] = True
    if cap is None or count_gpu <= cap:
        assert n_cap == count_gpu
        missing = certain_in & ~in_gpu
        extra = certain_out & in_gpu
        assert not missing.any(), f"{missing.sum()} certain survivors missing, e.g. {np.nonzero(missing)[0][:5]}"
        assert not extra.any(), f"{extra.sum()} certain non-survivors listed"
        lo = certain_in.sum()
        hi = lo + uncertain.sum()
        assert lo <= count_gpu <= hi
    return int(uncertain.sum())


def check_topk(topk_gpu, count_gpu, surv_idx_or, zstar_or, k, uncertain=None):
    """topk_gpu: GPU top-k list [k] (ascending, -1 padded); surv_idx_or /
    zstar_or: oracle survivors and their fp64 merged logits; uncertain:
    optional bool [N] of entries whose survivor status is inside the
    threshold band (their membership may differ)."""
    t = np.asarray(topk_gpu, np.int64)
    surv = np.asarray(surv_idx_or, np.int64)
    n = surv.size
    zs = np.asarray(zstar_or, np.float64)
    unc_s = np.zeros(n, bool) if uncertain is None else np.asarray(uncertain, bool)[surv]
    if uncertain is None:
        assert count_gpu == min(k, n), f"top-k count {count_gpu} != {min(k, n)}"
    else:
        n_unc_out = int(np.asarray(uncertain, bool).sum() - unc_s.sum())
        lo, hi = min(k, n - int(unc_s.sum())), min(k, n + n_unc_out)
        assert lo <= count_gpu <= hi, f"top-k count {count_gpu} not in [{lo}, {hi}]"
    sel = t[:count_gpu]
    assert (t[count_gpu:] == -1).all(), "top-k padding is not -1"
    assert (np.diff(sel) > 0).all(), "top-k not strictly ascending"
    got = set(int(s) for s in sel)
    if n == 0:
        assert uncertain is not None or not got
        return 0
    kk = min(k, n)
    order = np.lexsort((surv, -zs))
    kth = zs[order[kk - 1]]
    band = (np.abs(zs - kth) <= TOPK_BAND) | unc_s
    want_in = set(int(surv[i]) for i in order[:kk] if not band[i])
    want_out = set(int(surv[i]) for i in order[kk:] if not band[i])
    assert want_in <= got, f"missing top-k members {sorted(want_in - got)[:5]}"
    assert not (want_out & got), f"wrong top-k members {sorted(want_out & got)[:5]}"
    listed = set(surv.tolist())
    for s in got - listed:
        assert uncertain is not None and uncertain[s], f"top-k member {s} is not a survivor"
    return int(band.sum())
