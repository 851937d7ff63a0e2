"""Parity of lsa_sparse_attention (core attention over the selected rows plus
a local window; every row both key and value, shared by all heads) with the
oracle, through the C ABI.

Tolerance, derived from the arithmetic of the kernel (bf16 inputs, products
exact on the matrix cores, fp32 accumulation, softmax in the exp2 domain, the
weights carried as an exact bf16 pair):
  * score error |ds| <= 2^-18 * scale * max_j sum_d |q_d r_jd|  (fp32 sums of
    exact products) + 2^-21 * max_j |s_j|  (rounding of the exp2 argument);
  * each weight then moves by a relative 2 |ds| (numerator and normaliser),
    the bf16 pair leaves a relative 2^-16, and the fp32 sums and rescalings
    of the output (one per 32-row tile and per split) at most
    (n / 32 + 64) * 2^-23;
so |out_gpu - out_oracle| <= (2 |ds| + 2^-16 + (n / 32 + 64) * 2^-23) * A, with
A = sum_j p_j |r_jd| / sum_j p_j (the oracle's weighted magnitude), per
(request, head, dim)."""
import math

import numpy as np
import pytest
import torch

import lsa_inputs as gen
import sparse_kv_cache_lsa_amd as lsa
from gpu_util import DEV, bf16_dev, host
from oracle import oracle

pytestmark = pytest.mark.gpu


def _bound(q, rows, scale, wabs):
    """Per-(head, dim) tolerance of the GPU output, from the rule above."""
    if rows.shape[0] == 0:
        return np.zeros_like(wabs)
    qa = np.abs(gen.bf16_bits_to_f32(q)).astype(np.float64)
    ra = np.abs(gen.bf16_bits_to_f32(rows)).astype(np.float64)
    mag = qa @ ra.T                                   # [H][n] sum_d |q_d r_jd|
    ds = 2.0 ** -18 * scale * mag.max(axis=1) + 2.0 ** -21 * scale * mag.max(axis=1)
    acc = (rows.shape[0] / 32 + 64) * 2.0 ** -23
    return (2 * ds[:, None] + 2.0 ** -16 + acc) * wabs + 1e-30


def _run(a, scale, hc=None, wc=None, use_win=True):
    B, H, D = a.q.shape
    k, W = a.hot.shape[1], (a.win.shape[1] if use_win else 0)
    out = torch.full((B, H, D), float("nan"), dtype=torch.float32, device=DEV)
    ws_n = lsa.lsa_sparse_attention_workspace_bytes(B, H, D, k, W)
    ws = torch.empty((max(ws_n, 1),), dtype=torch.uint8, device=DEV) if ws_n else None
    hcd = None if hc is None else torch.from_numpy(np.asarray(hc, np.int32)).to(DEV)
    wcd = None if wc is None else torch.from_numpy(np.asarray(wc, np.int32)).to(DEV)
    lsa.lsa_sparse_attention(bf16_dev(a.q), bf16_dev(a.hot), out, scale, hot_count=hcd,
                             win=bf16_dev(a.win) if use_win and W else None,
                             win_count=wcd if use_win and W else None, ws=ws)
    torch.cuda.synchronize()
    return host(out), ws_n


def _check(a, scale, got, hc=None, wc=None, use_win=True, requests=None):
    B, H, D = a.q.shape
    k, W = a.hot.shape[1], (a.win.shape[1] if use_win else 0)
    worst = 0.0
    for b in (range(B) if requests is None else requests):
        nh = k if hc is None else min(max(int(hc[b]), 0), k)
        nw = W if wc is None else min(max(int(wc[b]), 0), W)
        rows = np.concatenate([a.hot[b, :nh], a.win[b, :nw] if use_win else a.win[b, :0]])
        want, wabs = oracle.attention(a.q[b], rows, scale, want_wabs=True)
        tol = _bound(a.q[b], rows, scale, wabs)
        err = np.abs(got[b].astype(np.float64) - want)
        assert np.isfinite(got[b]).all(), f"request {b}: non-finite output"
        assert (err <= tol).all(), (f"request {b}: max err {err.max():.3g}, "
                                    f"worst err/tol {(err / tol).max():.3g}")
        pos = tol > 1e-30
        worst = max(worst, float((err[pos] / tol[pos]).max(initial=0)))
    return worst


@pytest.mark.parametrize("name,B,k", [("ctx128k", 1, 2048), ("ctx512k", 16, 2048),
                                      ("ctx1m", 32, 2048)])
def test_attention_matches_oracle_at_workload_shapes(name, B, k):
    # the three decode workloads' shapes: k selected rows plus the local window
    H, W = gen.ATT_HEADS, gen.ATT_WINDOW
    a = gen.attention_inputs(B, H, k, W, wid=61 + B)
    scale = gen.att_scale()
    got, ws_n = _run(a, scale)
    print(name, "splits workspace", ws_n, "worst err/tol", _check(a, scale, got))


def test_attention_ragged_counts_and_empty_requests():
    # per-request counts below k and W (ragged tails inside a tile), a request
    # with no selected rows, one with no window, one with nothing at all
    B, H, k, W = 6, 64, 700, 50
    a = gen.attention_inputs(B, H, k, W, wid=70)
    hc = np.array([700, 333, 0, 31, 699, 0], np.int32)
    wc = np.array([50, 17, 49, 0, 1, 0], np.int32)
    scale = gen.att_scale()
    got, _ = _run(a, scale, hc, wc)
    _check(a, scale, got, hc, wc)
    assert not got[5].any()                     # no rows: zeros


@pytest.mark.parametrize("H,k,W", [(16, 100, 0), (128, 300, 64), (32, 0, 77), (64, 5, 3),
                                   (48, 4097, 0)])
def test_attention_head_counts_and_single_split(H, k, W):
    # H not a multiple of the 64-head block, window only, hot only, a few rows
    # (one split, written without the combine step), a long list
    B = 3
    a = gen.attention_inputs(B, H, k, W, wid=71 + H)
    scale = gen.att_scale()
    got, _ = _run(a, scale, use_win=W > 0)
    _check(a, scale, got, use_win=W > 0)


def test_attention_large_scores_and_counts_beyond_limits():
    # scores of order 100 (scale 4): the exp2-domain softmax stays finite and
    # exact to the bound; counts above k / W are clamped, negative ones read
    # as zero
    B, H, k, W = 4, 64, 200, 40
    a = gen.attention_inputs(B, H, k, W, wid=80)
    hc = np.array([1000, -5, 200, 150], np.int32)
    wc = np.array([-1, 90, 40, 0], np.int32)
    got, _ = _run(a, 4.0, hc, wc)
    _check(a, 4.0, got, hc, wc)


@pytest.mark.parametrize("peaked", [False, True])
def test_attention_at_the_row_limit(peaked):
    # one request at the documented limit k + W = 2^20 rows (2^20 - 64 selected
    # rows and a 64-row window) with 16 heads: 256 splits of 4,096 rows, whose
    # partials the combine step adds in 16 rounds; the oracle checks four
    # sampled heads over all the rows.  At the workload's scale the weights
    # spread over the whole list; at scale 0.5 (scores of std ~11) a few rows
    # anywhere in the list carry most of each head's weight, so a split or a
    # combine round that went wrong would move the output far past the bound.
    B, H, k, W = 1, 16, (1 << 20) - 64, 64
    a = gen.attention_inputs(B, H, k, W, wid=90)
    scale = 0.5 if peaked else gen.att_scale()
    got, ws_n = _run(a, scale)
    assert ws_n == lsa.lsa_sparse_attention_workspace_bytes(B, H, gen.ATT_ROW, k, W) > 0
    assert np.isfinite(got).all()
    heads = [0, 5, 10, 15]
    q = a.q[0][heads]
    rows = np.concatenate([a.hot[0], a.win[0]])
    want, wabs = oracle.attention(q, rows, scale, want_wabs=True)
    tol = _bound(q, rows, scale, wabs)
    err = np.abs(got[0][heads].astype(np.float64) - want)
    assert (err <= tol).all(), f"max err {err.max():.3g}, worst err/tol {(err / tol).max():.3g}"
    print("row limit, peaked" if peaked else "row limit", "worst err/tol", float((err / tol).max()),
          "max |out|", float(np.abs(want).max()))


def test_attention_same_inputs_same_bits():
    a = gen.attention_inputs(8, 64, 1000, 100, wid=81)
    x, _ = _run(a, gen.att_scale())
    y, _ = _run(a, gen.att_scale())
    assert np.array_equal(x, y)
