"""Parity of lsa_focal_bce_grad (student BCE + focal loss and its gradient
with respect to W_q, fp32 on the GPU) with the fp64 oracle, through the C ABI.

Bars: loss relative error <= 1e-5; dW_q relative Frobenius error <= 1e-4 and
max |error| <= 1e-3 max |dW_q|."""
import numpy as np
import pytest
import torch

import lsa_inputs as gen
import sparse_kv_cache_lsa_amd as lsa
from gpu_util import DEV, dev, host
from oracle import oracle

pytestmark = pytest.mark.gpu


def _gpu(h, Wq, Wg, bias, K, y, gamma, H, dI):
    Q, D = h.shape
    N = K.shape[0]
    loss = torch.full((1,), float("nan"), dtype=torch.float32, device=DEV)
    dW = torch.full((H * dI, D), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(lsa.lsa_focal_bce_grad_workspace_bytes(Q, N, D, H, dI), dtype=torch.uint8,
                     device=DEV)
    lsa.lsa_focal_bce_grad(dev(h), dev(Wq), dev(Wg), bias, dev(K), dev(y), gamma, loss, dW, ws,
                           H=H, dI=dI)
    torch.cuda.synchronize()
    return float(host(loss)[0]), host(dW)


def _check(h, Wq, Wg, bias, K, y, gamma, H, dI):
    lg, dWg = _gpu(h, Wq, Wg, bias, K, y, gamma, H, dI)
    lo, dWo, _ = oracle.focal_bce_grad(h, Wq, Wg, bias, K, y, gamma, H, dI)
    assert abs(lg - lo) <= 1e-5 * abs(lo), (lg, lo)
    err = dWg.astype(np.float64) - dWo
    fro = np.linalg.norm(err) / np.linalg.norm(dWo)
    assert fro <= 1e-4, fro
    assert np.abs(err).max() <= 1e-3 * np.abs(dWo).max()
    return lg, lo, fro


def _random_student(rng, Q, N, D, H, dI, pos=0.1):
    h = gen.to_bf16_bits(rng.standard_normal((Q, D)).astype(np.float32))
    Wq = (rng.standard_normal((H * dI, D)) / np.sqrt(D)).astype(np.float32)
    Wg = (rng.standard_normal((H, D)) / np.sqrt(D)).astype(np.float32)
    K = gen.to_bf16_bits((rng.standard_normal((N, dI)) / np.sqrt(dI)).astype(np.float32))
    y = (rng.random((Q, N)) < pos).astype(np.uint8)
    return h, Wq, Wg, K, y


def test_focal_full_label_workload():
    w = gen.LABELS
    h, Wq, Wg, K, b = gen.student(w)
    # the labels are the oracle's majority-vote labels of the workload's teacher logits
    y = np.empty((w.Q, w.N), np.uint8)
    for q in range(w.Q):
        x = gen.teacher_logits(w, q)
        sel = np.stack([oracle.nucleus(x[l], w.top_p)[0] for l in range(w.L)])
        y[q] = oracle.vote(sel, w.theta)[1]
    print("labels ready", flush=True)
    lg, lo, fro = _check(h, Wq, Wg, b, K, y, w.gamma, w.H, w.dI)
    print(f"loss gpu {lg:.7f} oracle {lo:.7f}; dW rel fro err {fro:.2e}")


@pytest.mark.parametrize("Q,N,D,H,dI", [(1, 1, 128, 1, 64), (3, 100, 128, 3, 64), (5, 1000, 256, 8, 128),
                                         (64, 4097, 128, 64, 64), (17, 333, 384, 5, 128),
                                         (2, 50, 640, 2, 64), (4, 500, 2048, 6, 64),
                                         (3, 200, 1536, 3, 128), (2, 300, 512, 7, 64),
                                         (3, 500, 16384, 8, 64),        # the largest hidden size
                                         (1, 4000000, 128, 1, 64)])     # the largest entry count
def test_focal_ragged_shapes(Q, N, D, H, dI):
    # D picks the projection's slices of D (1, 2, 4 or 8) and the gate rows'
    # (1, 2 or 4 times as many); H dI / 32 not a multiple of 4 takes two row
    # tiles a wave in the gradient
    rng = np.random.default_rng(Q * 1000 + N)
    h, Wq, Wg, K, y = _random_student(rng, Q, N, D, H, dI)
    _check(h, Wq, Wg, 0.37, K, y, 2.0, H, dI)


@pytest.mark.parametrize("gamma", [0.0, 0.5, 1.0, 2.0, 5.0, 8.0, 9.0])
def test_focal_gamma_values(gamma):
    rng = np.random.default_rng(5)
    h, Wq, Wg, K, y = _random_student(rng, 8, 2000, 128, 4, 64, pos=0.3)
    _check(h, Wq, Wg, -0.5, K, y, gamma, 4, 64)


def test_focal_gamma_zero_is_twice_bce():
    # with gamma = 0 the focal term equals the BCE term: loss = 2 * mean BCE
    rng = np.random.default_rng(9)
    h, Wq, Wg, K, y = _random_student(rng, 4, 500, 128, 2, 64)
    lg, _ = _gpu(h, Wq, Wg, 0.0, K, y, 0.0, 2, 64)
    _, _, z = oracle.focal_bce_grad(h, Wq, Wg, 0.0, K, y, 0.0, 2, 64, want_grad=False, want_z=True)
    bce = np.mean(np.logaddexp(0.0, z) - y * z)
    assert lg == pytest.approx(2 * bce, rel=1e-5)
