"""Helpers shared by the GPU tests: host<->device conversion and the oracle
chain for one request (the oracle runs on the CPU, on the same inputs)."""
from __future__ import annotations

import numpy as np
import torch

from oracle import oracle

DEV = "cuda"


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def bf16_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return bf16_dev(x)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def oracle_request(inp, q, g, b: int, k: int):
    """Oracle chain for request b: per-layer z (fp64 [L][N]), survivors,
    merged z*, top-k."""
    w = inp.w
    z = np.stack([oracle.score(inp.keys[l][b], None if inp.scale[l] is None else inp.scale[l][b],
                               q[l, b], g[l, b], float(inp.bias[l])) for l in range(w.L)])
    sel = oracle.threshold(z)
    surv, zstar, count = oracle.merge_compact(sel, z)
    topk, kcount = oracle.topk(surv, zstar, k)
    return z, surv, zstar, count, topk, kcount
