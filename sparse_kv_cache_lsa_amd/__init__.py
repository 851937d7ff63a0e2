"""MI355X (gfx950) Lookahead Sparse Attention indexer hot path.

A thin binding of ``liblsa.so``: every function below has the name of the C
entry point it calls, turns torch tensors into device pointers and sizes, and
raises ``LSAError`` on a non-OK status.  All computation happens in the HIP
kernels; torch only provides device memory and streams.  If the library is not
built, every call raises.
"""
from __future__ import annotations

import ctypes as C

from ._abi import (LSA_CAND_CHUNK, LSA_KEY_BF16, LSA_KEY_FP8_E4M3, LSAError, check, load,
                   ptr_array)

__all__ = [
    "LSAError", "LSA_KEY_BF16", "LSA_KEY_FP8_E4M3", "LSA_CAND_CHUNK", "load", "lsa_version",
    "lsa_trigger_due", "lsa_project_query", "lsa_query_weights_packed_bytes",
    "lsa_pack_query_weights", "lsa_project_query_packed", "lsa_score", "lsa_select_or_compact",
    "lsa_topk_workspace_bytes", "lsa_topk", "lsa_gather_hot", "lsa_fetch_workspace_bytes",
    "lsa_resident_reset", "lsa_fetch_survivors", "lsa_gather_resident",
    "lsa_label_vote_workspace_bytes", "lsa_label_vote",
    "lsa_focal_bce_grad_workspace_bytes", "lsa_focal_bce_grad",
]


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _p(t):
    return None if t is None else t.data_ptr()


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("LSA tensors must live on the GPU")
        if t is not None and not t.is_contiguous():
            raise ValueError("LSA tensors must be contiguous")


def _expect(fn, name, t, shape):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{fn}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _row_bytes(t) -> int:
    """Bytes of one row of a [B][rows][...] tensor."""
    n = 1
    for d in t.shape[2:]:
        n *= d
    return n * t.element_size()


def _same_rows(fn, row_tensors, row_bytes, B, batch_tensors):
    """The row size and the batch size that a call passes to the library must
    hold for every tensor, or a kernel would read or write past one of them."""
    for t in row_tensors:
        if t.dim() < 3 or _row_bytes(t) != row_bytes or t.shape[0] != B:
            raise ValueError(f"{fn}: every row tensor must be [B={B}][rows][...] with "
                             f"{row_bytes}-byte rows")
    for t in batch_tensors:
        if t.shape[0] != B:
            raise ValueError(f"{fn}: batch size {t.shape[0]} of an index/table tensor is not B={B}")


def lsa_version() -> str:
    return load().lsa_version().decode()


def lsa_trigger_due(decode_step: int, tau: int = 64) -> bool:
    return bool(load().lsa_trigger_due(int(decode_step), int(tau)))


def lsa_project_query(h, Wq, Wg, q, g, *, h_layer_stride: int = 0, stream=None):
    """h bf16 [B][D] (or [L][B][D] with h_layer_stride = B*D); Wq/Wg: lists of
    L bf16 tensors [H*dI][D] / [H][D]; q out bf16 [L][B][H][dI]; g out f32 [L][B][H]."""
    _dev(h, q, g, *Wq, *Wg)
    L, B, H, dI = q.shape
    D = h.shape[-1]
    _check_project("lsa_project_query", h, g, L, B, H, D, h_layer_stride)
    if len(Wq) != L or len(Wg) != L:
        raise ValueError("lsa_project_query: one W_q and one W_g per layer")
    for l in range(L):
        _expect("lsa_project_query", f"Wq[{l}]", Wq[l], (H * dI, D))
        _expect("lsa_project_query", f"Wg[{l}]", Wg[l], (H, D))
    wq, _k1 = ptr_array([_p(w) for w in Wq])
    wg, _k2 = ptr_array([_p(w) for w in Wg])
    check(load().lsa_project_query(L, B, D, H, dI, _p(h), int(h_layer_stride), wq, wg, _p(q),
                                   _p(g), _stream(stream)))


def _check_project(fn, h, g, L, B, H, D, stride):
    _expect(fn, "g", g, (L, B, H))
    # the kernels read rows b*D .. of h, and layer l from l*stride on
    if h.numel() < (L - 1) * stride + B * D:
        raise ValueError(f"{fn}: h holds {h.numel()} elements; B*D (+ (L-1)*h_layer_stride) "
                         f"= {(L - 1) * stride + B * D} are read")


def lsa_query_weights_packed_bytes(H: int, dI: int, D: int) -> int:
    return int(load().lsa_query_weights_packed_bytes(H, dI, D))


def lsa_pack_query_weights(Wq, Wg, packed, *, stream=None):
    """One layer: Wq bf16 [H*dI][D], Wg bf16 [H][D] -> packed (uint8 tensor of
    lsa_query_weights_packed_bytes(H, dI, D) bytes)."""
    _dev(Wq, Wg, packed)
    H, D = Wg.shape
    dI = Wq.shape[0] // H
    check(load().lsa_pack_query_weights(H, dI, D, _p(Wq), _p(Wg), _p(packed), _stream(stream)))


def lsa_project_query_packed(h, packed, q, g, *, h_layer_stride: int = 0, stream=None):
    """lsa_project_query with a list of L packed weight buffers."""
    _dev(h, q, g, *packed)
    L, B, H, dI = q.shape
    D = h.shape[-1]
    _check_project("lsa_project_query_packed", h, g, L, B, H, D, h_layer_stride)
    need = lsa_query_weights_packed_bytes(H, dI, D)
    if len(packed) != L or any(p.numel() * p.element_size() < need for p in packed):
        raise ValueError(f"lsa_project_query_packed: one packed buffer of {need} bytes per layer")
    wp, _k = ptr_array([_p(w) for w in packed])
    check(load().lsa_project_query_packed(L, B, D, H, dI, _p(h), int(h_layer_stride), wp, _p(q),
                                          _p(g), _stream(stream)))


def lsa_score(keys, key_scale, q, g, bias, sel_mask, cand_idx, cand_z, cand_count, z=None,
              I=None, *, stream=None):
    """keys: list of L tensors [B][N][dI] (bf16 bits, or e4m3 codes with
    key_scale a list of L fp32 [B][N]); bias: L host floats.  Outputs:
    sel_mask int32 [L][B][ceil(N/32)]; chunk candidate lists cand_idx int32 /
    cand_z f32 [B][nchunks][LSA_CAND_CHUNK], cand_count int32 [B][nchunks];
    optional per-layer z and I, f32 [L][B][N]."""
    fp8 = key_scale is not None
    _dev(q, g, sel_mask, cand_idx, cand_z, cand_count, z, I, *keys, *(key_scale or []))
    L, B, H, dI = q.shape
    N = keys[0].shape[1]
    if N > 0:
        fn = "lsa_score"
        if len(keys) != L or len(bias) < L or (fp8 and len(key_scale) != L):
            raise ValueError(f"{fn}: one key tensor, bias (and scale) per layer")
        for l in range(L):
            _expect(fn, f"keys[{l}]", keys[l], (B, N, dI))
            if keys[l].element_size() != (1 if fp8 else 2):
                raise ValueError(f"{fn}: keys must be 1-byte e4m3 codes or 2-byte bf16")
            if fp8:
                _expect(fn, f"key_scale[{l}]", key_scale[l], (B, N))
        nch = (N + LSA_CAND_CHUNK - 1) // LSA_CAND_CHUNK
        _expect(fn, "g", g, (L, B, H))
        _expect(fn, "sel_mask", sel_mask, (L, B, (N + 31) // 32))
        _expect(fn, "cand_idx", cand_idx, (B, nch, LSA_CAND_CHUNK))
        _expect(fn, "cand_z", cand_z, (B, nch, LSA_CAND_CHUNK))
        _expect(fn, "cand_count", cand_count, (B, nch))
        _expect(fn, "z", z, (L, B, N))
        _expect(fn, "I", I, (L, B, N))
    kp, _k1 = ptr_array([_p(k) for k in keys])
    if fp8:
        sp, _k2 = ptr_array([_p(s) for s in key_scale])
    else:
        sp = None
    b = (C.c_float * L)(*[float(x) for x in bias])
    check(load().lsa_score(L, B, N, H, dI, LSA_KEY_FP8_E4M3 if fp8 else LSA_KEY_BF16, kp, sp,
                           _p(q), _p(g), b, _p(sel_mask), _p(cand_idx), _p(cand_z),
                           _p(cand_count), _p(z), _p(I), _stream(stream)))


def lsa_select_or_compact(cand_idx, cand_z, cand_count, N, surv_idx, surv_z, surv_count, *,
                          stream=None):
    """Chunk candidate lists of lsa_score (N entries per request) ->
    surv_idx i32 [B][cap], surv_z f32 [B][cap], surv_count i32 [B]."""
    _dev(cand_idx, cand_z, cand_count, surv_idx, surv_z, surv_count)
    B, cap = surv_idx.shape
    nch = (int(N) + LSA_CAND_CHUNK - 1) // LSA_CAND_CHUNK
    fn = "lsa_select_or_compact"
    _expect(fn, "cand_idx", cand_idx, (B, nch, LSA_CAND_CHUNK))
    _expect(fn, "cand_z", cand_z, (B, nch, LSA_CAND_CHUNK))
    _expect(fn, "cand_count", cand_count, (B, nch))
    _expect(fn, "surv_z", surv_z, (B, cap))
    _expect(fn, "surv_count", surv_count, (B,))
    check(load().lsa_select_or_compact(B, int(N), _p(cand_idx), _p(cand_z), _p(cand_count), cap,
                                       _p(surv_idx), _p(surv_z), _p(surv_count),
                                       _stream(stream)))


def lsa_topk_workspace_bytes(B: int, cap: int, k: int) -> int:
    return int(load().lsa_topk_workspace_bytes(B, cap, k))


def lsa_topk(surv_idx, surv_z, surv_count, topk_idx, topk_count, ws=None, *, stream=None):
    _dev(surv_idx, surv_z, surv_count, topk_idx, topk_count, ws)
    B, cap = surv_idx.shape
    k = topk_idx.shape[1]
    _expect("lsa_topk", "surv_z", surv_z, (B, cap))
    _expect("lsa_topk", "surv_count", surv_count, (B,))
    _expect("lsa_topk", "topk_idx", topk_idx, (B, k))
    _expect("lsa_topk", "topk_count", topk_count, (B,))
    check(load().lsa_topk(B, cap, k, _p(surv_idx), _p(surv_z), _p(surv_count), _p(topk_idx),
                          _p(topk_count), _p(ws),
                          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def lsa_gather_hot(pool, idx, hot, *, stream=None):
    """pool [B][N][row] (any dtype), idx i32 [B][k], hot out [B][k][row]."""
    _dev(pool, idx, hot)
    B, N = pool.shape[0], pool.shape[1]
    k = idx.shape[1]
    row_bytes = _row_bytes(hot)
    _same_rows("lsa_gather_hot", (pool, hot), row_bytes, B, (idx,))
    check(load().lsa_gather_hot(B, N, k, row_bytes, _p(pool), _p(idx), _p(hot), _stream(stream)))


def lsa_fetch_workspace_bytes(B: int, N: int, cap: int) -> int:
    return int(load().lsa_fetch_workspace_bytes(B, N, cap))


def lsa_resident_reset(slot_of, entry_of, *, stream=None):
    """slot_of int32 [B][N], entry_of int32 [B][S] -> all -1 (nothing resident)."""
    _dev(slot_of, entry_of)
    B, N = slot_of.shape
    check(load().lsa_resident_reset(B, N, entry_of.shape[1], _p(slot_of), _p(entry_of),
                                    _stream(stream)))


def lsa_fetch_survivors(cold_pool, surv_idx, surv_count, slot_of, entry_of, rows, fetch_count,
                        ws=None, *, stream=None):
    """cold_pool [B][N][row] in pinned host memory (or on the GPU); surv_idx
    i32 [B][cap] ascending, surv_count i32 [B]; slot_of i32 [B][N], entry_of
    i32 [B][S] and rows [B][S][row] (the resident set, updated in place);
    fetch_count out i32 [B] = rows copied."""
    if not (cold_pool.is_cuda or cold_pool.is_pinned()):
        raise ValueError("the cold pool must be pinned host memory or a GPU tensor")
    if not cold_pool.is_contiguous():
        raise ValueError("LSA tensors must be contiguous")
    _dev(surv_idx, surv_count, slot_of, entry_of, rows, fetch_count, ws)
    B, N = cold_pool.shape[0], cold_pool.shape[1]
    S = entry_of.shape[1]
    cap = surv_idx.shape[1]
    row_bytes = _row_bytes(cold_pool)
    _same_rows("lsa_fetch_survivors", (cold_pool, rows), row_bytes, B,
               (surv_idx, surv_count, slot_of, entry_of, fetch_count))
    if slot_of.shape[1] != N or rows.shape[1] != S:
        raise ValueError("lsa_fetch_survivors: slot_of must be [B][N] and rows [B][S][row] "
                         "with S = entry_of.shape[1]")
    check(load().lsa_fetch_survivors(B, N, S, row_bytes, _p(cold_pool), cap, _p(surv_idx),
                                     _p(surv_count), _p(slot_of), _p(entry_of), _p(rows),
                                     _p(fetch_count), _p(ws),
                                     0 if ws is None else ws.numel() * ws.element_size(),
                                     _stream(stream)))


def lsa_gather_resident(rows, slot_of, idx, hot, *, stream=None):
    """rows [B][S][row], slot_of i32 [B][N], idx i32 [B][k] -> hot [B][k][row]."""
    _dev(rows, slot_of, idx, hot)
    B, S = rows.shape[0], rows.shape[1]
    N = slot_of.shape[1]
    k = idx.shape[1]
    row_bytes = _row_bytes(hot)
    _same_rows("lsa_gather_resident", (rows, hot), row_bytes, B, (slot_of, idx))
    check(load().lsa_gather_resident(B, N, S, k, row_bytes, _p(rows), _p(slot_of), _p(idx),
                                     _p(hot), _stream(stream)))


def lsa_label_vote_workspace_bytes(Q: int, L: int, N: int) -> int:
    return int(load().lsa_label_vote_workspace_bytes(Q, L, N))


def lsa_label_vote(logits, top_p, theta, count, label, layer_mask=None, ws=None, *, stream=None):
    """logits f32 [Q][L][N] -> count u8 [Q][N], label u8 [Q][N], optional
    layer_mask [Q][L][ceil(N/32)]."""
    _dev(logits, count, label, layer_mask, ws)
    Q, L, N = logits.shape
    _expect("lsa_label_vote", "count", count, (Q, N))
    _expect("lsa_label_vote", "label", label, (Q, N))
    _expect("lsa_label_vote", "layer_mask", layer_mask, (Q, L, (N + 31) // 32))
    check(load().lsa_label_vote(Q, L, N, float(top_p), int(theta), _p(logits), _p(layer_mask),
                                _p(count), _p(label), _p(ws),
                                0 if ws is None else ws.numel() * ws.element_size(),
                                _stream(stream)))


def lsa_focal_bce_grad_workspace_bytes(Q: int, N: int, D: int, H: int, dI: int) -> int:
    return int(load().lsa_focal_bce_grad_workspace_bytes(Q, N, D, H, dI))


def lsa_focal_bce_grad(h, Wq, Wg, bias, K, label, gamma, loss, dWq, ws=None, *, H: int,
                       dI: int, stream=None):
    _dev(h, Wq, Wg, K, label, loss, dWq, ws)
    Q, D = h.shape
    N = K.shape[0]
    fn = "lsa_focal_bce_grad"
    _expect(fn, "Wq", Wq, (H * dI, D))
    _expect(fn, "Wg", Wg, (H, D))
    _expect(fn, "K", K, (N, dI))
    _expect(fn, "label", label, (Q, N))
    _expect(fn, "dWq", dWq, (H * dI, D))
    if loss.numel() < 1:
        raise ValueError(f"{fn}: loss needs one element")
    check(load().lsa_focal_bce_grad(Q, N, D, H, dI, float(gamma), _p(h), _p(Wq), _p(Wg),
                                    float(bias), _p(K), _p(label), _p(loss), _p(dWq), _p(ws),
                                    0 if ws is None else ws.numel() * ws.element_size(),
                                    _stream(stream)))
