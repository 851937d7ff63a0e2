"""MI355X (gfx950) Lookahead Sparse Attention indexer hot path.

A thin binding of ``liblsa.so``: every function below has the name of the C
entry point it calls, turns torch tensors into device pointers and sizes, and
raises ``LSAError`` on a non-OK status.  All computation happens in the HIP
kernels; torch only provides device memory and streams.  If the library is not
built, every call raises.
"""
from __future__ import annotations

import ctypes as C

from ._abi import (LSA_CAND_CHUNK, LSA_KEY_BF16, LSA_KEY_FP8_E4M3, LSA_TOPK_NOALLOC_MAX_BYTES,
                   LSAError, check, load, ptr_array)

__all__ = [
    "LSAError", "LSA_KEY_BF16", "LSA_KEY_FP8_E4M3", "LSA_CAND_CHUNK", "load", "lsa_version",
    "lsa_trigger_due", "lsa_project_query", "lsa_query_weights_packed_bytes",
    "lsa_pack_query_weights", "lsa_project_query_packed", "lsa_score", "lsa_score_strided",
    "lsa_append_rows", "lsa_select_or_compact",
    "lsa_select_or_compact_masks_workspace_bytes", "lsa_select_or_compact_masks",
    "lsa_topk_workspace_bytes", "lsa_topk", "lsa_topk_noalloc", "lsa_lightning_score",
    "lsa_gather_hot", "lsa_fetch_workspace_bytes",
    "lsa_resident_reset", "lsa_fetch_survivors", "lsa_gather_resident",
    "lsa_sparse_attention_workspace_bytes", "lsa_sparse_attention",
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


def _dtype(fn, name, t, *names):
    """t's dtype must be one of the torch dtypes named (what the kernels read or write)."""
    if t is not None and str(t.dtype).replace("torch.", "") not in names:
        raise ValueError(f"{fn}: {name} has dtype {t.dtype}, expected {' or '.join(names)}")


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


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
    L, B, H, dI = q.shape
    D = h.shape[-1]
    _check_project("lsa_project_query", h, q, g, L, B, H, D, h_layer_stride)
    if len(Wq) != L or len(Wg) != L:
        raise ValueError("lsa_project_query: one W_q and one W_g per layer")
    for l in range(L):
        _expect("lsa_project_query", f"Wq[{l}]", Wq[l], (H * dI, D))
        _expect("lsa_project_query", f"Wg[{l}]", Wg[l], (H, D))
        _dtype("lsa_project_query", f"Wq[{l}]", Wq[l], "bfloat16", "int16", "uint16")
        _dtype("lsa_project_query", f"Wg[{l}]", Wg[l], "bfloat16", "int16", "uint16")
    _dev(h, q, g, *Wq, *Wg)
    wq, _k1 = ptr_array([_p(w) for w in Wq])
    wg, _k2 = ptr_array([_p(w) for w in Wg])
    check(load().lsa_project_query(L, B, D, H, dI, _p(h), int(h_layer_stride), wq, wg, _p(q),
                                   _p(g), _stream(stream)))


def _check_project(fn, h, q, g, L, B, H, D, stride):
    _expect(fn, "g", g, (L, B, H))
    _dtype(fn, "h", h, "bfloat16", "int16", "uint16")
    _dtype(fn, "q", q, "bfloat16", "int16", "uint16")
    _dtype(fn, "g", g, "float32")
    # the kernels read rows b*D .. of h, and layer l from l*stride on
    if h.numel() < (L - 1) * stride + B * D:
        raise ValueError(f"{fn}: h holds {h.numel()} elements; B*D (+ (L-1)*h_layer_stride) "
                         f"= {(L - 1) * stride + B * D} are read")


def lsa_query_weights_packed_bytes(H: int, dI: int, D: int) -> int:
    return int(load().lsa_query_weights_packed_bytes(H, dI, D))


def lsa_pack_query_weights(Wq, Wg, packed, *, stream=None):
    """One layer: Wq bf16 [H*dI][D], Wg bf16 [H][D] -> packed (uint8 tensor of
    lsa_query_weights_packed_bytes(H, dI, D) bytes)."""
    H, D = Wg.shape
    dI = Wq.shape[0] // H
    _expect("lsa_pack_query_weights", "Wq", Wq, (H * dI, D))
    need = lsa_query_weights_packed_bytes(H, dI, D)
    if need == 0 or _nbytes(packed) < need:
        raise ValueError(f"lsa_pack_query_weights: packed must hold {need} bytes, has "
                         f"{_nbytes(packed)}")
    _dtype("lsa_pack_query_weights", "Wq", Wq, "bfloat16", "int16", "uint16")
    _dtype("lsa_pack_query_weights", "Wg", Wg, "bfloat16", "int16", "uint16")
    _dev(Wq, Wg, packed)
    check(load().lsa_pack_query_weights(H, dI, D, _p(Wq), _p(Wg), _p(packed), _stream(stream)))


def lsa_project_query_packed(h, packed, q, g, *, h_layer_stride: int = 0, stream=None):
    """lsa_project_query with a list of L packed weight buffers."""
    L, B, H, dI = q.shape
    D = h.shape[-1]
    _check_project("lsa_project_query_packed", h, q, g, L, B, H, D, h_layer_stride)
    need = lsa_query_weights_packed_bytes(H, dI, D)
    if len(packed) != L or any(p.numel() * p.element_size() < need for p in packed):
        raise ValueError(f"lsa_project_query_packed: one packed buffer of {need} bytes per layer")
    _dev(h, q, g, *packed)
    wp, _k = ptr_array([_p(w) for w in packed])
    check(load().lsa_project_query_packed(L, B, D, H, dI, _p(h), int(h_layer_stride), wp, _p(q),
                                          _p(g), _stream(stream)))


def lsa_score(keys, key_scale, q, g, bias, sel_mask, cand_idx, cand_z, cand_count, z=None,
              I=None, *, stream=None):
    """keys: list of L tensors [B][N][dI] (bf16 bits, or e4m3 codes with
    key_scale a list of L fp32 [B][N]); bias: a GPU float32 tensor [L] (or L
    host floats, copied to the GPU by this call).  Outputs:
    sel_mask int32 [L][B][ceil(N/32)]; chunk candidate lists cand_idx int32 /
    cand_z f32 [B][nchunks][LSA_CAND_CHUNK], cand_count int32 [B][nchunks];
    optional per-layer z and I, f32 [L][B][N]."""
    _score("lsa_score", keys, key_scale, q, g, bias, None, sel_mask, cand_idx, cand_z,
           cand_count, z, I, stream)


def lsa_score_strided(keys, key_scale, q, g, bias, N, sel_mask, cand_idx, cand_z, cand_count,
                      z=None, I=None, *, stream=None):
    """lsa_score over the first N entries of growing caches: keys [B][N_cap][dI]
    (and scales [B][N_cap]) with N <= N_cap; outputs sized by N."""
    _score("lsa_score_strided", keys, key_scale, q, g, bias, int(N), sel_mask, cand_idx,
           cand_z, cand_count, z, I, stream)


def _score(fn, keys, key_scale, q, g, bias, n_live, sel_mask, cand_idx, cand_z, cand_count, z,
           I, stream):
    fp8 = key_scale is not None
    L, B, H, dI = q.shape
    cap = keys[0].shape[1]
    N = cap if n_live is None else n_live
    if not 0 <= N <= cap:
        raise ValueError(f"{fn}: N={N} outside [0, {cap}] (the cache holds {cap} entries)")
    if N > 0:
        if len(keys) != L or len(bias) < L or (fp8 and len(key_scale) != L):
            raise ValueError(f"{fn}: one key tensor, bias (and scale) per layer")
        for l in range(L):
            _expect(fn, f"keys[{l}]", keys[l], (B, cap, dI))
            if keys[l].element_size() != (1 if fp8 else 2):
                raise ValueError(f"{fn}: keys must be 1-byte e4m3 codes or 2-byte bf16")
            if fp8:
                _expect(fn, f"key_scale[{l}]", key_scale[l], (B, cap))
        nch = (N + LSA_CAND_CHUNK - 1) // LSA_CAND_CHUNK
        _expect(fn, "g", g, (L, B, H))
        _expect(fn, "sel_mask", sel_mask, (L, B, (N + 31) // 32))
        _expect(fn, "cand_idx", cand_idx, (B, nch, LSA_CAND_CHUNK))
        _expect(fn, "cand_z", cand_z, (B, nch, LSA_CAND_CHUNK))
        _expect(fn, "cand_count", cand_count, (B, nch))
        _expect(fn, "z", z, (L, B, N))
        _expect(fn, "I", I, (L, B, N))
        _dtype(fn, "q", q, "bfloat16", "int16", "uint16")
        for name, t in (("g", g), ("cand_z", cand_z), ("z", z), ("I", I)):
            _dtype(fn, name, t, "float32")
        for name, t in (("sel_mask", sel_mask), ("cand_idx", cand_idx),
                        ("cand_count", cand_count)):
            _dtype(fn, name, t, "int32", "uint32")
        for l in range(L if fp8 else 0):
            _dtype(fn, f"key_scale[{l}]", key_scale[l], "float32")
    _dev(q, g, sel_mask, cand_idx, cand_z, cand_count, z, I, *keys, *(key_scale or []))
    bias = _bias_tensor(fn, bias, L, q.device)
    kp, _k1 = ptr_array([_p(k) for k in keys])
    if fp8:
        sp, _k2 = ptr_array([_p(s) for s in key_scale])
    else:
        sp = None
    kdt = LSA_KEY_FP8_E4M3 if fp8 else LSA_KEY_BF16
    if n_live is None:
        check(load().lsa_score(L, B, N, H, dI, kdt, kp, sp, _p(q), _p(g), _p(bias),
                               _p(sel_mask), _p(cand_idx), _p(cand_z), _p(cand_count), _p(z),
                               _p(I), _stream(stream)))
    else:
        check(load().lsa_score_strided(L, B, N, cap, H, dI, kdt, kp, sp, _p(q), _p(g), _p(bias),
                                       _p(sel_mask), _p(cand_idx), _p(cand_z), _p(cand_count),
                                       _p(z), _p(I), _stream(stream)))


def lsa_append_rows(src, dst, dst_start, n=None, *, stream=None):
    """dst[b][dst_start + i] = src[b][i] for i < n (n = src.shape[1] by
    default): src [B][n_src][...], dst [B][N_cap][...] with the same row."""
    fn = "lsa_append_rows"
    B = src.shape[0]
    n = src.shape[1] if n is None else int(n)
    rb = _row_bytes(src) if src.dim() >= 3 else src.element_size()
    drb = _row_bytes(dst) if dst.dim() >= 3 else dst.element_size()
    if dst.shape[0] != B or rb != drb:
        raise ValueError(f"{fn}: src and dst must have the same batch and row size")
    if not 0 <= n <= src.shape[1] or not 0 <= dst_start or dst_start + n > dst.shape[1]:
        raise ValueError(f"{fn}: rows [{dst_start}, {dst_start + n}) do not fit the cache of "
                         f"{dst.shape[1]} rows (or n > the {src.shape[1]} source rows)")
    _dev(src, dst)
    check(load().lsa_append_rows(B, n, rb, _p(src), src.shape[1], _p(dst), dst.shape[1],
                                 int(dst_start), _stream(stream)))


def _bias_tensor(fn, bias, L, device):
    """The per-layer bias as the device fp32 [L] array the library reads.  A
    GPU tensor is passed as it is (a captured graph then reads its current
    values on every replay); a host sequence is copied to a new device tensor
    (an allocation and a copy: not for use under graph capture)."""
    import torch
    if isinstance(bias, torch.Tensor) and bias.is_cuda:
        if bias.dtype != torch.float32 or not bias.is_contiguous() or bias.numel() < L:
            raise ValueError(f"{fn}: bias must be a contiguous float32 tensor of at least L={L} "
                             "values")
        return bias
    vals = [float(x) for x in (bias.tolist() if hasattr(bias, "tolist") else bias)]
    if len(vals) < L:
        raise ValueError(f"{fn}: {len(vals)} bias values for L={L} layers")
    return torch.tensor(vals[:L], dtype=torch.float32, device=device)


def lsa_select_or_compact(cand_idx, cand_z, cand_count, N, surv_idx, surv_z, surv_count, *,
                          stream=None):
    """Chunk candidate lists of lsa_score (N entries per request) ->
    surv_idx i32 [B][cap], surv_z f32 [B][cap], surv_count i32 [B]."""
    B, cap = surv_idx.shape
    nch = (int(N) + LSA_CAND_CHUNK - 1) // LSA_CAND_CHUNK
    fn = "lsa_select_or_compact"
    _expect(fn, "cand_idx", cand_idx, (B, nch, LSA_CAND_CHUNK))
    _expect(fn, "cand_z", cand_z, (B, nch, LSA_CAND_CHUNK))
    _expect(fn, "cand_count", cand_count, (B, nch))
    _expect(fn, "surv_z", surv_z, (B, cap))
    _expect(fn, "surv_count", surv_count, (B,))
    for name, t in (("cand_idx", cand_idx), ("cand_count", cand_count), ("surv_idx", surv_idx),
                    ("surv_count", surv_count)):
        _dtype(fn, name, t, "int32")
    _dtype(fn, "cand_z", cand_z, "float32")
    _dtype(fn, "surv_z", surv_z, "float32")
    _dev(cand_idx, cand_z, cand_count, surv_idx, surv_z, surv_count)
    check(load().lsa_select_or_compact(B, int(N), _p(cand_idx), _p(cand_z), _p(cand_count), cap,
                                       _p(surv_idx), _p(surv_z), _p(surv_count),
                                       _stream(stream)))


def lsa_select_or_compact_masks_workspace_bytes(B: int, N: int) -> int:
    return int(load().lsa_select_or_compact_masks_workspace_bytes(B, N))


def lsa_select_or_compact_masks(sel_mask, z, surv_idx, surv_z, surv_count, ws=None, *,
                                stream=None):
    """Dense per-layer selections sel_mask int32/uint32 [L][B][ceil(N/32)] and
    logits z f32 [L][B][N] -> surv_idx i32 [B][cap], surv_z f32 [B][cap],
    surv_count i32 [B]; ws: uint8 tensor of
    lsa_select_or_compact_masks_workspace_bytes(B, N) bytes."""
    fn = "lsa_select_or_compact_masks"
    L, B, N = z.shape
    cap = surv_idx.shape[1] if surv_idx.dim() == 2 else -1
    _expect(fn, "sel_mask", sel_mask, (L, B, (N + 31) // 32))
    _expect(fn, "surv_idx", surv_idx, (B, cap))
    _expect(fn, "surv_z", surv_z, (B, cap))
    _expect(fn, "surv_count", surv_count, (B,))
    _dtype(fn, "z", z, "float32")
    _dtype(fn, "surv_z", surv_z, "float32")
    _dtype(fn, "sel_mask", sel_mask, "int32", "uint32")
    _dtype(fn, "surv_idx", surv_idx, "int32")
    _dtype(fn, "surv_count", surv_count, "int32")
    _dev(sel_mask, z, surv_idx, surv_z, surv_count, ws)
    check(load().lsa_select_or_compact_masks(L, B, N, _p(sel_mask), _p(z), cap, _p(surv_idx),
                                             _p(surv_z), _p(surv_count), _p(ws), _nbytes(ws),
                                             _stream(stream)))


def lsa_topk_workspace_bytes(B: int, cap: int, k: int) -> int:
    return int(load().lsa_topk_workspace_bytes(B, cap, k))


def lsa_topk(surv_idx, surv_z, surv_count, topk_idx, topk_count, ws=None, *, stream=None):
    B, cap = surv_idx.shape
    k = topk_idx.shape[1]
    _expect("lsa_topk", "surv_z", surv_z, (B, cap))
    _expect("lsa_topk", "surv_count", surv_count, (B,))
    _expect("lsa_topk", "topk_idx", topk_idx, (B, k))
    _expect("lsa_topk", "topk_count", topk_count, (B,))
    for name, t in (("surv_idx", surv_idx), ("surv_count", surv_count), ("topk_idx", topk_idx),
                    ("topk_count", topk_count)):
        _dtype("lsa_topk", name, t, "int32")
    _dtype("lsa_topk", "surv_z", surv_z, "float32")
    _dev(surv_idx, surv_z, surv_count, topk_idx, topk_count, ws)
    check(load().lsa_topk(B, cap, k, _p(surv_idx), _p(surv_z), _p(surv_count), _p(topk_idx),
                          _p(topk_count), _p(ws),
                          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def lsa_topk_noalloc(surv_idx, surv_z, surv_count, topk_idx, topk_count, *, stream=None):
    """lsa_topk with the library's own scratch instead of a workspace (for
    callers that cannot allocate; calls that overlap on one GPU race)."""
    B, cap = surv_idx.shape
    k = topk_idx.shape[1]
    _expect("lsa_topk_noalloc", "surv_z", surv_z, (B, cap))
    _expect("lsa_topk_noalloc", "surv_count", surv_count, (B,))
    _expect("lsa_topk_noalloc", "topk_idx", topk_idx, (B, k))
    _expect("lsa_topk_noalloc", "topk_count", topk_count, (B,))
    for name, t in (("surv_idx", surv_idx), ("surv_count", surv_count), ("topk_idx", topk_idx),
                    ("topk_count", topk_count)):
        _dtype("lsa_topk_noalloc", name, t, "int32")
    _dtype("lsa_topk_noalloc", "surv_z", surv_z, "float32")
    _dev(surv_idx, surv_z, surv_count, topk_idx, topk_count)
    check(load().lsa_topk_noalloc(B, cap, k, _p(surv_idx), _p(surv_z), _p(surv_count),
                                  _p(topk_idx), _p(topk_count), _stream(stream)))


def lsa_lightning_score(keys, key_scale, q, w, surv_idx, surv_count, score, *, stream=None):
    """keys [B][N][dI] (bf16, or e4m3 codes with key_scale f32 [B][N]), q bf16
    [B][H][dI], w f32 [B][H], surv_idx i32 [B][cap], surv_count i32 [B] ->
    score f32 [B][cap]."""
    fn = "lsa_lightning_score"
    fp8 = key_scale is not None
    B, N, dI = keys.shape
    H = q.shape[1]
    cap = surv_idx.shape[1]
    _expect(fn, "q", q, (B, H, dI))
    _expect(fn, "w", w, (B, H))
    _expect(fn, "key_scale", key_scale, (B, N))
    _expect(fn, "surv_count", surv_count, (B,))
    _expect(fn, "score", score, (B, cap))
    if keys.element_size() != (1 if fp8 else 2):
        raise ValueError(f"{fn}: keys must be 1-byte e4m3 codes (with key_scale) or 2-byte bf16")
    _dtype(fn, "q", q, "bfloat16", "int16", "uint16")
    for name, t in (("w", w), ("key_scale", key_scale), ("score", score)):
        _dtype(fn, name, t, "float32")
    _dtype(fn, "surv_idx", surv_idx, "int32")
    _dtype(fn, "surv_count", surv_count, "int32")
    _dev(keys, key_scale, q, w, surv_idx, surv_count, score)
    check(load().lsa_lightning_score(B, N, cap, H, dI, LSA_KEY_FP8_E4M3 if fp8 else LSA_KEY_BF16,
                                     _p(keys), _p(key_scale), _p(q), _p(w), _p(surv_idx),
                                     _p(surv_count), _p(score), _stream(stream)))


def lsa_gather_hot(pool, idx, hot, *, stream=None):
    """pool [B][N][row] (any dtype), idx i32 [B][k], hot out [B][k][row]."""
    B, N = pool.shape[0], pool.shape[1]
    k = idx.shape[1]
    row_bytes = _row_bytes(hot)
    _same_rows("lsa_gather_hot", (pool, hot), row_bytes, B, (idx,))
    _expect("lsa_gather_hot", "idx", idx, (B, k))
    if hot.shape[1] != k:
        raise ValueError(f"lsa_gather_hot: hot holds {hot.shape[1]} rows per request, idx {k}")
    _dtype("lsa_gather_hot", "idx", idx, "int32")
    _dev(pool, idx, hot)
    check(load().lsa_gather_hot(B, N, k, row_bytes, _p(pool), _p(idx), _p(hot), _stream(stream)))


def lsa_sparse_attention_workspace_bytes(B: int, H: int, D: int, k: int, W: int) -> int:
    return int(load().lsa_sparse_attention_workspace_bytes(B, H, D, k, W))


def lsa_sparse_attention(q, hot, out, scale, hot_count=None, win=None, win_count=None, ws=None,
                         *, stream=None):
    """q bf16 [B][H][D], hot bf16 [B][k][D] (selected rows), optional
    hot_count i32 [B], win bf16 [B][W][D] (local window) and win_count i32
    [B] -> out f32 [B][H][D]; ws: uint8 tensor of
    lsa_sparse_attention_workspace_bytes(B, H, D, k, W) bytes."""
    fn = "lsa_sparse_attention"
    B, H, D = q.shape
    k = hot.shape[1]
    W = 0 if win is None else win.shape[1]
    _expect(fn, "hot", hot, (B, k, D))
    _expect(fn, "out", out, (B, H, D))
    _expect(fn, "hot_count", hot_count, (B,))
    if win is not None:
        _expect(fn, "win", win, (B, W, D))
    _expect(fn, "win_count", win_count, (B,))
    for name, t in (("q", q), ("hot", hot), ("win", win)):
        _dtype(fn, name, t, "bfloat16", "int16", "uint16")
    _dtype(fn, "out", out, "float32")
    _dtype(fn, "hot_count", hot_count, "int32")
    _dtype(fn, "win_count", win_count, "int32")
    _dev(q, hot, out, hot_count, win, win_count, ws)
    check(load().lsa_sparse_attention(B, H, D, k, W, float(scale), _p(q), _p(hot), _p(hot_count),
                                      _p(win), _p(win_count), _p(out), _p(ws), _nbytes(ws),
                                      _stream(stream)))


def lsa_fetch_workspace_bytes(B: int, N: int, cap: int) -> int:
    return int(load().lsa_fetch_workspace_bytes(B, N, cap))


def lsa_resident_reset(slot_of, entry_of, *, stream=None):
    """slot_of int32 [B][N], entry_of int32 [B][S] -> all -1 (nothing resident)."""
    B, N = slot_of.shape
    if entry_of.dim() != 2 or entry_of.shape[0] != B:
        raise ValueError(f"lsa_resident_reset: entry_of must be [B={B}][S]")
    _dtype("lsa_resident_reset", "slot_of", slot_of, "int32")
    _dtype("lsa_resident_reset", "entry_of", entry_of, "int32")
    _dev(slot_of, entry_of)
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
    B, N = cold_pool.shape[0], cold_pool.shape[1]
    S = entry_of.shape[1]
    cap = surv_idx.shape[1]
    row_bytes = _row_bytes(cold_pool)
    _same_rows("lsa_fetch_survivors", (cold_pool, rows), row_bytes, B,
               (surv_idx, surv_count, slot_of, entry_of, fetch_count))
    if slot_of.shape[1] != N or rows.shape[1] != S:
        raise ValueError("lsa_fetch_survivors: slot_of must be [B][N] and rows [B][S][row] "
                         "with S = entry_of.shape[1]")
    for name, t in (("surv_idx", surv_idx), ("surv_count", surv_count), ("slot_of", slot_of),
                    ("entry_of", entry_of), ("fetch_count", fetch_count)):
        _dtype("lsa_fetch_survivors", name, t, "int32")
    _dev(surv_idx, surv_count, slot_of, entry_of, rows, fetch_count, ws)
    check(load().lsa_fetch_survivors(B, N, S, row_bytes, _p(cold_pool), cap, _p(surv_idx),
                                     _p(surv_count), _p(slot_of), _p(entry_of), _p(rows),
                                     _p(fetch_count), _p(ws),
                                     0 if ws is None else ws.numel() * ws.element_size(),
                                     _stream(stream)))


def lsa_gather_resident(rows, slot_of, idx, hot, *, stream=None):
    """rows [B][S][row], slot_of i32 [B][N], idx i32 [B][k] -> hot [B][k][row]."""
    B, S = rows.shape[0], rows.shape[1]
    N = slot_of.shape[1]
    k = idx.shape[1]
    row_bytes = _row_bytes(hot)
    _same_rows("lsa_gather_resident", (rows, hot), row_bytes, B, (slot_of, idx))
    if hot.shape[1] != k:
        raise ValueError(f"lsa_gather_resident: hot holds {hot.shape[1]} rows per request, idx {k}")
    _dtype("lsa_gather_resident", "slot_of", slot_of, "int32")
    _dtype("lsa_gather_resident", "idx", idx, "int32")
    _dev(rows, slot_of, idx, hot)
    check(load().lsa_gather_resident(B, N, S, k, row_bytes, _p(rows), _p(slot_of), _p(idx),
                                     _p(hot), _stream(stream)))


def lsa_label_vote_workspace_bytes(Q: int, L: int, N: int) -> int:
    return int(load().lsa_label_vote_workspace_bytes(Q, L, N))


def lsa_label_vote(logits, top_p, theta, count, label, layer_mask=None, ws=None, *, stream=None):
    """logits f32 [Q][L][N] -> count u8 [Q][N], label u8 [Q][N], optional
    layer_mask [Q][L][ceil(N/32)]."""
    Q, L, N = logits.shape
    _expect("lsa_label_vote", "count", count, (Q, N))
    _expect("lsa_label_vote", "label", label, (Q, N))
    _expect("lsa_label_vote", "layer_mask", layer_mask, (Q, L, (N + 31) // 32))
    _dtype("lsa_label_vote", "logits", logits, "float32")
    _dtype("lsa_label_vote", "count", count, "uint8")
    _dtype("lsa_label_vote", "label", label, "uint8")
    _dtype("lsa_label_vote", "layer_mask", layer_mask, "int32", "uint32")
    _dev(logits, count, label, layer_mask, ws)
    check(load().lsa_label_vote(Q, L, N, float(top_p), int(theta), _p(logits), _p(layer_mask),
                                _p(count), _p(label), _p(ws),
                                0 if ws is None else ws.numel() * ws.element_size(),
                                _stream(stream)))


def lsa_focal_bce_grad_workspace_bytes(Q: int, N: int, D: int, H: int, dI: int) -> int:
    return int(load().lsa_focal_bce_grad_workspace_bytes(Q, N, D, H, dI))


def lsa_focal_bce_grad(h, Wq, Wg, bias, K, label, gamma, loss, dWq, ws=None, *, H: int,
                       dI: int, stream=None):
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
    _dtype(fn, "h", h, "bfloat16", "int16", "uint16")
    _dtype(fn, "K", K, "bfloat16", "int16", "uint16")
    for name, t in (("Wq", Wq), ("Wg", Wg), ("loss", loss), ("dWq", dWq)):
        _dtype(fn, name, t, "float32")
    _dtype(fn, "label", label, "uint8")
    _dev(h, Wq, Wg, K, label, loss, dWq, ws)
    check(load().lsa_focal_bce_grad(Q, N, D, H, dI, float(gamma), _p(h), _p(Wq), _p(Wg),
                                    float(bias), _p(K), _p(label), _p(loss), _p(dWq), _p(ws),
                                    0 if ws is None else ws.numel() * ws.element_size(),
                                    _stream(stream)))
