"""Device buffers for one indexer trigger and the call sequence of the hot
path (project -> score -> select/compact -> top-k -> gather), and the resident
set that survivors are fetched into from a host cold pool.  Allocation uses
torch; every step is one C entry point of liblsa.so."""
from __future__ import annotations

from dataclasses import dataclass

from . import (LSA_CAND_CHUNK, lsa_fetch_survivors, lsa_fetch_workspace_bytes, lsa_gather_hot,
               lsa_gather_resident, lsa_pack_query_weights, lsa_project_query,
               lsa_project_query_packed, lsa_query_weights_packed_bytes, lsa_resident_reset,
               lsa_score, lsa_select_or_compact, lsa_topk, lsa_topk_workspace_bytes)


@dataclass
class TriggerBuffers:
    N: int
    q: object
    g: object
    mask: object
    cand_idx: object
    cand_z: object
    cand_count: object
    surv_idx: object
    surv_z: object
    surv_count: object
    ws_topk: object
    topk_idx: object
    topk_count: object
    hot: object

    @classmethod
    def allocate(cls, L, B, N, H, dI, k, row_elems=512, cap=None, device="cuda"):
        import torch
        cap = N if cap is None else cap
        W = (N + 31) // 32
        nch = (N + LSA_CAND_CHUNK - 1) // LSA_CAND_CHUNK
        u8 = torch.uint8
        return cls(
            N=N,
            q=torch.empty((L, B, H, dI), dtype=torch.bfloat16, device=device),
            g=torch.empty((L, B, H), dtype=torch.float32, device=device),
            mask=torch.empty((L, B, W), dtype=torch.int32, device=device),
            cand_idx=torch.empty((B, nch, LSA_CAND_CHUNK), dtype=torch.int32, device=device),
            cand_z=torch.empty((B, nch, LSA_CAND_CHUNK), dtype=torch.float32, device=device),
            cand_count=torch.empty((B, nch), dtype=torch.int32, device=device),
            surv_idx=torch.empty((B, cap), dtype=torch.int32, device=device),
            surv_z=torch.empty((B, cap), dtype=torch.float32, device=device),
            surv_count=torch.empty((B,), dtype=torch.int32, device=device),
            ws_topk=torch.empty((max(1, lsa_topk_workspace_bytes(B, cap, k)),), dtype=u8,
                                device=device),
            topk_idx=torch.empty((B, k), dtype=torch.int32, device=device),
            topk_count=torch.empty((B,), dtype=torch.int32, device=device),
            hot=torch.empty((B, k, max(row_elems, 8)), dtype=torch.int16, device=device),
        )


def pack_weights(Wq, Wg, stream=None):
    """Packed copies (one uint8 buffer per layer) of the query weights, for
    lsa_project_query_packed; done once, when the weights are loaded."""
    import torch
    out = []
    for wq, wg in zip(Wq, Wg):
        H, D = wg.shape
        p = torch.empty(lsa_query_weights_packed_bytes(H, wq.shape[0] // H, D), dtype=torch.uint8,
                        device=wq.device)
        lsa_pack_query_weights(wq, wg, p, stream=stream)
        out.append(p)
    return out


def run_trigger(buf: TriggerBuffers, h, Wq, Wg, keys, key_scale, bias, pool=None, *,
                stream=None, project=True, z_layers=None, packed=None):
    """One indexer trigger.  With project=False the query buffers are used as
    they are (the caller filled buf.q / buf.g); with packed (pack_weights)
    the projection reads the packed weights.  z_layers: optional f32
    [L][B][N] that receives every layer's logit (extra write traffic)."""
    if project and packed is not None:
        lsa_project_query_packed(h, packed, buf.q, buf.g, stream=stream)
    elif project:
        lsa_project_query(h, Wq, Wg, buf.q, buf.g, stream=stream)
    lsa_score(keys, key_scale, buf.q, buf.g, bias, buf.mask, buf.cand_idx, buf.cand_z,
              buf.cand_count, z_layers, stream=stream)
    lsa_select_or_compact(buf.cand_idx, buf.cand_z, buf.cand_count, buf.N, buf.surv_idx,
                          buf.surv_z, buf.surv_count, stream=stream)
    lsa_topk(buf.surv_idx, buf.surv_z, buf.surv_count, buf.topk_idx, buf.topk_count,
             buf.ws_topk, stream=stream)
    if pool is not None:
        lsa_gather_hot(pool, buf.topk_idx, buf.hot, stream=stream)


@dataclass
class ResidentSet:
    """GPU-resident rows of a cold pool kept in pinned host memory: S slots
    per request and the two slot tables.  fetch() brings in the survivors of a
    trigger (rows already resident are reused), gather() copies top-k rows
    out of the set."""
    slot_of: object
    entry_of: object
    rows: object
    fetch_count: object
    ws: object

    @classmethod
    def allocate(cls, B, N, S, row_elems, cap=None, dtype=None, device="cuda", stream=None):
        import torch
        cap = N if cap is None else cap
        dtype = torch.int16 if dtype is None else dtype
        r = cls(slot_of=torch.empty((B, N), dtype=torch.int32, device=device),
                entry_of=torch.empty((B, S), dtype=torch.int32, device=device),
                rows=torch.empty((B, S, row_elems), dtype=dtype, device=device),
                fetch_count=torch.empty((B,), dtype=torch.int32, device=device),
                ws=torch.empty((max(1, lsa_fetch_workspace_bytes(B, N, cap)),),
                               dtype=torch.uint8, device=device))
        r.reset(stream)
        return r

    def reset(self, stream=None):
        """Nothing resident."""
        lsa_resident_reset(self.slot_of, self.entry_of, stream=stream)

    def fetch(self, cold_pool, surv_idx, surv_count, stream=None):
        """Survivors ([B][cap] ascending, counts [B]) into the set;
        fetch_count[b] = rows read from the cold pool, -1 if they do not fit."""
        lsa_fetch_survivors(cold_pool, surv_idx, surv_count, self.slot_of, self.entry_of,
                            self.rows, self.fetch_count, self.ws, stream=stream)

    def gather(self, idx, hot, stream=None):
        lsa_gather_resident(self.rows, self.slot_of, idx, hot, stream=stream)
