"""Device buffers for one indexer trigger and the call sequence of the hot
path (project -> score -> select/compact -> top-k -> gather), the resident set
that survivors are fetched into from a host cold pool, and a decode session
over caches that grow between triggers.  Allocation uses torch; every step is
one C entry point of liblsa.so."""
from __future__ import annotations

from dataclasses import dataclass

from . import (LSA_CAND_CHUNK, lsa_append_rows, lsa_fetch_survivors, lsa_fetch_workspace_bytes,
               lsa_gather_hot, lsa_gather_resident, lsa_lightning_score, lsa_pack_query_weights,
               lsa_project_query,
               lsa_project_query_packed, lsa_query_weights_packed_bytes, lsa_resident_reset,
               lsa_score, lsa_score_strided, lsa_select_or_compact, lsa_topk,
               lsa_topk_workspace_bytes)


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
                stream=None, project=True, z_layers=None, packed=None, fine=None):
    """One indexer trigger.  With project=False the query buffers are used as
    they are (the caller filled buf.q / buf.g); with packed (pack_weights)
    the projection reads the packed weights.  z_layers: optional f32
    [L][B][N] that receives every layer's logit (extra write traffic).
    fine: optional (keys, key_scale, q, w, score) of the fine-grained
    indexer; the top-k then ranks the survivors by lsa_lightning_score
    (written to score [B][cap]) instead of their merged logit."""
    if project and packed is not None:
        lsa_project_query_packed(h, packed, buf.q, buf.g, stream=stream)
    elif project:
        lsa_project_query(h, Wq, Wg, buf.q, buf.g, stream=stream)
    lsa_score(keys, key_scale, buf.q, buf.g, bias, buf.mask, buf.cand_idx, buf.cand_z,
              buf.cand_count, z_layers, stream=stream)
    lsa_select_or_compact(buf.cand_idx, buf.cand_z, buf.cand_count, buf.N, buf.surv_idx,
                          buf.surv_z, buf.surv_count, stream=stream)
    rank = buf.surv_z
    if fine is not None:
        fk, fs, fq, fw, rank = fine
        lsa_lightning_score(fk, fs, fq, fw, buf.surv_idx, buf.surv_count, rank, stream=stream)
    lsa_topk(buf.surv_idx, rank, buf.surv_count, buf.topk_idx, buf.topk_count, buf.ws_topk,
             stream=stream)
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


class StreamingSession:
    """Decode-time indexer state of B requests whose compressed caches keep
    growing: per-layer key caches of N_cap entries per request (the first N
    live), a host cold pool of KV rows and the GPU-resident set fetched from it.

    append() adds entries to the caches (lsa_append_rows); trigger() runs one
    lookahead trigger over the live entries (project -> score the first N ->
    OR/compact -> top-k -> fetch the survivors, reusing rows already resident ->
    gather the top-k rows into `hot`); decode() is the host loop over decode
    steps that triggers at lsa_trigger_due(t, tau) and appends the entries of
    each finished window before the trigger, so the trigger at step t sees
    N0 + (t // tau) * per_window entries.  Steps between triggers reuse `hot`.
    Every computation is a C entry point; torch only allocates."""

    def __init__(self, L, B, N_cap, H, dI, k, row_elems, S, cold_pool, key_dtype="bf16",
                 tau=64, per_window=16, device="cuda"):
        import torch
        from . import lsa_trigger_due  # noqa: F401  (the cadence is the library's)
        self.L, self.B, self.N_cap, self.H, self.dI, self.k = L, B, N_cap, H, dI, k
        self.tau, self.per_window, self.N = tau, per_window, 0
        self.fp8 = key_dtype == "e4m3"
        kdt = torch.uint8 if self.fp8 else torch.bfloat16
        self.keys = [torch.zeros((B, N_cap, dI), dtype=kdt, device=device) for _ in range(L)]
        self.scale = ([torch.zeros((B, N_cap), dtype=torch.float32, device=device)
                       for _ in range(L)] if self.fp8 else None)
        self.cold = cold_pool
        W_cap = (N_cap + 31) // 32
        nch_cap = (N_cap + LSA_CAND_CHUNK - 1) // LSA_CAND_CHUNK
        # flat capacity buffers; each trigger views their leading part with the
        # shapes of the live N (the kernels index them densely by N)
        self._mask = torch.empty(L * B * W_cap, dtype=torch.int32, device=device)
        self._cidx = torch.empty(B * nch_cap * LSA_CAND_CHUNK, dtype=torch.int32, device=device)
        self._cz = torch.empty(B * nch_cap * LSA_CAND_CHUNK, dtype=torch.float32, device=device)
        self._cc = torch.empty(B * nch_cap, dtype=torch.int32, device=device)
        self.q = torch.empty((L, B, H, dI), dtype=torch.bfloat16, device=device)
        self.g = torch.empty((L, B, H), dtype=torch.float32, device=device)
        self.surv_idx = torch.empty((B, N_cap), dtype=torch.int32, device=device)
        self.surv_z = torch.empty((B, N_cap), dtype=torch.float32, device=device)
        self.surv_count = torch.empty((B,), dtype=torch.int32, device=device)
        self.ws_topk = torch.empty((max(1, lsa_topk_workspace_bytes(B, N_cap, k)),),
                                   dtype=torch.uint8, device=device)
        self.topk_idx = torch.empty((B, k), dtype=torch.int32, device=device)
        self.topk_count = torch.empty((B,), dtype=torch.int32, device=device)
        self.hot = torch.zeros((B, k, row_elems), dtype=cold_pool.dtype, device=device)
        self.res = ResidentSet.allocate(B, N_cap, S, row_elems, dtype=cold_pool.dtype,
                                        device=device)
        self.triggers = []   # (step, N, survivors per request)

    def append(self, new_keys, new_scale=None, stream=None):
        """New entries of every request: new_keys list of L [B][n][dI] (and
        new_scale list of L [B][n] for e4m3 keys), appended after the live
        ones."""
        n = new_keys[0].shape[1]
        if self.N + n > self.N_cap:
            raise ValueError(f"the caches hold {self.N_cap} entries; {self.N} + {n} do not fit")
        for l in range(self.L):
            lsa_append_rows(new_keys[l], self.keys[l], self.N, stream=stream)
            if self.fp8:
                lsa_append_rows(new_scale[l], self.scale[l], self.N, stream=stream)
        self.N += n

    def _views(self):
        N, L, B = self.N, self.L, self.B
        W = (N + 31) // 32
        nch = (N + LSA_CAND_CHUNK - 1) // LSA_CAND_CHUNK
        return (self._mask[:L * B * W].view(L, B, W),
                self._cidx[:B * nch * LSA_CAND_CHUNK].view(B, nch, LSA_CAND_CHUNK),
                self._cz[:B * nch * LSA_CAND_CHUNK].view(B, nch, LSA_CAND_CHUNK),
                self._cc[:B * nch].view(B, nch))

    def trigger(self, h, packed, bias, stream=None):
        """One lookahead trigger over the N live entries (h bf16 [B][D])."""
        mask, cidx, cz, cc = self._views()
        lsa_project_query_packed(h, packed, self.q, self.g, stream=stream)
        lsa_score_strided(self.keys, self.scale, self.q, self.g, bias, self.N, mask, cidx, cz,
                          cc, stream=stream)
        lsa_select_or_compact(cidx, cz, cc, self.N, self.surv_idx, self.surv_z, self.surv_count,
                              stream=stream)
        lsa_topk(self.surv_idx, self.surv_z, self.surv_count, self.topk_idx, self.topk_count,
                 self.ws_topk, stream=stream)
        self.res.fetch(self.cold, self.surv_idx, self.surv_count, stream=stream)
        self.res.gather(self.topk_idx, self.hot, stream=stream)

    def decode(self, T, hidden_of, packed, bias, window_source, on_trigger=None, on_step=None,
               stream=None):
        """Decode steps [0, T): at every step with lsa_trigger_due(t, tau) the
        entries of the window that just ended are appended
        (window_source(i) -> (new_keys, new_scale) for trigger i >= 1) and the
        trigger runs on hidden_of(i); on_trigger(i, t) after each trigger,
        on_step(t) after every step (e.g. the core attention on `hot`)."""
        from . import lsa_trigger_due
        i = 0
        for t in range(T):
            if lsa_trigger_due(t, self.tau):
                if i > 0:
                    nk, ns = window_source(i)
                    self.append(nk, ns, stream=stream)
                self.trigger(hidden_of(i), packed, bias, stream=stream)
                if on_trigger is not None:
                    on_trigger(i, t)
                i += 1
            if on_step is not None:
                on_step(t)
        return i
