"""ctypes wrapper of the plain CPU oracle (``lsa_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark.  The product library never imports it.

Every function takes and returns numpy arrays.  Storage formats follow the
boundary: bf16 is passed as ``uint16`` bit patterns, e4m3 as ``uint8`` codes.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblsa_oracle.so")
# A test may point the wrapper at another build of the oracle source (the
# mutation tests build copies with one planted mistake each).
_ALT_LIB = os.environ.get("LSA_ORACLE_LIB")
_lib = None


GCC_FLAGS = ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
             "-ffp-contract=off"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, IEEE semantics kept)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", *GCC_FLAGS, "-I", _HERE, _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # One OpenMP runtime per process: torch carries its own libgomp (soname
    # libgomp.so.1, the one this library needs).  With torch loaded first the
    # dynamic loader binds this library to that copy; loaded the other way
    # round, the process maps the system libgomp as well, and two OpenMP
    # runtimes in one process each start their own thread pools.
    import torch  # noqa: F401
    if _ALT_LIB:
        lib = C.CDLL(_ALT_LIB)
    else:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = C.CDLL(_LIB_PATH)
    P = C.c_void_p
    i32, i64, f64 = C.c_int, C.c_int64, C.c_double
    sig = {
        "lsa_or_bf16_to_double": (f64, [C.c_uint16]),
        "lsa_or_bf16_from_double": (C.c_uint16, [f64]),
        "lsa_or_e4m3_to_double": (f64, [C.c_uint8]),
        "lsa_or_softplus": (f64, [f64]),
        "lsa_or_sigmoid": (f64, [f64]),
        "lsa_or_project": (None, [i32, i32, i32, P, P, P, P, P, P]),
        "lsa_or_query_collapse": (None, [i32, i32, P, P, P]),
        "lsa_or_score": (None, [i32, i32, i32, i32, P, P, P, P, f64, P, i64, P]),
        "lsa_or_threshold": (None, [i64, P, P]),
        "lsa_or_merge_compact": (i64, [i32, i64, P, P, i64, P, P]),
        "lsa_or_topk": (i64, [i64, P, P, i64, P]),
        "lsa_or_gather": (None, [i64, i64, P, i64, P, P]),
        "lsa_or_fetch": (i64, [i64, i64, i64, P, i64, P, P, P, P]),
        "lsa_or_nucleus": (i64, [i64, P, f64, P, P]),
        "lsa_or_vote": (None, [i32, i64, P, i32, P, P]),
        "lsa_or_focal_bce_grad": (f64, [i32, i64, i32, i32, i32, f64, P, P, P, f64, P, P, P, P]),
        "lsa_or_focal_bce_loss64": (f64, [i32, i64, i32, i32, i32, f64, P, P, P, f64, P, P]),
        "lsa_or_num_threads": (i32, []),
        "lsa_or_set_num_threads": (None, [i32]),
        "lsa_or_trigger_due": (i32, [i64, i32]),
        "lsa_or_attention": (None, [i64, i32, i32, P, P, f64, P, P]),
        "lsa_or_lightning": (None, [i32, i32, i32, i32, P, P, P, P, P, i64, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---- storage formats ------------------------------------------------------

def bf16_to_double(bits) -> np.ndarray:
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([lib.lsa_or_bf16_to_double(int(v)) for v in b]).reshape(np.shape(bits))


def bf16_from_double(a) -> np.ndarray:
    lib = _load()
    x = np.asarray(a, dtype=np.float64).ravel()
    return np.array([lib.lsa_or_bf16_from_double(float(v)) for v in x],
                    dtype=np.uint16).reshape(np.shape(a))


def e4m3_to_double(codes) -> np.ndarray:
    lib = _load()
    c = np.asarray(codes, dtype=np.uint8).ravel()
    return np.array([lib.lsa_or_e4m3_to_double(int(v)) for v in c]).reshape(np.shape(codes))


def softplus(x: float) -> float:
    return _load().lsa_or_softplus(float(x))


def sigmoid(x: float) -> float:
    return _load().lsa_or_sigmoid(float(x))


def trigger_due(t: int, tau: int) -> bool:
    return bool(_load().lsa_or_trigger_due(int(t), int(tau)))


def num_threads() -> int:
    return _load().lsa_or_num_threads()


def set_num_threads(n: int) -> None:
    """Threads of the oracle's parallel loops (for timing on one core)."""
    _load().lsa_or_set_num_threads(int(n))


# ---- O1 projection ----------------------------------------------------------

def project(h, Wq, Wg, H: int, dI: int, want_a: bool = False):
    """One (layer, request): h bf16 [D], Wq bf16 [H*dI][D], Wg bf16 [H][D].
    Returns q (uint16 [H][dI]), g (float32 [H]) and optionally a (fp64)."""
    lib = _load()
    h = _c(h, np.uint16)
    Wq = _c(Wq, np.uint16)
    Wg = _c(Wg, np.uint16)
    D = h.shape[-1]
    q = np.empty(H * dI, np.uint16)
    g = np.empty(H, np.float32)
    a = np.empty(H * dI, np.float64) if want_a else None
    lib.lsa_or_project(D, H, dI, _p(h), _p(Wq), _p(Wg), _p(q), _p(g), _p(a))
    q = q.reshape(H, dI)
    return (q, g, a.reshape(H, dI)) if want_a else (q, g)


def query_collapse(q, g) -> np.ndarray:
    lib = _load()
    q = _c(q, np.uint16)
    g = _c(g, np.float32)
    H, dI = q.shape
    out = np.empty(dI, np.float64)
    lib.lsa_or_query_collapse(H, dI, _p(q), _p(g), _p(out))
    return out


# ---- O3 score / O4 threshold / O5 merge ----------------------------------

def score(keys, scale, q, g, bias: float, idx=None) -> np.ndarray:
    """keys: uint16 [N][dI] (bf16) or uint8 [N][dI] (e4m3, with scale f32 [N]).
    Returns fp64 z for all entries, or for the entries listed in idx."""
    lib = _load()
    key_dtype = 0 if keys.dtype == np.uint16 else 1
    keys = np.ascontiguousarray(keys)
    N, dI = keys.shape
    q = _c(q, np.uint16)
    g = _c(g, np.float32)
    H = q.shape[0]
    sc = _c(scale, np.float32) if scale is not None else None
    if idx is not None:
        idx = _c(idx, np.int64)
        n = idx.shape[0]
    else:
        n = N
    z = np.empty(n, np.float64)
    lib.lsa_or_score(N, H, dI, key_dtype, _p(keys), _p(sc), _p(q), _p(g),
                     float(bias), _p(idx), n, _p(z))
    return z


def threshold(z) -> np.ndarray:
    lib = _load()
    z = _c(z, np.float64)
    sel = np.empty(z.shape, np.uint8)
    lib.lsa_or_threshold(z.size, _p(z), _p(sel))
    return sel


def merge_compact(sel, z, cap: int | None = None):
    """sel uint8 [L][N], z fp64 [L][N] -> (idx int32 [min(count,cap)],
    zstar fp64, true count)."""
    lib = _load()
    sel = _c(sel, np.uint8)
    z = _c(z, np.float64)
    L, N = sel.shape
    if cap is None:
        cap = N
    idx = np.empty(max(cap, 1), np.int32)
    zs = np.empty(max(cap, 1), np.float64)
    count = lib.lsa_or_merge_compact(L, N, _p(sel), _p(z), cap, _p(idx), _p(zs))
    m = min(count, cap)
    return idx[:m].copy(), zs[:m].copy(), int(count)


def topk(surv_idx, surv_z, k: int):
    lib = _load()
    si = _c(surv_idx, np.int32)
    sz = _c(surv_z, np.float64)
    out = np.empty(max(k, 1), np.int32)
    cnt = lib.lsa_or_topk(si.shape[0], _p(si), _p(sz), k, _p(out))
    return out[:k].copy(), int(cnt)


def gather(pool, idx) -> np.ndarray:
    """pool: uint8 [N][row_bytes]; idx int32 [k] -> uint8 [k][row_bytes]."""
    lib = _load()
    pool = _c(pool, np.uint8)
    idx = _c(idx, np.int32)
    N, rb = pool.shape
    hot = np.empty((idx.shape[0], rb), np.uint8)
    lib.lsa_or_gather(N, rb, _p(pool), idx.shape[0], _p(idx), _p(hot))
    return hot


# ---- O10 cold-pool fetch ------------------------------------------------------

def fetch(cold, surv, slot_of, entry_of, rows) -> int:
    """One request, in place.  cold uint8 [N][row_bytes] (the cold pool);
    surv int32 [n] ascending survivors; slot_of int32 [N], entry_of int32 [S],
    rows uint8 [S][row_bytes] (the resident set, updated in place).  Returns
    the number of rows copied, or -1 if the free slots do not suffice."""
    lib = _load()
    cold = _c(cold, np.uint8)
    surv = _c(surv, np.int32)
    for a, dt in ((slot_of, np.int32), (entry_of, np.int32), (rows, np.uint8)):
        if a.dtype != dt or not a.flags.c_contiguous:
            raise ValueError("fetch updates slot_of/entry_of/rows in place: pass contiguous arrays")
    N, rb = cold.shape
    S = entry_of.shape[0]
    assert slot_of.shape == (N,) and rows.shape == (S, rb)
    return int(lib.lsa_or_fetch(N, S, rb, _p(cold), surv.shape[0], _p(surv), _p(slot_of),
                                _p(entry_of), _p(rows)))


def gather_resident(rows, slot_of, idx) -> np.ndarray:
    """Rows of the resident set for entry indices idx (zero row for idx < 0 or
    an entry not resident)."""
    idx = np.asarray(idx, np.int64)
    slot = np.full(idx.shape, -1, np.int32)
    ok = idx >= 0
    slot[ok] = slot_of[idx[ok]]
    return gather(rows, slot)


# ---- O8 labels -------------------------------------------------------------

def nucleus(x, top_p: float, want_mass: bool = False):
    lib = _load()
    x = _c(x, np.float32)
    N = x.shape[0]
    sel = np.empty(N, np.uint8)
    mass = np.empty(N, np.float64) if want_mass else None
    n = lib.lsa_or_nucleus(N, _p(x), float(top_p), _p(sel), _p(mass))
    return (sel, int(n), mass) if want_mass else (sel, int(n))


def vote(sel, theta: int):
    lib = _load()
    sel = _c(sel, np.uint8)
    L, N = sel.shape
    count = np.empty(N, np.uint8)
    label = np.empty(N, np.uint8)
    lib.lsa_or_vote(L, N, _p(sel), int(theta), _p(count), _p(label))
    return count, label


# ---- O9 loss / gradient --------------------------------------------------

def focal_bce_grad(h, Wq, Wg, bias: float, K, y, gamma: float, H: int, dI: int,
                   want_grad: bool = True, want_z: bool = False):
    """h bf16 [Q][D], Wq f32 [H*dI][D], Wg f32 [H][D], K bf16 [N][dI], y u8 [Q][N]."""
    lib = _load()
    h = _c(h, np.uint16)
    Wq = _c(Wq, np.float32)
    Wg = _c(Wg, np.float32)
    K = _c(K, np.uint16)
    y = _c(y, np.uint8)
    Q, D = h.shape
    N = K.shape[0]
    dW = np.empty((H * dI, D), np.float64) if want_grad else None
    z = np.empty((Q, N), np.float64) if want_z else None
    loss = lib.lsa_or_focal_bce_grad(Q, N, D, H, dI, float(gamma), _p(h), _p(Wq),
                                     _p(Wg), float(bias), _p(K), _p(y), _p(dW), _p(z))
    return loss, dW, z


def focal_bce_loss64(h, Wq, Wg, bias: float, K, y, gamma: float, H: int, dI: int) -> float:
    lib = _load()
    h = _c(h, np.float64)
    Wq = _c(Wq, np.float64)
    Wg = _c(Wg, np.float64)
    K = _c(K, np.float64)
    y = _c(y, np.uint8)
    Q, D = h.shape
    N = K.shape[0]
    return lib.lsa_or_focal_bce_loss64(Q, N, D, H, dI, float(gamma), _p(h), _p(Wq),
                                       _p(Wg), float(bias), _p(K), _p(y))


def attention(q, rows, scale: float, want_wabs: bool = False):
    """Core attention of one request: q bf16 [H][D], rows bf16 [n][D] (each
    row both key and value) -> out fp64 [H][D] (and optionally
    sum_j p_j |row_j| / sum_j p_j, [H][D])."""
    lib = _load()
    q = _c(q, np.uint16)
    rows = _c(rows, np.uint16)
    H, D = q.shape
    n = rows.shape[0] if rows.size else 0
    if n:
        assert rows.shape[1] == D
    out = np.empty((H, D), np.float64)
    wabs = np.empty((H, D), np.float64) if want_wabs else None
    lib.lsa_or_attention(n, D, H, _p(q), _p(rows) if n else None, float(scale), _p(out),
                         _p(wabs))
    return (out, wabs) if want_wabs else out



def lightning(keys, scale, q, w, idx) -> np.ndarray:
    """Fine-grained score of the entries idx: keys [N][dI] (bf16 bits, or
    e4m3 codes with scale fp32 [N]), q bf16 [H][dI], w fp32 [H] ->
    sum_h w_h * relu(q_h . k_s * sigma_s), fp64 [n]."""
    lib = _load()
    kdt = 0 if keys.dtype == np.uint16 else 1
    keys = np.ascontiguousarray(keys)
    q = _c(q, np.uint16)
    w = _c(w, np.float32)
    idx = _c(idx, np.int32)
    H, dI = q.shape
    out = np.empty(max(idx.shape[0], 1), np.float64)
    sc = None if scale is None else _c(scale, np.float32)
    lib.lsa_or_lightning(keys.shape[0], H, dI, kdt, _p(keys), _p(sc), _p(q), _p(w), _p(idx),
                         idx.shape[0], _p(out))
    return out[:idx.shape[0]].copy()

# ---- O12 decode session over a growing key cache --------------------------

def stream_session(keys, scale, queries, bias, N0: int, tau: int, T: int, per_window: int,
                   k: int, cold=None, S: int = 0):
    """One request of a decode session (gist.science technical summary, 2.1,
    periodic-trigger and dynamic-fetch bullets; paper.oopus.info review,
    section 2: every tau steps the indexer looks ahead over every entry
    compressed so far).

    keys: list of L arrays [N_cap][dI] (bf16 bits or e4m3 codes) holding every
    entry the session will have; scale: list of L fp32 [N_cap] (e4m3) or None.
    The cache holds N0 entries at step 0 and per_window more after each
    window of tau steps (the entries compressed from that window's tokens),
    so at step t it holds N0 + (t // tau) * per_window entries.  At every step
    t in [0, T) with trigger_due(t, tau) the indexer scores the entries
    present then: queries(i) gives the i-th trigger's (q [L][H][dI] bf16 bits,
    g [L][H] fp32); bias [L].

    With cold (uint8 [N_cap][row_bytes], the cold pool) and S slots, each
    trigger fetches its survivors into the resident set (fetch: rows still
    resident are kept) and gathers its top-k rows from it.

    Returns one dict per trigger: step, N, z (fp64 [L][N]), survivors, zstar,
    count, topk, kcount and, with cold: fetched, slot_of, entry_of, hot."""
    L = len(keys)
    N_cap = keys[0].shape[0]
    out = []
    if cold is not None:
        slot_of = np.full(N_cap, -1, np.int32)
        entry_of = np.full(S, -1, np.int32)
        rows = np.zeros((S, cold.shape[1]), np.uint8)
    i = 0
    for t in range(T):
        if not trigger_due(t, tau):
            continue
        N = N0 + (t // tau) * per_window
        assert N <= N_cap, "the session needs more entries than the cache holds"
        q, g = queries(i)
        z = np.stack([score(keys[l][:N], None if scale is None or scale[l] is None
                            else scale[l][:N], q[l], g[l], float(bias[l])) for l in range(L)])
        surv, zstar, count = merge_compact(threshold(z), z)
        top, kc = topk(surv, zstar, k)
        rec = {"step": t, "N": N, "z": z, "survivors": surv, "zstar": zstar, "count": count,
               "topk": top, "kcount": kc}
        if cold is not None:
            rec["fetched"] = fetch(cold, surv, slot_of, entry_of, rows)
            rec["slot_of"] = slot_of.copy()
            rec["entry_of"] = entry_of.copy()
            rec["hot"] = gather_resident(rows, slot_of, top[:kc])
        out.append(rec)
        i += 1
    return out
