"""ctypes loader of liblsa.so (the gfx950 LSA indexer library).

There is no fallback: if the library is missing, every call raises."""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblsa.so")

LSA_OK, LSA_E_ARG, LSA_E_SHAPE, LSA_E_DTYPE, LSA_E_HIP, LSA_E_WORKSPACE = range(6)
LSA_KEY_BF16, LSA_KEY_FP8_E4M3 = 0, 1
LSA_CAND_CHUNK = 4096
LSA_TOPK_NOALLOC_MAX_BYTES = 16 << 20
LSA_ATT_ROW = 512
STATUS_NAMES = {0: "LSA_OK", 1: "LSA_E_ARG", 2: "LSA_E_SHAPE", 3: "LSA_E_DTYPE",
                4: "LSA_E_HIP", 5: "LSA_E_WORKSPACE"}

P = C.c_void_p
I32 = C.c_int
I64 = C.c_int64
SZ = C.c_size_t
PP = C.POINTER(C.c_void_p)
PF = C.POINTER(C.c_float)

# name -> (restype, argtypes), mirroring include/lsa.h
SIGNATURES = {
    "lsa_last_error": (C.c_char_p, []),
    "lsa_version": (C.c_char_p, []),
    "lsa_trigger_due": (I32, [I64, I32]),
    "lsa_project_query": (I32, [I32, I32, I32, I32, I32, P, I64, PP, PP, P, P, P]),
    "lsa_query_weights_packed_bytes": (SZ, [I32, I32, I32]),
    "lsa_pack_query_weights": (I32, [I32, I32, I32, P, P, P, P]),
    "lsa_project_query_packed": (I32, [I32, I32, I32, I32, I32, P, I64, PP, P, P, P]),
    "lsa_score": (I32, [I32, I32, I32, I32, I32, I32, PP, PP, P, P, P, P, P, P, P, P, P, P]),
    "lsa_score_strided": (I32, [I32, I32, I32, I64, I32, I32, I32, PP, PP, P, P, P, P, P, P, P, P,
                                P, P]),
    "lsa_append_rows": (I32, [I32, I32, I32, P, I64, P, I64, I64, P]),
    "lsa_select_or_compact": (I32, [I32, I32, P, P, P, I32, P, P, P, P]),
    "lsa_select_or_compact_masks_workspace_bytes": (SZ, [I32, I32]),
    "lsa_select_or_compact_masks": (I32, [I32, I32, I32, P, P, I32, P, P, P, P, SZ, P]),
    "lsa_topk_workspace_bytes": (SZ, [I32, I32, I32]),
    "lsa_topk": (I32, [I32, I32, I32, P, P, P, P, P, P, SZ, P]),
    "lsa_topk_noalloc": (I32, [I32, I32, I32, P, P, P, P, P, P]),
    "lsa_lightning_score": (I32, [I32, I32, I32, I32, I32, I32, P, P, P, P, P, P, P, P]),
    "lsa_gather_hot": (I32, [I32, I32, I32, I32, P, P, P, P]),
    "lsa_sparse_attention_workspace_bytes": (SZ, [I32, I32, I32, I32, I32]),
    "lsa_sparse_attention": (I32, [I32, I32, I32, I32, I32, C.c_float, P, P, P, P, P, P, P, SZ,
                                   P]),
    "lsa_fetch_workspace_bytes": (SZ, [I32, I32, I32]),
    "lsa_resident_reset": (I32, [I32, I32, I32, P, P, P]),
    "lsa_fetch_survivors": (I32, [I32, I32, I32, I32, P, I32, P, P, P, P, P, P, P, SZ, P]),
    "lsa_gather_resident": (I32, [I32, I32, I32, I32, I32, P, P, P, P, P]),
    "lsa_label_vote_workspace_bytes": (SZ, [I32, I32, I32]),
    "lsa_label_vote": (I32, [I32, I32, I32, C.c_float, I32, P, P, P, P, P, SZ, P]),
    "lsa_focal_bce_grad_workspace_bytes": (SZ, [I32, I32, I32, I32, I32]),
    "lsa_focal_bce_grad": (I32, [I32, I32, I32, I32, I32, C.c_float, P, P, P, C.c_float, P, P,
                                 P, P, P, SZ, P]),
}

_lib = None


class LSAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def mapped_runtimes(names=("libamdhip64", "libhsa-runtime64", "libgomp")):
    """Files of the HIP, HSA and OpenMP runtimes mapped into this process,
    by runtime name (read from /proc/self/maps)."""
    found = {n: set() for n in names}
    try:
        with open("/proc/self/maps") as f:
            for ln in f:
                parts = ln.split()
                if len(parts) < 6:
                    continue
                base = os.path.basename(parts[-1])
                for n in names:
                    if base.startswith(n + "."):
                        found[n].add(os.path.realpath(parts[-1]))
    except OSError:
        pass
    return found


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m sparse_kv_cache_lsa_amd.build`")
    # torch ships its own HIP and HSA runtimes (sonames libamdhip64.so.7 and
    # libhsa-runtime64.so.1, the ones liblsa.so needs).  Loading torch first
    # lets the dynamic loader bind liblsa.so to those already-loaded copies;
    # loading liblsa.so first would map the system runtimes as well, and two
    # HIP runtimes in one process do not share streams, devices or code
    # objects.  So torch is imported here, and the process is checked for
    # exactly one HIP runtime.
    import torch  # noqa: F401
    lib = C.CDLL(LIB_PATH)
    hip = mapped_runtimes(("libamdhip64",))["libamdhip64"]
    if len(hip) > 1:
        raise RuntimeError("two HIP runtimes are mapped in this process (" + ", ".join(sorted(hip)) +
                           "): load liblsa.so only through this module, after torch")
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(status: int):
    if status != LSA_OK:
        msg = load().lsa_last_error().decode(errors="replace")
        raise LSAError(status, msg)


def ptr_array(ptrs):
    arr = (C.c_void_p * len(ptrs))(*[C.c_void_p(p) for p in ptrs])
    return C.cast(arr, PP), arr
