"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and its host-only logic (trigger cadence, workspace sizes,
argument validation that returns before any launch) behaves as documented."""
import ctypes as C
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lsa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lsa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from sparse_kv_cache_lsa_amd import _abi
    if not os.path.exists(_abi.LIB_PATH):
        from sparse_kv_cache_lsa_amd import build
        build.build()
    return _abi.load()


def test_header_symbols_exported(lib):
    names = _declared()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), f"{n} declared in lsa.h but not exported"
    from sparse_kv_cache_lsa_amd import _abi
    assert set(names) == set(_abi.SIGNATURES), "binding signatures out of sync with lsa.h"


def test_binding_names_match_entry_points():
    import sparse_kv_cache_lsa_amd as pkg
    for n in _declared():
        if n in ("lsa_last_error",):
            continue
        assert hasattr(pkg, n), f"python binding lacks {n}"


def test_trigger_cadence(lib):
    due = [t for t in range(300) if lib.lsa_trigger_due(t, 64)]
    assert due == [0, 64, 128, 192, 256]
    for T in (1, 64, 65, 1000):
        assert sum(lib.lsa_trigger_due(t, 64) for t in range(T)) == math.ceil(T / 64)
    assert lib.lsa_trigger_due(-64, 64) == 0 and lib.lsa_trigger_due(5, 0) == 0


def test_trigger_due_matches_oracle(lib):
    # the library's cadence against the oracle's, over negative steps, step 0
    # and many windows, for several periods (tau <= 0: never due)
    from oracle import oracle
    for tau in (1, 2, 3, 16, 64, 100, 0, -1):
        for t in range(-64, 10_000):
            assert lib.lsa_trigger_due(t, tau) == int(oracle.trigger_due(t, tau)), (t, tau)


def _status(lib, name, *args):
    return getattr(lib, name)(*args)


def test_validation_errors_return_before_launch(lib):
    from sparse_kv_cache_lsa_amd import _abi
    P = None
    fake = C.c_void_p(16)   # never dereferenced: validation fails first
    arr, _keep = _abi.ptr_array([16])
    bias = (C.c_float * 1)(0.0)
    # bad dtype
    st = lib.lsa_score(1, 1, 64, 8, 64, 7, arr, None, fake, fake, bias, fake, fake, fake, fake, None, None, None)
    assert st == _abi.LSA_E_DTYPE and b"dtype" in lib.lsa_last_error()
    # unsupported head dim
    st = lib.lsa_score(1, 1, 64, 8, 96, 0, arr, None, fake, fake, bias, fake, fake, fake, fake, None, None, None)
    assert st == _abi.LSA_E_SHAPE and b"dI" in lib.lsa_last_error()
    # too many heads, too many layers
    assert lib.lsa_score(1, 1, 64, 65, 64, 0, arr, None, fake, fake, bias, fake, fake, fake, fake, None, None, None) == _abi.LSA_E_SHAPE
    assert lib.lsa_score(9, 1, 64, 8, 64, 0, arr, None, fake, fake, bias, fake, fake, fake, fake, None, None, None) == _abi.LSA_E_SHAPE
    # bf16 keys of one (layer, request) at 2^31 bytes: N = 2^23, dI = 128
    assert lib.lsa_score(1, 1, 1 << 23, 8, 128, 0, arr, None, fake, fake, bias, fake, fake, fake, fake, None, None, None) == _abi.LSA_E_SHAPE
    # e4m3 without scales
    assert lib.lsa_score(1, 1, 64, 8, 64, 1, arr, None, fake, fake, bias, fake, fake, fake, fake, None, None, None) == _abi.LSA_E_ARG
    # null output
    assert lib.lsa_score(1, 1, 64, 8, 64, 0, arr, None, fake, fake, bias, fake, P, fake, fake, None, None, None) == _abi.LSA_E_ARG
    # misaligned query
    assert lib.lsa_score(1, 1, 64, 8, 64, 0, arr, None, C.c_void_p(18), fake, bias, fake, fake, fake, fake, None, None, None) == _abi.LSA_E_ARG
    # select: negative capacity, missing candidate lists
    assert lib.lsa_select_or_compact(2, 1000, fake, fake, fake, -1, fake, fake, fake, None) == _abi.LSA_E_ARG
    assert lib.lsa_select_or_compact(2, 1000, None, fake, fake, 10, fake, fake, fake, None) == _abi.LSA_E_ARG
    # top-k: negative k; long lists need the workspace
    assert lib.lsa_topk(1, 10, -1, fake, fake, fake, fake, fake, None, 0, None) == _abi.LSA_E_ARG
    assert lib.lsa_topk_workspace_bytes(2, 100000, 2048) > 0
    assert lib.lsa_topk(2, 100000, 2048, fake, fake, fake, fake, fake, None, 0, None) == _abi.LSA_E_WORKSPACE
    # top-k on the library's scratch: sizes past its capacity are refused
    # before anything is resolved or launched
    big = (200, 262144, 2048)
    assert lib.lsa_topk_workspace_bytes(*big) > _abi.LSA_TOPK_NOALLOC_MAX_BYTES
    assert lib.lsa_topk_noalloc(*big, fake, fake, fake, fake, fake, None) == _abi.LSA_E_SHAPE
    assert b"scratch" in lib.lsa_last_error()
    assert lib.lsa_topk_noalloc(1, 10, -1, fake, fake, fake, fake, fake, None) == _abi.LSA_E_ARG
    # gather: row size not a multiple of 16
    assert lib.lsa_gather_hot(1, 10, 4, 24, fake, fake, fake, None) == _abi.LSA_E_ARG
    # fetch: bad sizes, bad row size, short workspace, pageable cold pool
    Fe = lambda B, N, S, rb, cap, cold=fake, ws=fake, nws=1 << 30: lib.lsa_fetch_survivors(
        B, N, S, rb, cold, cap, fake, fake, fake, fake, fake, fake, ws, nws, None)
    assert Fe(2, 1000, -1, 1024, 100) == _abi.LSA_E_SHAPE
    assert Fe(2, 1 << 25, 10, 1024, 100) == _abi.LSA_E_SHAPE
    assert Fe(65535, 1 << 20, 1 << 16, 16, 1 << 20) == _abi.LSA_E_SHAPE   # 2^32 rows
    assert Fe(2, 1000, 100, 24, 100) == _abi.LSA_E_ARG
    assert Fe(2, 1000, 100, 1024, 100, cold=None) == _abi.LSA_E_ARG
    assert Fe(2, 1000, 100, 1024, 100, cold=C.c_void_p(24)) == _abi.LSA_E_ARG
    assert Fe(2, 1000, 100, 1024, 100, ws=None, nws=0) == _abi.LSA_E_WORKSPACE
    assert Fe(2, 1000, 100, 1024, 100, nws=8) == _abi.LSA_E_WORKSPACE
    pageable = (C.c_uint8 * 4096)()
    page = C.c_void_p((C.addressof(pageable) + 15) & ~15)
    assert Fe(1, 2, 2, 1024, 2, cold=page) == _abi.LSA_E_ARG
    assert b"cold pool" in lib.lsa_last_error()
    assert lib.lsa_resident_reset(0, 10, 10, fake, fake, None) == _abi.LSA_E_SHAPE
    assert lib.lsa_resident_reset(1, 10, 10, None, fake, None) == _abi.LSA_E_ARG
    assert lib.lsa_gather_resident(1, 10, 10, 4, 24, fake, fake, fake, fake, None) == _abi.LSA_E_ARG
    assert lib.lsa_gather_resident(1, 10, 10, 4, 32, None, fake, fake, fake, None) == _abi.LSA_E_ARG
    # projection: hidden size not a multiple of 64
    assert lib.lsa_project_query(1, 1, 100, 8, 64, fake, 0, arr, arr, fake, fake, None) == _abi.LSA_E_SHAPE
    # packed projection: bad D, null or misaligned packed buffers
    assert lib.lsa_project_query_packed(1, 1, 100, 8, 64, fake, 0, arr, fake, fake, None) == _abi.LSA_E_SHAPE
    assert lib.lsa_project_query_packed(1, 1, 128, 8, 64, fake, 0, None, fake, fake, None) == _abi.LSA_E_ARG
    arr_bad, _keep2 = _abi.ptr_array([20])
    assert lib.lsa_project_query_packed(1, 1, 128, 8, 64, fake, 0, arr_bad, fake, fake, None) == _abi.LSA_E_ARG
    assert lib.lsa_pack_query_weights(8, 64, 100, fake, fake, fake, None) == _abi.LSA_E_SHAPE
    assert lib.lsa_pack_query_weights(8, 96, 128, fake, fake, fake, None) == _abi.LSA_E_SHAPE
    assert lib.lsa_pack_query_weights(8, 64, 128, fake, fake, None, None) == _abi.LSA_E_ARG
    assert lib.lsa_pack_query_weights(8, 64, 128, fake, fake, C.c_void_p(20), None) == _abi.LSA_E_ARG
    # label vote: too many layers, top_p out of range, no mask and no workspace
    assert lib.lsa_label_vote(1, 33, 100, 0.6, 3, fake, fake, fake, fake, None, 0, None) == _abi.LSA_E_SHAPE
    assert lib.lsa_label_vote(1, 3, 65537, 0.6, 3, fake, fake, fake, fake, None, 0, None) == _abi.LSA_E_SHAPE
    assert lib.lsa_label_vote(1 << 28, 8, 100, 0.6, 3, fake, fake, fake, fake, None, 0, None) == _abi.LSA_E_SHAPE
    assert lib.lsa_label_vote(1, 3, 100, 0.0, 3, fake, fake, fake, fake, None, 0, None) == _abi.LSA_E_ARG
    assert lib.lsa_label_vote(1, 3, 100, 1.5, 3, fake, fake, fake, fake, None, 0, None) == _abi.LSA_E_ARG
    assert lib.lsa_label_vote(1, 3, 100, 0.6, 3, fake, None, fake, fake, None, 0, None) == _abi.LSA_E_WORKSPACE
    assert lib.lsa_label_vote(1, 3, 100, 0.6, 3, C.c_void_p(20), fake, fake, fake, None, 0, None) == _abi.LSA_E_ARG
    # focal: Q above 64, D not a multiple of 64, unsupported dI, short workspace
    F = lambda Q, N, D, H, dI, g=2.0, ws=fake, nws=1 << 30: lib.lsa_focal_bce_grad(
        Q, N, D, H, dI, g, fake, fake, fake, 0.0, fake, fake, fake, fake, ws, nws, None)
    assert F(65, 10, 128, 1, 64) == _abi.LSA_E_SHAPE
    assert F(4, 10, 192, 1, 64) == _abi.LSA_E_SHAPE
    assert F(4, 10, 128, 1, 96) == _abi.LSA_E_SHAPE
    assert F(4, 10, 128, 1, 64, g=-1.0) == _abi.LSA_E_ARG
    assert F(4, 10, 128, 1, 64, ws=C.c_void_p(256), nws=16) == _abi.LSA_E_WORKSPACE
    assert F(4, 10, 128, 1, 64, ws=C.c_void_p(16 + 256)) == _abi.LSA_E_WORKSPACE   # misaligned


def test_packed_weight_sizes(lib):
    # T = ceil((H*dI + H) / 16) tiles x D/64 units x 2 KiB
    assert lib.lsa_query_weights_packed_bytes(64, 128, 4096) == 516 * 64 * 2048
    assert lib.lsa_query_weights_packed_bytes(5, 64, 320) == 21 * 5 * 2048
    assert lib.lsa_query_weights_packed_bytes(65, 64, 320) == 0
    assert lib.lsa_query_weights_packed_bytes(8, 64, 100) == 0


def test_workspace_sizes(lib):
    # fetch: survivor bitmap [B][ceil(N/32)] u32 plus two [B][cap] i32 lists
    assert lib.lsa_fetch_workspace_bytes(32, 262144, 262144) >= 32 * 8192 * 4 + 2 * 32 * 262144 * 4
    assert lib.lsa_fetch_workspace_bytes(0, 10, 10) == 0
    W = (32768 + 31) // 32
    assert lib.lsa_label_vote_workspace_bytes(64, 20, 32768) == 64 * 20 * W * 4
    big = lib.lsa_focal_bce_grad_workspace_bytes(64, 32768, 4096, 64, 128)
    # at least the partial key gradients [N/128][64][dI] fp32 and the
    # transposed hidden states [D][64] bf16
    assert big >= 256 * 64 * 128 * 4 + 4096 * 64 * 2
    assert lib.lsa_focal_bce_grad_workspace_bytes(65, 10, 128, 1, 64) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from sparse_kv_cache_lsa_amd import _abi
    monkeypatch.setattr(_abi, "_lib", None)
    monkeypatch.setattr(_abi, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _abi.load()


def test_binding_checks_row_and_batch_sizes():
    """The binding refuses tensors whose rows or batch differ from the sizes
    it passes to the library (a kernel would otherwise run past one of them)."""
    import torch
    import sparse_kv_cache_lsa_amd as lsa
    pool = torch.zeros((2, 5, 512), dtype=torch.int16)
    ok = torch.zeros((2, 7, 1024), dtype=torch.uint8)
    lsa._same_rows("f", (pool, ok), 1024, 2, (torch.zeros(2, 3),))
    with pytest.raises(ValueError):
        lsa._same_rows("f", (pool, torch.zeros((2, 7, 512), dtype=torch.uint8)), 1024, 2, ())
    with pytest.raises(ValueError):
        lsa._same_rows("f", (pool, ok), 1024, 2, (torch.zeros(3, 3),))
    with pytest.raises(ValueError):
        lsa._same_rows("f", (pool, torch.zeros((3, 7, 1024), dtype=torch.uint8)), 1024, 2, ())


def test_binding_checks_sizes_and_dtypes_before_any_launch():
    """Every size and dtype that a kernel relies on is checked by the binding
    before the device check (so these CPU tensors are refused for their
    shape or dtype, not for living on the host)."""
    import torch
    import sparse_kv_cache_lsa_amd as lsa
    i32, f32, u8, bf = torch.int32, torch.float32, torch.uint8, torch.bfloat16
    z = lambda *sh, dt=f32: torch.zeros(sh, dtype=dt)

    def refused(call, what):
        with pytest.raises(ValueError, match=what):
            call()

    # gathers: hot must hold k rows per request
    refused(lambda: lsa.lsa_gather_hot(z(2, 10, 512, dt=torch.int16), z(2, 4, dt=i32),
                                       z(2, 3, 512, dt=torch.int16)), "hot holds 3 rows")
    refused(lambda: lsa.lsa_gather_resident(z(2, 6, 512, dt=torch.int16), z(2, 10, dt=i32),
                                            z(2, 4, dt=i32), z(2, 2, 512, dt=torch.int16)),
            "hot holds 2 rows")
    refused(lambda: lsa.lsa_gather_hot(z(2, 10, 512, dt=torch.int16), z(2, 4, dt=torch.int64),
                                       z(2, 4, 512, dt=torch.int16)), "idx has dtype")
    # packed weights: the buffer must hold the whole packed layout
    need = lsa.lsa_query_weights_packed_bytes(4, 64, 256)
    refused(lambda: lsa.lsa_pack_query_weights(z(256, 256, dt=bf), z(4, 256, dt=bf),
                                               z(need - 16, dt=u8)), f"hold {need} bytes")
    # resident reset: both tables of the same batch
    refused(lambda: lsa.lsa_resident_reset(z(3, 100, dt=i32), z(2, 50, dt=i32)), "entry_of")
    # score: dtypes of the query, gates, outputs and scales
    L, B, N, H, dI = 1, 2, 100, 4, 64
    nch = 1
    args = lambda q=z(L, B, H, dI, dt=bf), g=z(L, B, H), m=z(L, B, 4, dt=i32), ci=z(B, nch, 4096, dt=i32), cz=z(B, nch, 4096), cc=z(B, nch, dt=i32): (
        [z(B, N, dI, dt=bf)], None, q, g, [0.0], m, ci, cz, cc)
    refused(lambda: lsa.lsa_score(*args(g=z(L, B, H, dt=bf))), "g has dtype")
    refused(lambda: lsa.lsa_score(*args(q=z(L, B, H, dI))), "q has dtype")
    refused(lambda: lsa.lsa_score(*args(cz=z(B, nch, 4096, dt=torch.float64))), "cand_z has dtype")
    refused(lambda: lsa.lsa_score(*args(ci=z(B, nch, 4096, dt=torch.int64))), "cand_idx has dtype")
    refused(lambda: lsa.lsa_score([z(B, N, dI, dt=u8)], [z(B, N, dt=bf)], z(L, B, H, dI, dt=bf),
                                  z(L, B, H), [0.0], z(L, B, 4, dt=i32), z(B, nch, 4096, dt=i32),
                                  z(B, nch, 4096), z(B, nch, dt=i32)), "key_scale")
    # select, top-k: index and logit dtypes
    refused(lambda: lsa.lsa_select_or_compact(z(B, nch, 4096, dt=i32), z(B, nch, 4096),
                                              z(B, nch, dt=i32), N, z(B, N, dt=torch.int64),
                                              z(B, N), z(B, dt=i32)), "surv_idx has dtype")
    refused(lambda: lsa.lsa_select_or_compact_masks(z(L, B, 4, dt=i32), z(L, B, N, dt=torch.float16),
                                                    z(B, N, dt=i32), z(B, N), z(B, dt=i32)),
            "z has dtype")
    refused(lambda: lsa.lsa_select_or_compact_masks(z(L, B, 3, dt=i32), z(L, B, N),
                                                    z(B, N, dt=i32), z(B, N), z(B, dt=i32)),
            "sel_mask has shape")
    refused(lambda: lsa.lsa_topk(z(B, N, dt=i32), z(B, N, dt=torch.float64), z(B, dt=i32),
                                 z(B, 8, dt=i32), z(B, dt=i32)), "surv_z has dtype")
    # projection: fp32 query output refused
    refused(lambda: lsa.lsa_project_query(z(B, 256, dt=bf), [z(H * dI, 256, dt=bf)],
                                          [z(H, 256, dt=bf)], z(L, B, H, dI), z(L, B, H)),
            "q has dtype")
    # labels: count/label are bytes
    refused(lambda: lsa.lsa_label_vote(z(2, 3, 64), 0.6, 3, z(2, 64, dt=i32), z(2, 64, dt=u8)),
            "count has dtype")
    # a well-formed call on host tensors is refused for living on the host
    refused(lambda: lsa.lsa_topk(z(B, N, dt=i32), z(B, N), z(B, dt=i32), z(B, 8, dt=i32),
                                 z(B, dt=i32)), "on the GPU")
