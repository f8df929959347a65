"""The C-ABI library loads, exports what include/csa2.h declares, and rejects
bad arguments on the host before touching a GPU (CPU only: no compute call
here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

from _helpers import ROOT, ensure_built

HEADER = os.path.join(ROOT, "include", "csa2.h")


@pytest.fixture(scope="module")
def L():
    ensure_built()
    import compressed_sparse_attention_index_amd as csa
    return csa.lib()


def test_exports_every_declared_symbol(L):
    decls = re.findall(r"CSA2_API\s+[\w\s\*]+?\b(csa2_\w+)\s*\(", open(HEADER).read())
    assert len(decls) == 15
    for name in decls:
        assert hasattr(L, name), name


def test_version_and_status_strings(L):
    assert L.csa2_abi_version() == 7
    for st in range(7):
        assert len(L.csa2_status_string(st)) > 0
    assert L.csa2_status_string(0) == b"ok"


def test_workspace_sizes(L):
    import compressed_sparse_attention_index_amd as csa
    assert csa.workspace_size(csa.OP_INDEX_SCORE, 8, 1, 1 << 20) == 0
    assert csa.workspace_size(csa.OP_BLOCK_TOPK, 8, 1, 1 << 20) == 8 * (2 * 4096 + 2 * 128 + 3 * 131072) * 4
    assert csa.workspace_size(csa.OP_REINDEX_TOPK, 8, 1, 1 << 20, 512, 2048) == 8 * 2048 * 8 * 4
    assert csa.workspace_size(csa.OP_SPARSE_ATTN, 4096, 1, 1 << 16, 512, 0) == 0
    # Attention never splits a row over workgroups: no workspace at any size.
    assert csa.workspace_size(csa.OP_SPARSE_ATTN, 8, 1, 1 << 20, 512, 0) == 0
    assert csa.workspace_size(csa.OP_SPARSE_ATTN, 1, 1, 1 << 20, 512, 0) == 0
    assert csa.workspace_size(7, 1, 1, 1) == ctypes.c_size_t(-1).value
    assert csa.workspace_size(csa.OP_INDEX_SCORE, 0, 1, 1) == ctypes.c_size_t(-1).value


A = 1 << 20      # a fake, 16-byte aligned "device" address: never dereferenced
MIS = A + 4      # misaligned


def _score(L, q=A, w=A, k=A, kd=1, vis=A, B=1, n_q=1, N=64, sc=A, bm=A, pg=None):
    return L.csa2_index_score(q, w, k, kd, pg, vis, B, n_q, N, sc, bm, None, 0, None)


def test_bf16_score_entry_points_validation(L):
    f = L.csa2_index_score_bf16
    ok = (A, A, A, 1, None, A, 1, 1, 64, A, None)
    def call(**kw):
        args = list(ok)
        for i, v in kw.items():
            args[int(i[1:])] = v
        return f(*args)
    assert call(a9=None) == 1                 # scores required
    assert call(a0=None) == 1
    assert call(a3=5) == 3                    # key dtype
    assert call(a6=0) == 2
    assert call(a9=MIS) == 5
    assert f(A, A, A, 2, None, A, 1, 16, 64, A, None) == 3   # MXFP4 keys: decode rows only
    assert f(A, A, A, 3, None, A, 1, 16, 64, A, None) == 3   # MXFP4 keys and query: likewise
    g = L.csa2_flat_topk_bf16
    assert g(None, A, 1, 1, 64, 16, A, None, None) == 1
    assert g(A, A, 1, 1, 64, 16, None, None, None) == 1
    assert g(A, A, 1, 1, 64, 0, A, None, None) == 2
    assert g(A, A, 1, 1, 64, 513, A, None, None) == 2
    assert g(A, A, 0, 1, 64, 16, A, None, None) == 2
    assert g(A, A, 1, 1, 0, 16, A, None, None) == 2
    assert g(A, A, 1, 1, 64, 16, A, MIS, None) == 5


def _pg(bt=A, P=64, max_pages=1, num_pages=1):
    import compressed_sparse_attention_index_amd as csa
    return ctypes.byref(csa.PagingStruct(bt, P, max_pages, num_pages))


def test_index_score_validation(L):
    assert _score(L, q=None) == 1
    assert _score(L, sc=None, bm=None) == 1
    assert _score(L, kd=5) == 3
    assert _score(L, kd=4) == 3
    assert _score(L, kd=3, n_q=16) == 3    # MXFP4 keys and query: decode rows only
    assert _score(L, B=0) == 2
    assert _score(L, N=0) == 2
    assert _score(L, N=(1 << 22) + 1) == 2
    assert _score(L, B=70000) == 2
    assert _score(L, k=MIS) == 5


def test_paging_validation(L):
    # The page table is checked on the host before anything is enqueued:
    # N_cap must be max_pages * page_entries, page_entries a power of two in
    # [64, 65536], the pool addressable with 31-bit rows.
    assert _score(L, N=128, pg=_pg(max_pages=2, num_pages=4)) != 2   # valid: fails later (no GPU)
    assert _score(L, N=128, pg=_pg(bt=None, max_pages=2)) == 1
    assert _score(L, N=128, pg=_pg(bt=MIS, max_pages=2)) == 5
    assert _score(L, N=128, pg=_pg(max_pages=1)) == 2                # 64 != 128
    assert _score(L, N=96, pg=_pg(P=48, max_pages=2)) == 2           # not a power of two
    assert _score(L, N=64, pg=_pg(P=32, max_pages=2)) == 2           # below 64 entries
    assert _score(L, N=128, pg=_pg(max_pages=2, num_pages=0)) == 2
    assert _score(L, N=1 << 16, pg=_pg(P=1 << 16, num_pages=1 << 15)) == 2   # 2^31 rows
    assert _reindex(L, N=128, kb=16, pg=_pg(max_pages=1)) == 2
    f = L.csa2_kv_append
    assert f(A, None, A, 1, 1, 128, 0, _pg(max_pages=1), A, A, None, 0, None, None) == 2
    import compressed_sparse_attention_index_amd as csa
    for fn in ("csa2_sparse_attn_decode", "csa2_reuse_attn"):
        paged = csa.AttnOpts(128, -1, 0, csa.ATTN_PAGED, None, None)
        assert _attn(L, fn, opts=ctypes.byref(paged)) == 1          # flag without a table
        bad = csa.PagingStruct(A, 64, 1, 1)
        paged = csa.AttnOpts(128, -1, 0, csa.ATTN_PAGED, None, ctypes.pointer(bad))
        assert _attn(L, fn, opts=ctypes.byref(paged)) == 2          # 64 != N_cap
        ok = csa.PagingStruct(A, 1024, 128, 4096)
        paged = csa.AttnOpts(128, -1, 0, csa.ATTN_PAGED, None, ctypes.pointer(ok))
        assert _attn(L, fn, opts=ctypes.byref(paged), out=MIS) == 5   # accepted up to alignment


def test_block_topk_validation(L):
    f = L.csa2_block_topk
    assert f(None, A, 1, 1, 64, 16, A, None, 0, None) == 1
    assert f(A, A, 1, 1, 64, 0, A, None, 0, None) == 2
    assert f(A, A, 1, 1, 64, 2049, A, None, 0, None) == 2
    assert f(A, A, 1, 1, 0, 16, A, None, 0, None) == 2
    assert f(A, A, 1, 1, 64, 16, MIS, None, 0, None) == 5
    assert f(A, A, 1, 1, 64, 16, A, None, 0, None) == 4          # workspace required
    assert f(A, A, 1, 1, 64, 16, A, A, 4 * (2 * 4096 + 2 * 128 + 3 * 8) - 1, None) == 4
    assert f(A, A, 1, 1, (1 << 22) + 1, 16, A, A, 1 << 30, None) == 2


def test_block_topk_noalloc_validation(L):
    f = L.csa2_block_topk_noalloc
    assert f(None, A, 1, 1, 64, 16, A, None) == 1
    assert f(A, A, 1, 1, 64, 0, A, None) == 2
    assert f(A, A, 1, 1, 0, 16, A, None) == 2
    assert f(A, A, 1, 1, 64, 16, MIS, None) == 5
    # Beyond the fixed scratch array: more than 64 rows, or too many blocks.
    assert f(A, A, 65, 1, 64, 16, A, None) == 4
    assert f(A, A, 8, 2, 1 << 20, 16, A, None) == 4
    assert f(A, A, 10, 1, 1 << 20, 16, A, None) == 4


def _reindex(L, mode=1, sc=None, q=A, w=A, k=A, kd=1, pool=A, kb=2048, vis=A, B=1, n_q=1, N=1 << 20,
             top_k=512, out=A, ws=None, ws_bytes=0, pg=None):
    return L.csa2_reindex_topk(mode, sc, q, w, k, kd, pg, pool, kb, vis, B, n_q, N, top_k, out,
                               None, ws, ws_bytes, None)


def test_reindex_topk_validation(L):
    assert _reindex(L, mode=2) == 3                 # Reuse runs no indexer
    assert _reindex(L, mode=9) == 3
    assert _reindex(L, out=None) == 1
    assert _reindex(L, top_k=0) == 2
    assert _reindex(L, top_k=513) == 2
    assert _reindex(L, kb=0) == 2
    assert _reindex(L, pool=None) == 1              # flat selection needs scores
    assert _reindex(L, q=None) == 1                 # re-scoring needs the query
    assert _reindex(L, kd=4) == 3
    assert _reindex(L) == 4                         # no workspace for the re-scored pool
    assert _reindex(L, ws=A, ws_bytes=2048 * 8 * 4 - 1) == 4
    assert _reindex(L, mode=0, sc=A, q=None) == 4    # stored scores: no query needed, workspace is
    assert _reindex(L, vis=MIS) == 5


def _attn(L, fn="csa2_sparse_attn_decode", q=A, fp4=A, sc=A, N=1 << 17, idx=A, top_k=512, swa=A,
          S=128, p0=A, qp=A, scale=0.044, opts=None, B=64, n_q=1, out=A, lse=A, ws=None, wsb=0):
    return getattr(L, fn)(q, fp4, sc, N, idx, top_k, swa, S, p0, qp, scale, opts, B, n_q, out, lse,
                          ws, wsb, None)


def test_attention_validation(L):
    import compressed_sparse_attention_index_amd as csa
    for fn in ("csa2_sparse_attn_decode", "csa2_reuse_attn"):
        assert _attn(L, fn, q=None) == 1
        assert _attn(L, fn, idx=None) == 1
        assert _attn(L, fn, swa=None) == 1
        assert _attn(L, fn, top_k=513) == 2
        assert _attn(L, fn, top_k=-1) == 2
        assert _attn(L, fn, S=-1) == 2
        assert _attn(L, fn, N=0) == 2
        assert _attn(L, fn, B=70000) == 2
        assert _attn(L, fn, scale=float("nan")) == 2
        assert _attn(L, fn, scale=0.0) == 2
        assert _attn(L, fn, scale=-0.04) == 2
        assert _attn(L, fn, scale=float("inf")) == 2
        bad_fmt = csa.AttnOpts(128, -1, 2, 0)
        assert _attn(L, fn, opts=ctypes.byref(bad_fmt)) == 3
        e4m3 = csa.AttnOpts(128, -1, csa.KV_FP4_E4M3_16, 0)   # accepted up to the alignment check
        assert _attn(L, fn, opts=ctypes.byref(e4m3), out=MIS) == 5
        bad_win = csa.AttnOpts(129, -1, 0, 0)
        assert _attn(L, fn, opts=ctypes.byref(bad_win)) == 2
        bad_sink = csa.AttnOpts(128, -1, 0, csa.ATTN_SINK, MIS)
        assert _attn(L, fn, opts=ctypes.byref(bad_sink)) == 5
        null_sink = csa.AttnOpts(128, -1, 0, csa.ATTN_SINK, None)
        assert _attn(L, fn, opts=ctypes.byref(null_sink)) == 1
        bad_flag = csa.AttnOpts(128, -1, 0, 4, None)
        assert _attn(L, fn, opts=ctypes.byref(bad_flag)) == 3
        # Without the sink flag the pointer is not read: an ABI-1 caller's
        # 16-byte struct (no pointer field) passes validation up to the
        # workspace check, like NULL options.
        v1 = csa.AttnOptsV1(128, -1, 0, 0)
        assert _attn(L, fn, opts=ctypes.byref(v1), out=MIS) == 5
        unread = csa.AttnOpts(128, -1, 0, 0, MIS)
        assert _attn(L, fn, opts=ctypes.byref(unread), out=MIS) == 5
        assert _attn(L, fn, out=MIS) == 5


def test_binding_refuses_cpu_tensors(L):
    import torch
    import compressed_sparse_attention_index_amd as csa
    x = torch.zeros(1, 1, 32, 128, dtype=torch.int16)
    with pytest.raises(ValueError):
        csa.index_score(x, torch.zeros(1, 1, 32), torch.zeros(1, 64, 128, dtype=torch.uint8),
                        torch.zeros(1, 1, dtype=torch.int32), block_max=torch.zeros(1, 1, 8))


def test_kv_append_validation(L):
    f = L.csa2_kv_append
    def call(kv=A, swn=None, pos=A, B=1, n=1, N=64, fmt=0, fp4=A, sc=A, swa=None, S=0, p0=None):
        return f(kv, swn, pos, B, n, N, fmt, None, fp4, sc, swa, S, p0, None)
    assert call(kv=None) == 1
    assert call(fmt=2) == 3
    assert call(fmt=-1) == 3
    assert call(fmt=1, kv=MIS) == 5             # the E4M3 format passes up to the alignment check
    assert call(sc=None) == 1
    assert call(swn=A) == 1                     # window entries without a window cache
    assert call(swn=A, swa=A) == 1              # ... or without swa_pos0
    assert call(B=0) == 2
    assert call(n=0) == 2
    assert call(N=0) == 2
    assert call(S=-1) == 2
    assert call(kv=MIS) == 5
    assert call(swn=A, swa=MIS, S=128, p0=A) == 5


def test_layer_schedule_matches_oracle(L):
    # The library's schedule (host code) against the oracle's reading of the page.
    from oracle import pipeline
    names = {0: "full", 1: "reindex", 2: "reuse", 3: "swa", -1: None}
    for layer in range(-2, 42):
        assert names[L.csa2_layer_mode(layer)] == pipeline.layer_mode(layer), layer


def test_run_layer_state_validation(L):
    # Checked on the host before anything is enqueued.
    import compressed_sparse_attention_index_amd as csa
    args = csa.LayerArgs()
    st = csa.LayerStateStruct(A, None, A, 2048, A, 512, A, 1 << 20, 0, 0)
    run = lambda mode, a=ctypes.byref(args), s=ctypes.byref(st): L.csa2_run_layer(mode, a, s, A, A,
                                                                                  None)
    assert run(csa.MODE_REUSE) == 7           # no indices from an earlier layer
    assert run(csa.MODE_REINDEX) == 7         # no pool from an earlier Full layer
    assert run(9) == 3
    assert run(csa.MODE_REUSE, a=None) == 1
    st.top_k = 513
    assert run(csa.MODE_REUSE) == 2
    st.top_k, st.idx = 512, None
    assert run(csa.MODE_REUSE) == 1
    assert L.csa2_layer_workspace_size(8, 1, 1 << 20, 2048, 512) == (
        L.csa2_workspace_size(1, 8, 1, 1 << 20, 512, 2048) + 255) // 256 * 256 + \
        L.csa2_workspace_size(2, 8, 1, 1 << 20, 512, 2048)
