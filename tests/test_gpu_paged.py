"""Paged caches (DeepSeek-V4 essay §7.1: compressed KV and indexer K live in a
paged cache addressed through a per-request block table).

Every paged call is compared with the same call on the contiguous cache that
holds the same logical entries: the results must be bit-identical (the
kernels do the same arithmetic, only the addresses differ).  The contiguous
calls are checked against the oracle elsewhere; here the oracle's logical
view of the page pool (`pipeline.unpage`) is also compared with the
contiguous cache the pool was built from, and one scan row is checked
against the oracle directly on that view.
"""
import numpy as np
import pytest
import torch

from _helpers import check_attention, u16
from oracle import pipeline
import synth

pytestmark = pytest.mark.gpu

csa = None


@pytest.fixture(scope="module", autouse=True)
def _gpu_lib():
    global csa
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import compressed_sparse_attention_index_amd as m
    m.lib()
    csa = m


def _np(t):
    return t.detach().cpu().numpy()


def _table(B, max_pages, spare, seed):
    """Distinct pool pages for every (sequence, logical page), shuffled, with
    `spare` pages that no sequence uses."""
    rng = np.random.default_rng(seed)
    num_pages = B * max_pages + spare
    bt = rng.permutation(num_pages)[:B * max_pages].reshape(B, max_pages).astype(np.int32)
    return bt, num_pages


def _scatter(x, bt, P, num_pages, fill=0):
    """Contiguous [B, max_pages * P, ...] -> pool [num_pages * P, ...]."""
    B, max_pages = bt.shape
    pool = torch.full((num_pages * P,) + tuple(x.shape[2:]), fill, dtype=x.dtype)
    for b in range(B):
        for j in range(max_pages):
            pool[bt[b, j] * P:(bt[b, j] + 1) * P] = x[b, j * P:(j + 1) * P]
    return pool


def _paging(bt, P, num_pages):
    return csa.Paging(torch.from_numpy(bt).cuda(), P, num_pages)


@pytest.mark.parametrize("kdtype,P", [("fp8", 64), ("bf16", 256)])
def test_scan_paged(kdtype, P):
    B, T = 3, 2048
    d = synth.decode_workload(B=B, T=T, kdtype=kdtype, seed=201)
    vis = torch.tensor([[T], [1500], [77]], dtype=torch.int32).cuda()
    bt, num_pages = _table(B, T // P, 3, 201)
    pool = _scatter(d["k_idx"], bt, P, num_pages)
    view, mapped = pipeline.unpage(_np(pool), bt, P)
    assert mapped.all() and np.array_equal(view, _np(d["k_idx"]))
    out = {}
    for name, k, pg in (("contiguous", d["k_idx"].cuda(), None),
                        ("paged", pool.cuda(), _paging(bt, P, num_pages))):
        sc = torch.full((B, 1, T), float("nan"), device="cuda")
        bm = torch.full((B, 1, T // 8), float("nan"), device="cuda")
        print(f"scan {kdtype} P={P} {name}", flush=True)
        csa.index_score(d["q_idx"].cuda(), d["w_idx"].cuda(), k, vis, scores=sc, block_max=bm,
                        paging=pg)
        torch.cuda.synchronize()
        out[name] = (_np(sc), _np(bm))
    for a, b in zip(out["contiguous"], out["paged"]):
        assert np.array_equal(a, b, equal_nan=True)
    # One row straight against the oracle on the pool's logical view.
    raw = view[1].view(np.uint16) if kdtype == "bf16" else view[1]
    ref = pipeline.scores_prefix(u16(d["q_idx"][1, 0]), _np(d["w_idx"][1, 0]), raw, kdtype, 1500)
    got = out["paged"][0][1, 0, :1500].astype(np.float64)
    tol = 1e-5 * np.abs(ref) + 1e-6 * np.abs(ref).max()
    assert np.all(np.abs(got - ref) <= tol)


def test_prefill_gemm_paged():
    # Prefill-shaped rows (n_q >= 16) take the matrix-core kernel.
    d = synth.prefill_workload(n_q=32, prefix_tokens=4096, seed=202)
    N, P = d["k_idx"].shape[1], 64
    N_pad = (N + P - 1) // P * P
    k = torch.zeros(1, N_pad, 128, dtype=d["k_idx"].dtype)
    k[:, :N] = d["k_idx"]
    bt, num_pages = _table(1, N_pad // P, 2, 202)
    pool = _scatter(k, bt, P, num_pages)
    out = []
    for kk, pg in ((k.cuda(), None), (pool.cuda(), _paging(bt, P, num_pages))):
        sc = torch.full((1, 32, N_pad), float("nan"), device="cuda")
        print(f"prefill scan paged={pg is not None}", flush=True)
        csa.index_score(d["q_idx"].cuda(), d["w_idx"].cuda(), kk, d["vis_len"].cuda(), scores=sc,
                        paging=pg)
        torch.cuda.synchronize()
        out.append(_np(sc))
    assert np.array_equal(out[0], out[1], equal_nan=True)


@pytest.mark.parametrize("mode", ["full", "reindex"])
def test_pool_topk_paged(mode):
    B, T, P = 2, 4096, 128
    d = synth.decode_workload(B=B, T=T, kdtype="fp8", seed=203, reindex=True)
    vis = d["vis_len"].cuda()
    bm = torch.empty(B, 1, T // 8, device="cuda")
    csa.index_score(d["q_idx"].cuda(), d["w_idx"].cuda(), d["k_idx"].cuda(), vis, block_max=bm)
    pool_blocks = torch.empty(B, 1, 256, dtype=torch.int32, device="cuda")
    csa.block_topk(bm, vis, T, 256, pool_blocks)
    bt, num_pages = _table(B, T // P, 4, 203)
    kpool = _scatter(d["k_idx"], bt, P, num_pages)
    m = csa.MODE_FULL if mode == "full" else csa.MODE_REINDEX
    q, w = (d["q_idx"], d["w_idx"]) if mode == "full" else (d["q_idx2"], d["w_idx2"])
    res = []
    for k, pg in ((d["k_idx"].cuda(), None), (kpool.cuda(), _paging(bt, P, num_pages))):
        idx = torch.empty(B, 1, 512, dtype=torch.int32, device="cuda")
        key = torch.empty(B, 1, 512, device="cuda")
        print(f"pool top-k {mode} paged={pg is not None}", flush=True)
        csa.reindex_topk(m, vis, T, 512, idx, q_idx=q.cuda(), w_idx=w.cuda(), k_idx=k,
                         pool_blocks=pool_blocks, idx_score=key, paging=pg)
        torch.cuda.synchronize()
        res.append((_np(idx), _np(key)))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])


@pytest.mark.parametrize("n_q", [1, 16])
@pytest.mark.parametrize("kv_fmt", ["e8m0_32", "e4m3_16"])
def test_attention_paged(n_q, kv_fmt):
    B, T, P = 2, 2048, 64
    d = synth.decode_workload(B=B, T=T, kdtype="bf16", seed=204, kv_fmt=kv_fmt)
    g = torch.Generator().manual_seed(204)
    d["q"] = synth.to_bf16_bits(torch.randn(B, n_q, 64, 512, generator=g))
    d["q_pos"] = torch.full((B, n_q), T - 1, dtype=torch.int32)
    rng = np.random.default_rng(204)
    idx = np.stack([np.stack([np.sort(rng.choice(T, size=400, replace=False))
                              for _ in range(n_q)]) for _ in range(B)]).astype(np.int32)
    bt, num_pages = _table(B, T // P, 5, 204)
    # Logical page 3 of sequence 1 is unmapped: its selected ids are empty slots.
    bt_holes = bt.copy()
    bt_holes[1, 3] = -1
    fmt = csa.KV_FP4_E4M3_16 if kv_fmt == "e4m3_16" else csa.KV_MXFP4_E8M0_32
    fp4_pool = _scatter(d["kv_fp4"], bt, P, num_pages)
    sc_pool = _scatter(d["kv_scale"], bt, P, num_pages)
    idx_holes = idx.copy()
    idx_holes[1][(idx[1] >= 3 * P) & (idx[1] < 4 * P)] = -1

    def run(fp4, sc, ids, pg):
        out = torch.zeros(B, n_q, 64, 512, dtype=torch.int16, device="cuda")
        lse = torch.zeros(B, n_q, 64, device="cuda")
        csa.sparse_attn_decode(d["q"].cuda(), fp4.cuda(), sc.cuda(), torch.from_numpy(ids).cuda(),
                               d["swa"].cuda(), d["swa_pos0"].cuda(), d["q_pos"].cuda(),
                               d["sm_scale"], out, lse=lse, kv_fmt=fmt, paging=pg)
        torch.cuda.synchronize()
        return u16(out), _np(lse)

    print(f"attention paged n_q={n_q} {kv_fmt}", flush=True)
    flat = run(d["kv_fp4"], d["kv_scale"], idx, None)
    paged = run(fp4_pool, sc_pool, idx, _paging(bt, P, num_pages))
    assert np.array_equal(flat[0], paged[0]) and np.array_equal(flat[1], paged[1])
    flat_h = run(d["kv_fp4"], d["kv_scale"], idx_holes, None)
    paged_h = run(fp4_pool, sc_pool, idx, _paging(bt_holes, P, num_pages))
    assert np.array_equal(flat_h[0], paged_h[0]) and np.array_equal(flat_h[1], paged_h[1])
    # And the oracle on the logical view of the pool, one row.
    view_fp4, _ = pipeline.unpage(_np(fp4_pool), bt, P)
    view_sc, _ = pipeline.unpage(_np(sc_pool), bt, P)
    sel = idx[0, n_q - 1]
    o, l = pipeline.attention(u16(d["q"][0, n_q - 1]), view_fp4[0][sel], view_sc[0][sel],
                              np.arange(len(sel)), _np(d["swa"][0]), int(d["swa_pos0"][0]),
                              int(d["q_pos"][0, n_q - 1]), d["sm_scale"], kv_fmt=kv_fmt)
    check_attention(paged[0][0, n_q - 1], paged[1][0, n_q - 1], o, l, what="paged row")


@pytest.mark.parametrize("kv_fmt", ["e8m0_32", "e4m3_16"])
def test_kv_append_paged(kv_fmt):
    B, n_new, P = 2, 300, 64
    max_pages = 8
    N_cap = max_pages * P
    g = torch.Generator().manual_seed(205)
    kv_new = synth.to_bf16_bits(torch.randn(B, n_new, 512, generator=g))
    pos = torch.tensor([10, 200], dtype=torch.int32)
    bt, num_pages = _table(B, max_pages, 3, 205)
    bt[1, 5] = -1                 # positions 320..383 of sequence 1: skipped
    per = 16 if kv_fmt == "e4m3_16" else 32
    fmt = csa.KV_FP4_E4M3_16 if kv_fmt == "e4m3_16" else csa.KV_MXFP4_E8M0_32
    fp4 = torch.full((B, N_cap, 256), 0xA5, dtype=torch.uint8).cuda()
    sc = torch.full((B, N_cap, 512 // per), 0xA5, dtype=torch.uint8).cuda()
    fp4_pool = torch.full((num_pages * P, 256), 0x5A, dtype=torch.uint8).cuda()
    sc_pool = torch.full((num_pages * P, 512 // per), 0x5A, dtype=torch.uint8).cuda()
    print(f"kv_append paged {kv_fmt}", flush=True)
    csa.kv_append(kv_new.cuda(), pos.cuda(), fp4, sc, kv_fmt=fmt)
    csa.kv_append(kv_new.cuda(), pos.cuda(), fp4_pool, sc_pool, kv_fmt=fmt,
                  paging=_paging(bt, P, num_pages))
    torch.cuda.synchronize()
    for flat, pool in ((_np(fp4), _np(fp4_pool)), (_np(sc), _np(sc_pool))):
        used = np.zeros(num_pages, bool)
        for b in range(B):
            for j in range(max_pages):
                page = bt[b, j]
                if page < 0:
                    continue
                used[page] = True
                got = pool[page * P:(page + 1) * P]
                want = flat[b, j * P:(j + 1) * P].copy()
                # Rows the append did not write keep each cache's own fill.
                lo, hi = int(pos[b]), int(pos[b]) + n_new
                rows = np.arange(j * P, (j + 1) * P)
                untouched = (rows < lo) | (rows >= hi)
                want[untouched] = 0x5A
                assert np.array_equal(got, want), (b, j)
        # Pages no sequence maps (the spare ones and the unmapped hole) are
        # never written.
        for page in np.nonzero(~used)[0]:
            assert np.all(pool[page * P:(page + 1) * P] == 0x5A), page


def test_paged_full_layer_past_2g():
    # Two sequences of 2^22 entries (the largest accepted context) in
    # 4,096-entry pages of one pool: the main-KV pool is 2.2 GB and sequence
    # 1's last page is the pool's last, past 2^31 bytes.  The paged Full layer
    # (scan, block Top-K, pool Top-512, attention) gives the bits of the
    # contiguous one, which the workload tests check against the oracle.
    B, T, P = 2, 1 << 22, 4096
    d = synth.decode_workload(B=B, T=T, kdtype="fp8", seed=205, device="cuda")
    bt, num_pages = _table(B, T // P, 5, 205)
    hit = np.argwhere(bt == num_pages - 1)
    if len(hit):
        i, j = hit[0]
        bt[i, j], bt[1, -1] = bt[1, -1], bt[i, j]
    else:
        bt[1, -1] = num_pages - 1
    assert num_pages * P * 256 > 2 ** 31 and len(np.unique(bt)) == bt.size

    def scatter(x):
        pool = torch.zeros((num_pages * P,) + tuple(x.shape[2:]), dtype=x.dtype, device="cuda")
        for b in range(B):
            for j in range(T // P):
                pool[int(bt[b, j]) * P:(int(bt[b, j]) + 1) * P] = x[b, j * P:(j + 1) * P]
        return pool

    def layer(k, fp4, sc, pg):
        vis = d["vis_len"]
        bm = torch.empty(B, 1, T // 8, device="cuda")
        csa.index_score(d["q_idx"], d["w_idx"], k, vis, block_max=bm, paging=pg)
        pool = torch.empty(B, 1, 2048, dtype=torch.int32, device="cuda")
        csa.block_topk(bm, vis, T, 2048, pool)
        idx = torch.empty(B, 1, 512, dtype=torch.int32, device="cuda")
        csa.reindex_topk(csa.MODE_FULL, vis, T, 512, idx, q_idx=d["q_idx"], w_idx=d["w_idx"],
                         k_idx=k, pool_blocks=pool, paging=pg)
        out = torch.zeros(B, 1, 64, 512, dtype=torch.int16, device="cuda")
        lse = torch.zeros(B, 1, 64, device="cuda")
        csa.sparse_attn_decode(d["q"], fp4, sc, idx, d["swa"], d["swa_pos0"], d["q_pos"],
                               d["sm_scale"], out, lse=lse, paging=pg)
        torch.cuda.synchronize()
        return [_np(t) for t in (bm, pool, idx, out, lse)]

    print("paged full layer at 2^22 entries, pool past 2 GiB", flush=True)
    flat = layer(d["k_idx"], d["kv_fp4"], d["kv_scale"], None)
    paged = layer(scatter(d["k_idx"]), scatter(d["kv_fp4"]), scatter(d["kv_scale"]),
                  _paging(bt, P, num_pages))
    for a, b, name in zip(flat, paged, ("block max", "pool", "idx", "out", "lse")):
        assert np.array_equal(a, b), name
