"""The FP4 indexer QK path (DeepSeek-V4 essay §10.2): indexer keys stored as
MXFP4 (CSA2_KDTYPE_MXFP4), and with the query quantised to MXFP4 as well
(CSA2_KDTYPE_MXFP4_QK, the products on the scaled FP4 matrix instructions).
The keys dequantise exactly to bf16 and every product of two dequantised
values is exact, so the scan and the pool re-scoring are compared with the
oracle on the same stored bytes (parity, not recall); the recall of the FP4
path against unquantised keys is a property of the data and is reported by
the benchmark.
"""
import numpy as np
import pytest
import torch

from _helpers import check_selection, u16
from oracle import indexer, pipeline
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


def _oracle_rows(buf, rows, first, n):
    """Rows first .. first + n of an MXFP4 key buffer in the oracle's layout
    ([n, 68]: 64 bytes of E2M1, then the 4 scales)."""
    b = _np(buf)
    e2m1 = b[:rows * 64].reshape(rows, 64)[first:first + n]
    sc = b[rows * 64:].reshape(rows, 4)[first:first + n]
    return np.concatenate([e2m1, sc], axis=1)


def _keys(d, qk=False):
    B, T = d["B"], d["T"]
    return csa.Mxfp4Keys(d["k_idx"].cuda(), B * T, T, fp4_query=qk)


@pytest.mark.parametrize("qk", [False, True], ids=["keys", "qk"])
@pytest.mark.parametrize("T", [2048, 4133])
def test_scan_mxfp4_ragged(T, qk):
    kd = "mxfp4_qk" if qk else "mxfp4"
    vis = [0, 1, 7, 9, 33, 512, 513, T - 1, T]
    B = len(vis)
    d = synth.decode_workload(B=B, T=T, kdtype="mxfp4", seed=401, lognormal_sigma=0.5)
    vis_t = torch.tensor(vis, dtype=torch.int32).reshape(B, 1).cuda()
    sc = torch.full((B, 1, T), float("nan"), device="cuda")
    bm = torch.full((B, 1, (T + 7) // 8), float("nan"), device="cuda")
    print(f"scan {kd} T={T}", flush=True)
    csa.index_score(d["q_idx"].cuda(), d["w_idx"].cuda(), _keys(d, qk), vis_t, scores=sc,
                    block_max=bm)
    torch.cuda.synchronize()
    sc, bm = _np(sc), _np(bm)
    for b, v in enumerate(vis):
        kr = _oracle_rows(d["k_idx"], B * T, b * T, T)
        ref = pipeline.scores_prefix(u16(d["q_idx"][b, 0]), _np(d["w_idx"][b, 0]), kr, kd, v)
        g = sc[b, 0, :v].astype(np.float64)
        tol = 1e-5 * np.abs(ref) + 1e-6 * (np.abs(ref).max() if v else 0)
        assert np.all(np.abs(g - ref) <= tol), f"row {b}: max err {np.abs(g - ref).max()}"
        assert np.all(np.isnan(sc[b, 0, v:]))
        nb = (v + 7) // 8
        bref = indexer.block_max(ref, v)
        assert np.all(np.abs(bm[b, 0, :nb] - bref) <= 1e-5 * np.abs(bref) +
                      1e-6 * (np.abs(ref).max() if v else 0))


@pytest.mark.parametrize("qk", [False, True], ids=["keys", "qk"])
@pytest.mark.parametrize("mode", ["full", "reindex"])
def test_pool_topk_mxfp4(mode, qk):
    kd = "mxfp4_qk" if qk else "mxfp4"
    B, T = 2, 8192
    d = synth.decode_workload(B=B, T=T, kdtype="mxfp4", seed=402, reindex=True)
    keys = _keys(d, qk)
    vis = d["vis_len"].cuda()
    bm = torch.empty(B, 1, T // 8, device="cuda")
    csa.index_score(d["q_idx"].cuda(), d["w_idx"].cuda(), keys, vis, block_max=bm)
    pool = torch.empty(B, 1, 512, dtype=torch.int32, device="cuda")
    csa.block_topk(bm, vis, T, 512, pool)
    q, w = (d["q_idx"], d["w_idx"]) if mode == "full" else (d["q_idx2"], d["w_idx2"])
    idx = torch.empty(B, 1, 512, dtype=torch.int32, device="cuda")
    print(f"pool top-k {kd} {mode}", flush=True)
    csa.reindex_topk(csa.MODE_FULL if mode == "full" else csa.MODE_REINDEX, vis, T, 512, idx,
                     q_idx=q.cuda(), w_idx=w.cuda(), k_idx=keys, pool_blocks=pool)
    torch.cuda.synchronize()
    for b in range(B):
        kr = _oracle_rows(d["k_idx"], B * T, b * T, T)
        qr, wr = u16(q[b, 0]), _np(w[b, 0])
        if mode == "full":
            ref = pipeline.full_layer(qr, wr, kr, kd, T, k_blocks=512)
            check_selection(_np(pool[b, 0]), ref["pool"], lambda j: ref["block_max"][j],
                            what=f"pool row {b}")
            check_selection(_np(idx[b, 0]), ref["idx"], lambda t: ref["scores"][t],
                            what=f"idx row {b}")
        else:
            ref = pipeline.reindex_layer(qr, wr, kr, kd, _np(pool[b, 0]), T)
            check_selection(_np(idx[b, 0]), ref["idx"],
                            lambda t: pipeline.scores_at(qr, wr, kr, kd, t),
                            what=f"reindex row {b}")


@pytest.mark.parametrize("qk", [False, True], ids=["keys", "qk"])
def test_mxfp4_full_layer_at_maximum_context(qk):
    # 8 sequences of 2^22 entries (the largest accepted context): the key
    # buffer is 2.28 GB, so the last sequence's E2M1 rows and its scales lie
    # past 2^31 bytes.  Its row is ragged (vis = T - 3).
    kd = "mxfp4_qk" if qk else "mxfp4"
    B, T = 8, 1 << 22
    d = synth.decode_workload(B=B, T=T, kdtype="mxfp4", seed=403, device="cuda")
    d["vis_len"][B - 1, 0] = T - 3
    assert B * T * 68 > 2 ** 31
    keys = _keys(d, qk)
    vis = d["vis_len"]
    bm = torch.empty(B, 1, T // 8, device="cuda")
    print(f"full layer {kd} at 2^22 entries, B={B}", flush=True)
    csa.index_score(d["q_idx"], d["w_idx"], keys, vis, block_max=bm)
    pool = torch.empty(B, 1, 2048, dtype=torch.int32, device="cuda")
    csa.block_topk(bm, vis, T, 2048, pool)
    idx = torch.empty(B, 1, 512, dtype=torch.int32, device="cuda")
    csa.reindex_topk(csa.MODE_FULL, vis, T, 512, idx, q_idx=d["q_idx"], w_idx=d["w_idx"],
                     k_idx=keys, pool_blocks=pool)
    torch.cuda.synchronize()
    buf = d["k_idx"].cpu()
    for b in (0, B - 1):
        v = int(vis[b, 0])
        kr = _oracle_rows(buf, B * T, b * T, T)
        ref = pipeline.full_layer(u16(d["q_idx"][b, 0]), _np(d["w_idx"][b, 0]), kr, kd, v)
        check_selection(_np(pool[b, 0]), ref["pool"], lambda j: ref["block_max"][j],
                        what=f"pool row {b}")
        check_selection(_np(idx[b, 0]), ref["idx"], lambda t: ref["scores"][t],
                        what=f"idx row {b}")


@pytest.mark.parametrize("qk", [False, True], ids=["keys", "qk"])
def test_scan_mxfp4_paged(qk):
    # The E2M1 rows and the scale rows of a page pool follow the same table.
    B, T, P = 2, 2048, 128
    d = synth.decode_workload(B=B, T=T, kdtype="mxfp4", seed=403)
    rows = B * T
    buf = d["k_idx"]
    e2m1 = buf[:rows * 64].view(rows, 64)
    sc = buf[rows * 64:].view(rows, 4)
    rng = np.random.default_rng(403)
    max_pages = T // P
    num_pages = B * max_pages + 3
    bt = rng.permutation(num_pages)[:B * max_pages].reshape(B, max_pages).astype(np.int32)
    pool_rows = num_pages * P
    pool = torch.zeros(pool_rows * 68, dtype=torch.uint8)
    pe, ps = pool[:pool_rows * 64].view(pool_rows, 64), pool[pool_rows * 64:].view(pool_rows, 4)
    for b in range(B):
        for j in range(max_pages):
            src = slice(b * T + j * P, b * T + (j + 1) * P)
            dst = slice(int(bt[b, j]) * P, (int(bt[b, j]) + 1) * P)
            pe[dst] = e2m1[src]
            ps[dst] = sc[src]
    paging = csa.Paging(torch.from_numpy(bt).cuda(), P, num_pages)
    out = []
    for keys, pg in ((_keys(d, qk), None),
                     (csa.Mxfp4Keys(pool.cuda(), pool_rows, T, fp4_query=qk), paging)):
        s = torch.full((B, 1, T), float("nan"), device="cuda")
        print(f"scan mxfp4 paged={pg is not None}", flush=True)
        csa.index_score(d["q_idx"].cuda(), d["w_idx"].cuda(), keys, d["vis_len"].cuda(), scores=s,
                        paging=pg)
        torch.cuda.synchronize()
        out.append(_np(s))
    assert np.array_equal(out[0], out[1], equal_nan=True)


def test_fp4_query_special_blocks():
    # The query's in-kernel MXFP4 quantisation on blocks that take every
    # branch of the encoding: all zeros, subnormal bf16 values, values at the
    # bottom of the exponent range (the clamp to -127), E2M1 ties both ways,
    # very large values, a single nonzero element, signed zeros; the other
    # heads are Gaussian.  Scores against the oracle on the same bytes.
    from oracle import formats
    B, T = 1, 320
    d = synth.decode_workload(B=B, T=T, kdtype="mxfp4", seed=405)
    rng = np.random.default_rng(405)
    q = rng.standard_normal((32, 128))
    q[0] = 0.0
    q[1, :32] = rng.integers(-7, 8, 32) * 2.0 ** -133            # subnormal in bf16
    q[2, :32] = rng.integers(-7, 8, 32) * 2.0 ** -126            # amax near 2^-123: X clamps
    q[3, :8] = [1.25, 0.6875, 0.375, -0.3125, 0.875, -0.875, 2.5, -2.5]   # ties
    q[3, 20] = 3.0
    q[4] = rng.standard_normal(128) * 2.0 ** 100
    q[5] = 0.0
    q[5, [3, 40, 77, 127]] = [1.5, -3.0e-3, 7.0, -2.0e20]      # one element per block
    q[6, ::2] = -0.0
    q_raw = formats.f64_to_bf16(q)
    w = rng.uniform(0.5, 1.5, 32)
    w[4] = 2.0 ** -100
    q_t = torch.from_numpy(q_raw.view(np.int16)).reshape(1, 1, 32, 128).cuda()
    w_t = torch.from_numpy(w.astype(np.float32)).reshape(1, 1, 32).cuda()
    vis_t = torch.tensor([[T]], dtype=torch.int32).cuda()
    sc = torch.full((1, 1, T), float("nan"), device="cuda")
    print("fp4 query special blocks", flush=True)
    csa.index_score(q_t, w_t, _keys(d, True), vis_t, scores=sc)
    torch.cuda.synchronize()
    kr = _oracle_rows(d["k_idx"], T, 0, T)
    ref = pipeline.scores_prefix(q_raw, w.astype(np.float32).astype(np.float64), kr, "mxfp4_qk", T)
    g = _np(sc)[0, 0].astype(np.float64)
    tol = 1e-5 * np.abs(ref) + 1e-6 * np.abs(ref).max()
    assert np.all(np.abs(g - ref) <= tol), f"max err {np.abs(g - ref).max()}"


def test_mxfp4_keys_rejected_for_prefill_rows():
    d = synth.decode_workload(B=1, T=1024, kdtype="mxfp4", seed=404)
    q = torch.zeros(1, 16, 32, 128, dtype=torch.int16, device="cuda")
    w = torch.zeros(1, 16, 32, device="cuda")
    vis = torch.full((1, 16), 1024, dtype=torch.int32, device="cuda")
    sc = torch.empty(1, 16, 1024, device="cuda")
    for qk in (False, True):
        with pytest.raises(csa.Csa2Error) as e:
            csa.index_score(q, w, _keys(d, qk), vis, scores=sc)
        assert e.value.status == 3
