"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Selections must agree exactly except for ties within 1e-6 of the k-th key;
attention outputs within |g - o| <= 2e-3 + 1e-2 |o|.  Steps downstream of a
selection are fed the GPU's selection (after it passed its own check), so a
legal tie swap upstream cannot cascade.
"""
import numpy as np
import pytest
import torch

from _helpers import check_attention, check_selection, u16
from oracle import attention as oattn
from oracle import formats, indexer, pipeline
from oracle import topk as otopk
import synth

pytestmark = pytest.mark.gpu

csa = None


@pytest.fixture(scope="module", autouse=True)
def _gpu_lib():
    global csa
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import compressed_sparse_attention_index_amd as m
    m.lib()   # raises if the HIP library is missing
    csa = m


def _np(t):
    return t.detach().cpu().numpy()


def _kraw(d, b):
    k = _np(d["k_idx"][b])
    return (k.view(np.uint16), "bf16") if d["kdtype"] == "bf16" else (k, "fp8")


def _scan(d, vis=None, want_scores=True):
    B, n_q, N = d["B"], d["n_q"], d["k_idx"].shape[1]
    vis_t = (d["vis_len"] if vis is None else torch.as_tensor(vis, dtype=torch.int32).reshape(B, n_q)).cuda()
    sc = torch.full((B, n_q, N), float("nan"), device="cuda") if want_scores else None
    bm = torch.full((B, n_q, (N + 7) // 8), float("nan"), device="cuda")
    csa.index_score(d["q_idx"].cuda(), d["w_idx"].cuda(), d["k_idx"].cuda(), vis_t, scores=sc,
                    block_max=bm)
    torch.cuda.synchronize()
    return vis_t, sc, bm


# --------------------------------------------------------------------------- scan
@pytest.mark.parametrize("kdtype,T", [("bf16", 2048), ("fp8", 2048), ("fp8", 4133)])
def test_index_score_ragged(kdtype, T):
    vis = [0, 1, 7, 8, 9, 33, 511, 512, 513, T - 1, T]
    B = len(vis)
    d = synth.decode_workload(B=B, T=T, kdtype=kdtype, seed=11, heavy_frac=0.01)
    print(f"index_score kdtype={kdtype} T={T} vis={vis}", flush=True)
    _, sc, bm = _scan(d, vis)
    sc, bm = _np(sc), _np(bm)
    for b, v in enumerate(vis):
        kr, kd = _kraw(d, b)
        ref = pipeline.scores_prefix(u16(d["q_idx"][b, 0]), _np(d["w_idx"][b, 0]), kr, kd, v)
        g = sc[b, 0, :v].astype(np.float64)
        tol = 1e-5 * np.abs(ref) + 1e-6 * (np.abs(ref).max() if v else 0)
        assert np.all(np.abs(g - ref) <= tol), f"row {b}: max err {np.abs(g - ref).max()}"
        assert np.all(np.isnan(sc[b, 0, v:])), "scores past vis_len must stay unwritten"
        nb = (v + 7) // 8
        bref = indexer.block_max(ref, v)
        assert np.all(np.abs(bm[b, 0, :nb] - bref) <= 1e-5 * np.abs(bref) + 1e-6 * (np.abs(ref).max() if v else 0))
        assert np.all(np.isnan(bm[b, 0, nb:]))


@pytest.mark.parametrize("kdtype,n_q,prefix", [("bf16", 40, 1000), ("bf16", 70, 5000),
                                               ("fp8", 70, 5000)])
def test_index_score_prefill_rows(kdtype, n_q, prefix):
    # Prefill-shaped call (n_q >= 16): per-row visible lengths, shared keys;
    # 70 rows span several row groups plus a ragged one, and 2,500+ entries
    # span every key chunk of a group.
    d = synth.prefill_workload(n_q=n_q, prefix_tokens=prefix, seed=12, kdtype=kdtype)
    print(f"index_score prefill {kdtype} n_q={n_q} prefix={prefix}", flush=True)
    vis_t, sc, bm = _scan(d)
    sc, bm, vis = _np(sc), _np(bm), _np(vis_t)[0]
    kr, kd = _kraw(d, 0)
    for j in range(n_q):
        ref = pipeline.scores_prefix(u16(d["q_idx"][0, j]), _np(d["w_idx"][0, j]), kr, kd, vis[j])
        g = sc[0, j, :vis[j]].astype(np.float64)
        assert np.all(np.abs(g - ref) <= 1e-5 * np.abs(ref) + 1e-6 * np.abs(ref).max()), j
        assert np.all(np.isnan(sc[0, j, vis[j]:]))
        nb = (vis[j] + 7) // 8
        bref = indexer.block_max(ref, vis[j])
        assert np.all(np.abs(bm[0, j, :nb] - bref) <= 1e-5 * np.abs(bref) + 1e-6 * np.abs(ref).max()), j
        assert np.all(np.isnan(bm[0, j, nb:])), j


# --------------------------------------------------------------------------- selection
def _select_case(keys_rows, vis_rows, k, kind):
    """GPU block/flat selection on given fp32 keys vs the oracle on the same fp32 keys."""
    rows = len(keys_rows)
    n = max(len(x) for x in keys_rows)
    if kind == "blocks":
        N = 8 * n
        arr = torch.zeros(rows, 1, n, dtype=torch.float32)
    else:
        N = n
        arr = torch.zeros(rows, 1, n, dtype=torch.float32)
    for i, x in enumerate(keys_rows):
        arr[i, 0, :len(x)] = torch.from_numpy(np.asarray(x, dtype=np.float32))
    vis = torch.tensor(vis_rows, dtype=torch.int32).reshape(rows, 1).cuda()
    out = torch.full((rows, 1, k), -7, dtype=torch.int32, device="cuda")
    if kind == "blocks":
        csa.block_topk(arr.cuda(), vis, N, k, out)
    else:
        ks = torch.zeros(rows, 1, k, device="cuda")
        csa.reindex_topk(csa.MODE_FULL, vis, N, k, out, scores=arr.cuda(), idx_score=ks)
    torch.cuda.synchronize()
    out = _np(out)
    for i in range(rows):
        x32 = arr[i, 0].numpy().astype(np.float64)
        if kind == "blocks":
            nb = (vis_rows[i] + 7) // 8
            ref = otopk.block_topk(x32[:nb], k)
        else:
            ref = otopk.flat_topk(x32, vis_rows[i], k)
        assert np.array_equal(out[i, 0], ref), f"{kind} row {i}: exact selection differs"


@pytest.mark.parametrize("kind", ["blocks", "flat"])
def test_select_exact_on_fp32_keys(kind):
    rng = np.random.default_rng(21)
    rows, vis = [], []
    n = 9000
    cases = [
        rng.standard_normal(n),                         # distinct
        np.round(rng.standard_normal(n) * 4) / 4,       # heavy ties
        np.full(n, 3.25),                               # all equal
        -np.abs(rng.standard_normal(n)),                # negative
        np.where(rng.uniform(size=n) < 0.5, 0.0, rng.standard_normal(n)),  # many zeros
        rng.standard_normal(n) * 1e-30,                 # tiny range
        np.concatenate([rng.standard_normal(5000) + 1e6, rng.standard_normal(4000)]),  # two clusters
    ]
    vis_sizes = [n, n, n, n, 4001, 17, 0]
    for c, v in zip(cases, vis_sizes):
        rows.append(c)
        vis.append(8 * v if kind == "blocks" else v)
    if kind == "blocks":
        vis = [min(x, 8 * n) for x in vis]
    print(f"select {kind}", flush=True)
    for k in ((1, 16, 512, 2048) if kind == "blocks" else (1, 16, 100, 512)):
        _select_case(rows, vis, k, kind)


@pytest.mark.parametrize("n", [73728, 80000])
def test_flat_select_long_rows(n):
    # 73,728 items is the largest row held in registers; 80,000 takes the
    # streaming selection.
    rng = np.random.default_rng(23)
    rows = [rng.standard_normal(n), np.round(rng.standard_normal(n) * 8) / 8,
            rng.standard_normal(n) * 1e-3 + 5.0]
    vis = [n, n - 1, 40000]
    print(f"flat select long rows n={n}", flush=True)
    for k in (1, 512):
        _select_case(rows, vis, k, "flat")


def test_flat_select_many_rows():
    # More rows than compute units, so workgroups of every row kind run side
    # by side over several rounds of the grid.  Row kinds cycle (distinct,
    # heavy ties, all equal, short, empty, two clusters), so every marking
    # path (ballot stores, list marks, the whole-row pass) is exercised.
    rng = np.random.default_rng(25)
    n = 9000
    kinds = [
        lambda: rng.standard_normal(n),
        lambda: np.round(rng.standard_normal(n) * 4) / 4,
        lambda: np.full(n, -2.5),
        lambda: rng.standard_normal(n),
        lambda: rng.standard_normal(n),
        lambda: np.concatenate([rng.standard_normal(5000) + 1e6, rng.standard_normal(4000)]),
    ]
    vis_of = [n, n - 5, n, 300, 0, 7001]
    rows, vis = [], []
    for i in range(600):
        rows.append(kinds[i % 6]())
        vis.append(vis_of[i % 6])
    print("flat select 600 rows", flush=True)
    for k in (100, 512):
        _select_case(rows, vis, k, "flat")


def test_block_topk_workspace_contents():
    # The block Top-K histograms live in the workspace and must start at
    # zero; every call leaves them zeroed.  A workspace that did not start at
    # zero (garbage, or another row count's layout) must still give the exact
    # pool, by the slow exact pass, and be left zeroed for the next call.
    rng = np.random.default_rng(24)
    n, k = 20000, 2048
    keys = [rng.standard_normal(n), np.round(rng.standard_normal(n) * 4) / 4,
            np.full(n, -1.5), rng.standard_normal(n), rng.standard_normal(1000)]
    vis_rows = [8 * n, 8 * n - 3, 8 * n, 8 * 7001, 8 * 1000]    # the last has n <= k
    rows = len(keys)
    arr = torch.zeros(rows, 1, n, dtype=torch.float32)
    for i, x in enumerate(keys):
        arr[i, 0, :len(x)] = torch.from_numpy(x.astype(np.float32))
    bm = arr.cuda()
    N = 8 * n
    nbytes = csa.workspace_size(csa.OP_BLOCK_TOPK, rows, 1, N, 0, k)
    refs = [otopk.block_topk(arr[i, 0].numpy().astype(np.float64)[:(vis_rows[i] + 7) // 8], k)
            for i in range(rows)]

    def run(r, ws, label):
        vis = torch.tensor(vis_rows[:r], dtype=torch.int32).reshape(r, 1).cuda()
        out = torch.full((r, 1, k), -7, dtype=torch.int32, device="cuda")
        print(f"block_topk workspace case: {label}, rows={r}", flush=True)
        csa.block_topk(bm[:r], vis, N, k, out, ws=ws)
        torch.cuda.synchronize()
        out = _np(out)
        for i in range(r):
            assert np.array_equal(out[i, 0], refs[i]), f"{label}: row {i} differs"
        h = _np(ws[:2 * r * 4096 * 4].view(torch.int32)).reshape(2, r, 4096)
        for i in range(r):
            if (vis_rows[i] + 7) // 8 > k:
                assert not h[:, i].any(), f"{label}: row {i} histograms not left zeroed"

    for fill in (0xA7, 0xFF):
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device="cuda")
        run(rows, ws, f"garbage 0x{fill:02X}")
        run(rows, ws, "after a call")
        run(2, ws, "fewer rows")
        run(rows, ws, "more rows again")


def test_pool_topk_stored_scores_exact():
    # FULL mode from stored scores at the pool positions (fp32 keys, exact).
    rng = np.random.default_rng(22)
    rows, N, kb = 5, 20000, 2048
    sc = rng.standard_normal((rows, 1, N)).astype(np.float32)
    sc[1] = np.round(sc[1] * 2) / 2
    sc[2] = 1.0
    vis = np.array([N, N, N, 9999, 5], dtype=np.int32)
    pools = np.full((rows, 1, kb), -1, np.int32)
    for i in range(rows):
        nb = (vis[i] + 7) // 8
        sel = np.sort(rng.choice(nb, size=min(nb, 1500), replace=False))
        pools[i, 0, :len(sel)] = sel
    out = torch.zeros(rows, 1, 512, dtype=torch.int32, device="cuda")
    ks = torch.zeros(rows, 1, 512, device="cuda")
    csa.reindex_topk(csa.MODE_FULL, torch.from_numpy(vis).reshape(rows, 1).cuda(), N, 512, out,
                     scores=torch.from_numpy(sc).cuda(), pool_blocks=torch.from_numpy(pools).cuda(),
                     idx_score=ks)
    torch.cuda.synchronize()
    out, ks = _np(out), _np(ks)
    for i in range(rows):
        pos = otopk.pool_positions(pools[i, 0], vis[i])
        ref = otopk.pool_topk(sc[i, 0, pos].astype(np.float64), pos, 512)
        assert np.array_equal(out[i, 0], ref), i
        m = ref >= 0
        assert np.array_equal(ks[i, 0, m], sc[i, 0, ref[m]])
        assert np.all(np.isneginf(ks[i, 0, ~m]))


# --------------------------------------------------------------------------- Full / Reindex layers
def _full_layer_gpu(d, rescore_full):
    B, N = d["B"], d["k_idx"].shape[1]
    vis_t, sc, bm = _scan(d, want_scores=not rescore_full)
    pool = torch.zeros(B, 1, 2048, dtype=torch.int32, device="cuda")
    csa.block_topk(bm, vis_t, N, 2048, pool)
    idx = torch.zeros(B, 1, 512, dtype=torch.int32, device="cuda")
    if rescore_full:
        csa.reindex_topk(csa.MODE_FULL, vis_t, N, 512, idx, q_idx=d["q_idx"].cuda(),
                         w_idx=d["w_idx"].cuda(), k_idx=d["k_idx"].cuda(), pool_blocks=pool)
    else:
        csa.reindex_topk(csa.MODE_FULL, vis_t, N, 512, idx, scores=sc, pool_blocks=pool)
    torch.cuda.synchronize()
    return vis_t, bm, pool, idx


def _check_full_row(d, b, bm, pool, idx, vis):
    kr, kd = _kraw(d, b)
    ref = pipeline.full_layer(u16(d["q_idx"][b, 0]), _np(d["w_idx"][b, 0]), kr, kd, vis)
    check_selection(_np(pool[b, 0]), ref["pool"], lambda j: ref["block_max"][j], what=f"pool row {b}")
    # Pool Top-512 against the oracle run on the GPU's pool (hierarchy invariant:
    # also the global Top-512 whenever the pools agree).
    pos = otopk.pool_positions(_np(pool[b, 0]), vis)
    ref_idx = otopk.pool_topk(ref["scores"][pos], pos, 512)
    check_selection(_np(idx[b, 0]), ref_idx, lambda t: ref["scores"][t], what=f"idx row {b}")
    return ref


@pytest.mark.parametrize("rescore_full", [False, True])
@pytest.mark.parametrize("T,kdtype", [(2048, "bf16"), (20011, "fp8"), (16384, "fp8"), (200, "fp8")])
def test_full_layer(T, kdtype, rescore_full):
    d = synth.decode_workload(B=3, T=T, kdtype=kdtype, seed=31, heavy_frac=0.01)
    print(f"full layer T={T} {kdtype} rescore={rescore_full}", flush=True)
    vis_t, bm, pool, idx = _full_layer_gpu(d, rescore_full)
    for b in range(3):
        _check_full_row(d, b, bm, pool, idx, T)


def test_reindex_layer():
    T = 40000
    d = synth.decode_workload(B=2, T=T, kdtype="fp8", seed=32, lognormal_sigma=0.5, reindex=True)
    print("reindex layer", flush=True)
    vis_t, bm, pool, _ = _full_layer_gpu(d, True)
    idx2 = torch.zeros(2, 1, 512, dtype=torch.int32, device="cuda")
    csa.reindex_topk(csa.MODE_REINDEX, vis_t, T, 512, idx2, q_idx=d["q_idx2"].cuda(),
                     w_idx=d["w_idx2"].cuda(), k_idx=d["k_idx"].cuda(), pool_blocks=pool)
    torch.cuda.synchronize()
    for b in range(2):
        kr, kd = _kraw(d, b)
        re = pipeline.reindex_layer(u16(d["q_idx2"][b, 0]), _np(d["w_idx2"][b, 0]), kr, kd,
                                    _np(pool[b, 0]), T)
        key = dict(zip(re["positions"].tolist(), re["scores"].tolist()))
        check_selection(_np(idx2[b, 0]), re["idx"], lambda t: np.array([key[int(x)] for x in t]),
                        what=f"reindex row {b}")


# --------------------------------------------------------------------------- attention
def _attn_gpu(d, idx, q=None, swa=None, window=128, replay_start=-1, reuse=False, sink=None):
    kv_fmt = csa.KV_FP4_E4M3_16 if d.get("kv_fmt") == "e4m3_16" else csa.KV_MXFP4_E8M0_32
    q = d["q"] if q is None else q
    swa = d["swa"] if swa is None else swa
    B, n_q = q.shape[0], q.shape[1]
    out = torch.zeros(B, n_q, 64, 512, dtype=torch.int16, device="cuda")
    lse = torch.zeros(B, n_q, 64, device="cuda")
    fn = csa.reuse_attn if reuse else csa.sparse_attn_decode
    fn(q.cuda(), d["kv_fp4"].cuda(), d["kv_scale"].cuda(), idx.cuda(), swa.cuda(),
       d["swa_pos0"].cuda(), d["q_pos"].cuda(), d["sm_scale"], out, lse=lse, window=window,
       replay_start=replay_start, sink=None if sink is None else sink.cuda(), kv_fmt=kv_fmt)
    torch.cuda.synchronize()
    return u16(out), _np(lse)


def _attn_ref(d, b, j, idx_row, q=None, swa=None, window=128, replay_start=-1, sink=None):
    q = d["q"] if q is None else q
    swa = d["swa"] if swa is None else swa
    idx_row = np.asarray(idx_row, dtype=np.int64)
    sel = idx_row[idx_row >= 0]
    fp4 = _np(d["kv_fp4"][b][torch.as_tensor(sel, dtype=torch.long, device=d["kv_fp4"].device)])
    sc = _np(d["kv_scale"][b][torch.as_tensor(sel, dtype=torch.long, device=d["kv_scale"].device)])
    return pipeline.attention(u16(q[b, j]), fp4, sc, np.arange(len(sel)), _np(swa[b]),
                              int(d["swa_pos0"][b]), int(d["q_pos"][b, j]), d["sm_scale"],
                              window, replay_start, sink, kv_fmt=d.get("kv_fmt", "e8m0_32"))


@pytest.mark.parametrize("n_q", [1, 16])
@pytest.mark.parametrize("case", ["topk512", "ragged", "invalid", "dense", "window16", "replay",
                                  "seq_start", "no_main", "mixed_chunk"])
def test_attention_cases(case, n_q):
    # n_q = 1: decode rows (head-group kernel); n_q = 16: prefill-shaped rows
    # (one workgroup per row), the sequence's last 16 positions, each row with
    # its own entries and its own (partly stored) window.
    T, B = 2048, 3
    d = synth.decode_workload(B=B, T=T, kdtype="bf16", seed=41)
    rng = np.random.default_rng(41)
    if n_q > 1:
        g = torch.Generator().manual_seed(42)
        d["q"] = synth.to_bf16_bits(torch.randn(B, n_q, 64, 512, generator=g))
        d["q_pos"] = (torch.arange(n_q, dtype=torch.int32) + (T - n_q)).repeat(B, 1)
    window, replay = 128, -1
    top_k = 512
    if case == "ragged":
        top_k = 100
    if case == "dense":
        top_k = 300
    if case == "no_main":
        top_k = 0
    if case == "mixed_chunk":
        # 160 selected slots: one 64-entry chunk holds 32 selected and 32 window
        # entries, and the last chunk is half past the window.
        top_k = 160
    idx = np.stack([np.sort(rng.choice(T, size=max(top_k, 1), replace=False))[:top_k]
                    for _ in range(B * n_q)]).reshape(B, n_q, top_k)
    if case == "dense":
        idx = np.tile(np.arange(300), (B, n_q, 1))
    if case == "invalid":
        idx[:, :, ::3] = -1
        idx[0] = -1
    if case == "window16":
        window = 16
    if case == "replay":
        replay = T - 50
    if case == "seq_start":
        # queries near the sequence start: the window holds positions 0..q_pos
        d["swa_pos0"][:] = 0
        d["q_pos"][:, :] = (torch.tensor([0, 5, 127], dtype=torch.int32)[:, None]
                            + torch.arange(n_q, dtype=torch.int32)[None, :])
    idx_t = torch.from_numpy(idx.astype(np.int32))
    print(f"attention case={case} n_q={n_q}", flush=True)
    out, lse = _attn_gpu(d, idx_t, window=window, replay_start=replay)
    for b in range(B):
        for j in range(n_q):
            o, l = _attn_ref(d, b, j, idx[b, j], window=window, replay_start=replay)
            check_attention(out[b, j], lse[b, j], o, l, what=f"{case} row ({b}, {j})")


def test_attention_dense_equals_sdpa_through_gpu():
    # Every entry selected: the GPU result matches dense attention over all entries.
    T = 256
    d = synth.decode_workload(B=1, T=T, kdtype="bf16", seed=42)
    idx = torch.arange(T, dtype=torch.int32).reshape(1, 1, T)
    out, lse = _attn_gpu(d, idx)
    kv = np.concatenate([formats.mxfp4_to_f64(_np(d["kv_fp4"][0]), _np(d["kv_scale"][0])),
                         formats.e4m3_to_f64(_np(d["swa"][0]))])
    qf = formats.bf16_to_f64(u16(d["q"][0, 0]))
    qt = torch.from_numpy(qf)[None, :, None, :]
    kt = torch.from_numpy(kv)[None, None].expand(1, 64, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=d["sm_scale"])
    check_attention(out[0, 0], None, ref[0, :, 0].numpy(), None, what="dense")


def test_attention_extreme_scale_codes():
    # E8M0 codes across the range the dequantisation holds exactly in bf16,
    # one code per block index for every entry: 0 (the subnormal scale
    # 2^-127), 1, 2, 64, 100, 125, 126, 127, 224 and 190.  The E2M1 nibbles
    # come from N(0,1) values quantised as in the workloads, whose block
    # codes sit near 126, so at code 126 a block holds N(0,1)-like values and
    # at code c they are scaled by 2^(c - 126).  The query is zero on the
    # dims of the two huge blocks, so the logits stay O(1), and the window
    # (FP8, O(1)) is zero on the dims of the five tiny blocks.  Each output
    # dim is compared in units of its block's scale (at least 1 where the
    # window contributes): the tolerance's absolute term is meant for O(1)
    # values, and the tiny blocks then check the subnormal scales.
    T, B = 700, 2
    d = synth.decode_workload(B=B, T=T, kdtype="bf16", seed=81)
    rng = np.random.default_rng(81)
    codes = np.array([0, 1, 2, 64, 100, 125, 126, 126, 126, 127, 126, 126, 126, 126, 224, 190],
                     np.uint8)
    d["kv_scale"] = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(codes, (B, T, 16))))
    q = d["q"].view(torch.bfloat16).clone()
    q[..., 448:] = 0
    d["q"] = q.view(torch.int16)
    d["swa"] = d["swa"].clone()
    d["swa"][..., :160] = 0
    idx = np.stack([np.sort(rng.choice(T, size=512, replace=False)) for _ in range(B)])
    print("attention extreme E8M0 codes", flush=True)
    out, lse = _attn_gpu(d, torch.from_numpy(idx.astype(np.int32)).reshape(B, 1, 512))
    unit = np.ldexp(1.0, codes.astype(int) - 126)
    unit[5:14] = np.maximum(unit[5:14], 1.0)
    dim_scale = np.repeat(unit, 32)
    for b in range(B):
        o, l = _attn_ref(d, b, 0, idx[b])
        assert np.abs(o[:, 448:480]).max() > 2.0 ** 90
        check_attention(out[b, 0], lse[b, 0], o, l, what=f"extreme codes row {b}",
                        dim_scale=dim_scale)
        # The subnormal scales are not flushed: where the oracle's output in
        # the code-0 block exceeds two bf16 subnormal steps, the GPU's is not 0.
        g0 = out[b, 0][:, :32]
        big = np.abs(o[:, :32]) > 2 * 2.0 ** -133
        assert big.any() and np.all(g0[big] & 0x7FFF != 0)


# E4M3FN scale codes of the per-16 format, one per block index (dims 16 i
# .. 16 i + 15): the smallest subnormals and the subnormal/normal boundary
# (blocks 0, 1, 2, 8), scales with every mantissa bit set or clear, the
# largest value 448 (block 7) and 26 (block 14), negative codes (the
# dequantised values change sign) and 0 (a block of zeros, block 11).
_E4M3_CODES = np.array([0x01, 0x07, 0x08, 0x30, 0x38, 0x39, 0x3F, 0x7E,
                        0x81, 0xB8, 0xB0, 0x00, 0x3A, 0x40, 0x5D, 0x3F] * 2, np.uint8)
_E4M3_TINY = [0, 1, 2, 8]
_E4M3_BIG = [7, 14]


@pytest.mark.parametrize("case", ["recipe", "codes"])
@pytest.mark.parametrize("n_q", [1, 16])
def test_attention_e4m3_scales(case, n_q):
    # The per-16 E4M3 scale format through both attention kernels (decode
    # rows, n_q = 1, and prefill-shaped rows, n_q = 16).  "recipe": N(0,1)
    # entries encoded as in the workloads.  "codes": the same nibbles with
    # every entry's scales replaced by _E4M3_CODES.  There the query is zero
    # on the dims of the two big blocks and scaled by 1/4 elsewhere, so the
    # logits stay O(1) and the softmax spreads over many entries (P is
    # rounded to bf16 before P.V, an error of up to 2^-9 of each entry's
    # share, which a softmax peaked on a few entries of values up to 12 would
    # show above the O(1) tolerance); the window (FP8, O(1)) is zero on the
    # dims of the tiny blocks; each output
    # dim is compared in units of its block's |scale| (at least 1 where the
    # window contributes), so that the tiny blocks are checked at their own
    # resolution and the big ones are not held to an O(1) absolute bound.
    T, B = 1500, 2
    d = synth.decode_workload(B=B, T=T, kdtype="bf16", seed=91, kv_fmt="e4m3_16")
    assert d["kv_scale"].shape == (B, T, 32)
    rng = np.random.default_rng(91)
    g = torch.Generator().manual_seed(92)
    q = torch.randn(B, n_q, 64, 512, generator=g)
    dim_scale = None
    if case == "codes":
        d["kv_scale"] = torch.from_numpy(
            np.ascontiguousarray(np.broadcast_to(_E4M3_CODES, (B, T, 32))))
        unit = np.abs(formats.e4m3_to_f64(_E4M3_CODES))
        unit[11] = unit[27] = 1.0
        q *= 0.25
        for blk in _E4M3_BIG:
            for k in (blk, blk + 16):
                q[..., 16 * k:16 * k + 16] = 0
        d["swa"] = d["swa"].clone()
        for blk in _E4M3_TINY:
            for k in (blk, blk + 16):
                d["swa"][..., 16 * k:16 * k + 16] = 0
        tiny = np.zeros(32, bool)
        tiny[_E4M3_TINY] = tiny[[k + 16 for k in _E4M3_TINY]] = True
        unit = np.where(tiny, unit, np.maximum(unit, 1.0))
        dim_scale = np.repeat(unit, 16)
    d["q"] = synth.to_bf16_bits(q)
    d["q_pos"] = torch.full((B, n_q), T - 1, dtype=torch.int32)
    top_k = 300
    idx = np.stack([np.stack([np.sort(rng.choice(T, size=top_k, replace=False))
                              for _ in range(n_q)]) for _ in range(B)])
    idx[0, 0, ::7] = -1
    print(f"attention E4M3 scales case={case} n_q={n_q}", flush=True)
    out, lse = _attn_gpu(d, torch.from_numpy(idx.astype(np.int32)))
    for b in range(B):
        for j in sorted({0, n_q - 1}):
            o, l = _attn_ref(d, b, j, idx[b, j])
            if case == "codes":
                assert np.abs(o[:, 112:128]).max() > 100.0     # the 448 block is in the output
            check_attention(out[b, j], lse[b, j], o, l, what=f"E4M3 {case} row {b},{j}",
                            dim_scale=dim_scale)


@pytest.mark.parametrize("n_q", [1, 16])
def test_attention_single_entry_is_its_dequantisation(n_q):
    # Zero query, one selected entry and no window: every logit is 0, the
    # softmax weight is exactly 1, and each head's output is the entry
    # itself, dequantised: bit-exact in bf16 for both scale formats and both
    # kernels, over E8M0 codes whose values stay normal in fp32 and finite in
    # bf16 (3 .. 252) and the special E4M3 codes (subnormal, negative, zero,
    # 448).
    T, B = 64, 4
    for fmt, codes, dec in (("e8m0_32", np.array([3, 64, 100, 126, 127, 130, 200, 252] * 2, np.uint8),
                             formats.mxfp4_to_f64),
                            ("e4m3_16", _E4M3_CODES, formats.fp4e4_to_f64)):
        d = synth.decode_workload(B=B, T=T, kdtype="bf16", seed=93, kv_fmt=fmt)
        d["kv_scale"] = torch.from_numpy(
            np.ascontiguousarray(np.broadcast_to(codes, d["kv_scale"].shape)))
        d["q"] = torch.zeros(B, n_q, 64, 512, dtype=torch.int16)
        d["q_pos"] = torch.full((B, n_q), T - 1, dtype=torch.int32)
        idx = (np.arange(B * n_q).reshape(B, n_q, 1) * 3 % T).astype(np.int32)
        print(f"attention single entry {fmt} n_q={n_q}", flush=True)
        out, lse = _attn_gpu(d, torch.from_numpy(idx), window=0)
        got = (out.astype(np.uint32) << 16).view(np.float32)
        for b in range(B):
            for j in range(n_q):
                e = idx[b, j, 0]
                want = dec(_np(d["kv_fp4"][b, e])[None], _np(d["kv_scale"][b, e])[None])[0]
                assert np.array_equal(got[b, j], np.broadcast_to(want, (64, 512))), \
                    f"{fmt} row {b},{j}: the output is not entry {e}"
                assert np.all(lse[b, j] == 0.0)


def test_attention_single_split_and_reuse_identical():
    # 512 query rows: each workgroup covers a whole row (no split partials).
    d = synth.prefill_workload(n_q=512, prefix_tokens=4000, seed=43)
    N = d["kv_fp4"].shape[1]
    rng = np.random.default_rng(43)
    vis = _np(d["vis_len"])[0]
    idx = np.stack([np.sort(rng.choice(v, size=512, replace=False)) for v in vis]).astype(np.int32)
    idx_t = torch.from_numpy(idx).reshape(1, 512, 512)
    print("attention 512 rows", flush=True)
    out, lse = _attn_gpu(d, idx_t)
    out2, lse2 = _attn_gpu(d, idx_t, reuse=True)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    for j in (0, 1, 255, 511):
        o, l = _attn_ref(d, 0, j, idx[j])
        check_attention(out[0, j], lse[0, j], o, l, what=f"prefill row {j}")
    assert N == 2000 + 256


def test_attention_running_max_moves_mid_row():
    # 256 rows: each workgroup walks a whole row (10 chunks).  The window
    # entries, which come last, lie along head 0's query of row 0 (0.5 q plus
    # a little noise), so for that head their logits (about 11) exceed the
    # selected entries' by far more than the lazy-rescale margin: the running
    # max jumps partway through the row and the output and sums are rescaled.
    # The values stay O(1), so the bf16 rounding of P stays inside the
    # tolerance.
    d = synth.prefill_workload(n_q=256, prefix_tokens=4000, seed=46)
    q0 = d["q"][0, 0, 0].view(torch.bfloat16).float()
    g = synth.Gen(47)
    d["swa"] = synth.to_fp8_bytes(0.5 * q0 + 0.1 * g.normal(*d["swa"].shape))
    rng = np.random.default_rng(46)
    vis = _np(d["vis_len"])[0]
    idx = np.stack([np.sort(rng.choice(v, size=512, replace=False)) for v in vis]).astype(np.int32)
    print("attention 256 rows, window along one query", flush=True)
    out, lse = _attn_gpu(d, torch.from_numpy(idx).reshape(1, 256, 512))
    for j in (0, 97, 255):
        o, l = _attn_ref(d, 0, j, idx[j])
        check_attention(out[0, j], lse[0, j], o, l, what=f"row {j}")
    # Head 0 of row 0 is dominated by the window: its lse is far above the
    # others'.
    assert lse[0, 0, 0] > 8.0 and np.median(lse[0, 0]) < 8.0


def test_prepared_attention_calls_match_direct_calls():
    # sparse_attn_call / reuse_attn_call pack the arguments once; every run
    # makes the same C call, so the outputs are the direct call's bits.
    T, B = 3000, 8
    d = synth.decode_workload(B=B, T=T, kdtype="bf16", seed=92)
    rng = np.random.default_rng(92)
    idx = torch.from_numpy(np.stack([np.sort(rng.choice(T, size=512, replace=False))
                                     for _ in range(B)]).astype(np.int32)).reshape(B, 1, 512)
    print("prepared attention calls", flush=True)
    for reuse in (False, True):
        want, want_lse = _attn_gpu(d, idx, reuse=reuse)
        out = torch.zeros(B, 1, 64, 512, dtype=torch.int16, device="cuda")
        lse = torch.zeros(B, 1, 64, device="cuda")
        mk = csa.reuse_attn_call if reuse else csa.sparse_attn_call
        call = mk(d["q"].cuda(), d["kv_fp4"].cuda(), d["kv_scale"].cuda(), idx.cuda(),
                  d["swa"].cuda(), d["swa_pos0"].cuda(), d["q_pos"].cuda(), d["sm_scale"], out,
                  lse=lse)
        for _ in range(2):
            out.zero_()
            lse.zero_()
            call.run()
            torch.cuda.synchronize()
            assert np.array_equal(u16(out), want) and np.array_equal(_np(lse), want_lse), reuse


def test_attention_batch_invariant():
    # The same query rows in batches of 64, 8 and 1 (and at another position
    # in the batch) give bit-identical outputs and lse: a row's arithmetic
    # does not depend on the other rows of the call ([V4 essay §6.4]).
    T, B = 4000, 64
    d = synth.decode_workload(B=B, T=T, kdtype="bf16", seed=91)
    rng = np.random.default_rng(91)
    idx = np.stack([np.sort(rng.choice(T, size=512, replace=False)) for _ in range(B)])
    idx_t = torch.from_numpy(idx.astype(np.int32)).reshape(B, 1, 512)
    print("attention batch invariance 64 / 8 / 1", flush=True)
    full, full_lse = _attn_gpu(d, idx_t)

    def sub(rows):
        e = {k: (v[rows] if torch.is_tensor(v) and v.dim() > 0 and v.shape[0] == B else v)
             for k, v in d.items()}
        return _attn_gpu(e, idx_t[rows])

    o8, l8 = sub(slice(8, 16))
    assert np.array_equal(o8, full[8:16]) and np.array_equal(l8, full_lse[8:16])
    for b in (0, 13, 63):
        o1, l1 = sub(slice(b, b + 1))
        assert np.array_equal(o1, full[b:b + 1]) and np.array_equal(l1, full_lse[b:b + 1]), b
    # Row 13 placed first in a batch of 2 with row 40.
    o2, l2 = sub(torch.tensor([13, 40]))
    assert np.array_equal(o2[0], full[13]) and np.array_equal(o2[1], full[40])


def test_attention_batch_invariant_prefill_rows():
    # Prefill-shaped calls (16 query rows per sequence): the same sequences
    # in a batch of 4 and alone give bit-identical outputs.
    T, B, n_q = 3000, 4, 16
    d = synth.decode_workload(B=B, T=T, kdtype="bf16", seed=92)
    g = torch.Generator().manual_seed(93)
    d["q"] = synth.to_bf16_bits(torch.randn(B, n_q, 64, 512, generator=g))
    d["q_pos"] = (T - n_q + torch.arange(n_q, dtype=torch.int32)).repeat(B, 1)
    d["swa"] = synth.to_fp8_bytes(torch.randn(B, 160, 512, generator=g))
    d["swa_pos0"] = torch.full((B,), T - 160, dtype=torch.int32)
    rng = np.random.default_rng(92)
    idx = np.stack([np.sort(rng.choice(T - n_q, size=512, replace=False)) for _ in range(B * n_q)])
    idx_t = torch.from_numpy(idx.astype(np.int32)).reshape(B, n_q, 512)
    print("attention batch invariance, prefill rows", flush=True)
    full, full_lse = _attn_gpu(d, idx_t)
    for b in (0, 3):
        e = {k: (v[b:b + 1] if torch.is_tensor(v) and v.dim() > 0 and v.shape[0] == B else v)
             for k, v in d.items()}
        o1, l1 = _attn_gpu(e, idx_t[b:b + 1])
        assert np.array_equal(o1, full[b:b + 1]) and np.array_equal(l1, full_lse[b:b + 1]), b
    o, l = _attn_ref(d, 1, 5, idx[1 * n_q + 5])
    check_attention(full[1, 5], full_lse[1, 5], o, l, what="prefill row (1, 5)")


def test_deterministic_reruns():
    d = synth.decode_workload(B=2, T=30000, kdtype="fp8", seed=44)
    a = _full_layer_gpu(d, True)
    b = _full_layer_gpu(d, True)
    for x, y in zip(a[1:], b[1:]):
        assert torch.equal(x, y)
    o1 = _attn_gpu(d, a[3].cpu())
    o2 = _attn_gpu(d, a[3].cpu())
    assert np.array_equal(o1[0], o2[0]) and np.array_equal(o1[1], o2[1])


# --------------------------------------------------------------------------- KV append
def _append_inputs(rng, B, n_new):
    """bf16 entries with per-block magnitudes from 2^-30 to 2^30 and planted
    edge cases: E2M1 and E4M3 ties, an all-zero block, subnormal-range and
    huge values, negative zeros, values past the FP8 range."""
    scale = np.exp2(rng.integers(-30, 30, size=(B, n_new, 16, 1)))
    kv = (rng.standard_normal((B, n_new, 16, 32)) * scale).reshape(B, n_new, 512)
    sw = rng.standard_normal((B, n_new, 512)) * np.exp2(rng.integers(-12, 9, size=(B, n_new, 1)))
    kv[0, 0, 0:32] = 0.0
    kv[0, 0, 32:64] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4) * 2.0 ** -3
    kv[0, 0, 64:96] = rng.standard_normal(32) * 1e-39
    kv[0, 0, 96:128] = rng.standard_normal(32) * 1e30
    kv[0, 0, 128:136] = -0.0
    vals = formats.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    sw[0, 0, :126] = mids
    sw[0, 1, :126] = -mids
    sw[0, 2, :8] = [500.0, -1e4, 448.0, 2.0 ** -10, -(2.0 ** -10), -0.0, 1e-30, 464.0]
    kv_bits = torch.from_numpy(kv.astype(np.float32)).to(torch.bfloat16).view(torch.int16)
    sw_bits = torch.from_numpy(sw.astype(np.float32)).to(torch.bfloat16).view(torch.int16)
    return kv_bits, sw_bits


def test_kv_append_exact():
    rng = np.random.default_rng(51)
    B, n_new, N_cap, S_cap = 5, 3, 40, 16
    kv_bits, sw_bits = _append_inputs(rng, B, n_new)
    # Rows past either end of a cache are skipped: pos 38 writes rows 38, 39;
    # pos -1 writes rows 0, 1; window rows follow p - swa_pos0.
    pos = np.array([0, 10, 38, -1, 39], np.int32)
    swa_pos0 = np.array([0, 5, 30, 0, 39], np.int32)
    fp4 = np.full((B, N_cap, 256), 0xA5, np.uint8)
    sc = np.full((B, N_cap, 16), 0xA5, np.uint8)
    swa = np.full((B, S_cap, 512), 0xA5, np.uint8)
    g = [torch.from_numpy(a.copy()).cuda() for a in (fp4, sc, swa)]
    print("kv_append edge cases", flush=True)
    csa.kv_append(kv_bits.cuda(), torch.from_numpy(pos).cuda(), g[0], g[1],
                  swa_new=sw_bits.cuda(), swa_kv=g[2], swa_pos0=torch.from_numpy(swa_pos0).cuda())
    torch.cuda.synchronize()
    want = pipeline.kv_append(fp4, sc, swa, kv_bits.numpy().view(np.uint16),
                              sw_bits.numpy().view(np.uint16), pos, swa_pos0)
    for name, got, ref in zip(("kv_fp4", "kv_scale", "swa"), g, want):
        assert np.array_equal(_np(got), ref), f"{name} differs from the oracle"


def test_kv_append_without_window():
    rng = np.random.default_rng(52)
    B, n_new, N_cap = 2, 5, 8
    kv_bits, _ = _append_inputs(rng, B, n_new)
    pos = np.array([3, 0], np.int32)
    fp4 = np.zeros((B, N_cap, 256), np.uint8)
    sc = np.zeros((B, N_cap, 16), np.uint8)
    g = [torch.from_numpy(a.copy()).cuda() for a in (fp4, sc)]
    print("kv_append main only", flush=True)
    csa.kv_append(kv_bits.cuda(), torch.from_numpy(pos).cuda(), g[0], g[1])
    torch.cuda.synchronize()
    want = pipeline.kv_append(fp4, sc, None, kv_bits.numpy().view(np.uint16), None, pos, None)
    assert np.array_equal(_np(g[0]), want[0]) and np.array_equal(_np(g[1]), want[1])


def _e4m3_append_inputs(rng, B, n_new):
    """bf16 entries for the per-16 E4M3 encoder, per-block magnitudes 2^-14
    .. 2^14, with its edge cases in sequence 0: blocks whose amax / 6 is an
    E4M3 midpoint (a tie, to the even code), a block whose elements sit on
    the E2M1 midpoints times its scale (ties, to the even code), an all-zero
    block, a block whose scale rounds to 0, one whose scale saturates at
    448, one with subnormal scales, and negative zeros."""
    kv = rng.standard_normal((B, n_new, 32, 16)) * np.exp2(rng.integers(-14, 14, size=(B, n_new, 32, 1)))
    kv = kv.reshape(B, n_new, 512)
    e4 = formats.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (e4[:-1] + e4[1:]) / 2
    # amax = 6 x midpoint, exact in bf16 (a midpoint has at most 5
    # significant bits): block 0 of entries (0, i).
    for i in range(min(n_new, 3)):
        m = mids[[40, 41, 77][i]]
        kv[0, i, 0:16] = rng.uniform(-1, 1, 16) * m * 6
        kv[0, i, 3] = 6 * m
    # A block with amax 6 s, s = 1.25, and elements on the E2M1 midpoints times s.
    kv[0, 0, 16:32] = np.array([6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0,
                                -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, -6]) * 1.25
    kv[0, 0, 32:48] = 0.0
    kv[0, 0, 48:64] = rng.standard_normal(16) * 2.0 ** -14     # amax / 6 below 2^-10: scale 0
    kv[0, 0, 64:80] = rng.standard_normal(16) * 1e5             # scale saturates at 448
    kv[0, 0, 80:96] = rng.standard_normal(16) * 2.0 ** -8       # subnormal scales
    kv[0, 0, 96:112] = -0.0
    return torch.from_numpy(kv.astype(np.float32)).to(torch.bfloat16).view(torch.int16)


def test_kv_append_e4m3_exact():
    rng = np.random.default_rng(53)
    B, n_new, N_cap, S_cap = 4, 5, 24, 8
    kv_bits = _e4m3_append_inputs(rng, B, n_new)
    _, sw_bits = _append_inputs(rng, B, n_new)
    pos = np.array([0, 19, -2, 7], np.int32)
    swa_pos0 = np.array([0, 15, 0, 3], np.int32)
    fp4 = np.full((B, N_cap, 256), 0x5A, np.uint8)
    sc = np.full((B, N_cap, 32), 0x5A, np.uint8)
    swa = np.full((B, S_cap, 512), 0x5A, np.uint8)
    g = [torch.from_numpy(a.copy()).cuda() for a in (fp4, sc, swa)]
    print("kv_append E4M3 scales", flush=True)
    csa.kv_append(kv_bits.cuda(), torch.from_numpy(pos).cuda(), g[0], g[1],
                  swa_new=sw_bits.cuda(), swa_kv=g[2], swa_pos0=torch.from_numpy(swa_pos0).cuda(),
                  kv_fmt=csa.KV_FP4_E4M3_16)
    torch.cuda.synchronize()
    want = pipeline.kv_append(fp4, sc, swa, kv_bits.numpy().view(np.uint16),
                              sw_bits.numpy().view(np.uint16), pos, swa_pos0, kv_fmt="e4m3_16")
    # The planted cases are present: a tie of amax / 6, scale code 0, 0x7E.
    codes = want[1][0, 0]
    assert 0x00 in codes and 0x7E in codes
    for name, got, ref in zip(("kv_fp4", "kv_scale", "swa"), g, want):
        assert np.array_equal(_np(got), ref), f"{name} differs from the oracle"


def test_multi_query_decode_rows():
    # n_q = 4 query tokens per sequence below the matrix-core threshold (the
    # decode scan, speculative-verification shape): each row scans its own
    # visible prefix of its sequence's keys, and attends with its own
    # position.
    B, T, n_q = 2, 3000, 4
    d = synth.decode_workload(B=B, T=T, kdtype="fp8", seed=61)
    g = torch.Generator().manual_seed(62)
    d["n_q"] = n_q
    d["q_idx"] = synth.to_bf16_bits(torch.randn(B, n_q, 32, 128, generator=g))
    d["w_idx"] = torch.rand(B, n_q, 32, generator=g)
    d["q"] = synth.to_bf16_bits(torch.randn(B, n_q, 64, 512, generator=g))
    vis = [T - 3, T - 2, T - 1, T, 1999, 2000, 2001, 2008]
    d["q_pos"] = (torch.tensor(vis, dtype=torch.int32) - 1).reshape(B, n_q)
    print("multi-query decode rows n_q=4", flush=True)
    _, sc, bm = _scan(d, vis)
    sc, bm = _np(sc), _np(bm)
    for b in range(B):
        kr, kd = _kraw(d, b)
        for j in range(n_q):
            v = vis[b * n_q + j]
            ref = pipeline.scores_prefix(u16(d["q_idx"][b, j]), _np(d["w_idx"][b, j]), kr, kd, v)
            tol = 1e-5 * np.abs(ref) + 1e-6 * np.abs(ref).max()
            assert np.all(np.abs(sc[b, j, :v].astype(np.float64) - ref) <= tol), f"row ({b}, {j})"
            assert np.all(np.isnan(sc[b, j, v:]))
            bref = indexer.block_max(ref, v)
            nb = (v + 7) // 8
            assert np.all(np.abs(bm[b, j, :nb] - bref) <= 1e-5 * np.abs(bref) + 1e-6 * np.abs(ref).max())
    rng = np.random.default_rng(63)
    idx = np.stack([np.sort(rng.choice(vis[r], size=512, replace=False)) for r in range(B * n_q)])
    out, lse = _attn_gpu(d, torch.from_numpy(idx.astype(np.int32)).reshape(B, n_q, 512))
    for b in range(B):
        for j in range(n_q):
            o, l = _attn_ref(d, b, j, idx[b * n_q + j])
            check_attention(out[b, j], lse[b, j], o, l, what=f"attention row ({b}, {j})")


def test_multi_query_rows_through_selection():
    # n_q = 4 query tokens per sequence (draft verification) through the whole
    # decode path: each row scans its own visible prefix, gets its own pool,
    # Full Top-k and Reindex Top-k (its own second indexer query), and its
    # attention.  Pools of 128 blocks and top_k = 200 keep every stage a real
    # selection at these sizes.
    B, T, n_q, kb, top_k = 2, 6000, 4, 128, 200
    d = synth.decode_workload(B=B, T=T, kdtype="fp8", seed=65, heavy_frac=0.01)
    g = torch.Generator().manual_seed(66)
    d["n_q"] = n_q
    d["q_idx"] = synth.to_bf16_bits(torch.randn(B, n_q, 32, 128, generator=g))
    d["w_idx"] = torch.rand(B, n_q, 32, generator=g)
    q_idx2 = synth.to_bf16_bits(torch.randn(B, n_q, 32, 128, generator=g))
    w_idx2 = torch.rand(B, n_q, 32, generator=g)
    d["q"] = synth.to_bf16_bits(torch.randn(B, n_q, 64, 512, generator=g))
    vis = [T - 3, T - 2, T - 1, T, 4001, 4002, 4003, 4010]
    d["q_pos"] = (torch.tensor(vis, dtype=torch.int32) - 1).reshape(B, n_q)
    print("multi-query rows through block / pool Top-K and attention", flush=True)
    vis_t, _, bm = _scan(d, vis, want_scores=False)
    pool = torch.full((B, n_q, kb), -7, dtype=torch.int32, device="cuda")
    csa.block_topk(bm, vis_t, T, kb, pool)
    idx = torch.full((B, n_q, top_k), -7, dtype=torch.int32, device="cuda")
    csa.reindex_topk(csa.MODE_FULL, vis_t, T, top_k, idx, q_idx=d["q_idx"].cuda(),
                     w_idx=d["w_idx"].cuda(), k_idx=d["k_idx"].cuda(), pool_blocks=pool)
    idx2 = torch.full((B, n_q, top_k), -7, dtype=torch.int32, device="cuda")
    csa.reindex_topk(csa.MODE_REINDEX, vis_t, T, top_k, idx2, q_idx=q_idx2.cuda(),
                     w_idx=w_idx2.cuda(), k_idx=d["k_idx"].cuda(), pool_blocks=pool)
    out, lse = _attn_gpu(d, idx2.cpu())
    torch.cuda.synchronize()
    for b in range(B):
        kr, kd = _kraw(d, b)
        for j in range(n_q):
            v = vis[b * n_q + j]
            ref = pipeline.full_layer(u16(d["q_idx"][b, j]), _np(d["w_idx"][b, j]), kr, kd, v,
                                      k_blocks=kb, top_k=top_k)
            gp = _np(pool[b, j])
            check_selection(gp, ref["pool"], lambda t: ref["block_max"][t], what=f"pool ({b},{j})")
            pos = otopk.pool_positions(gp, v)
            ri = otopk.pool_topk(ref["scores"][pos], pos, top_k)
            check_selection(_np(idx[b, j]), ri, lambda t: ref["scores"][t], what=f"idx ({b},{j})")
            re = pipeline.reindex_layer(u16(q_idx2[b, j]), _np(w_idx2[b, j]), kr, kd, gp, v,
                                        top_k=top_k)
            key = dict(zip(re["positions"].tolist(), re["scores"].tolist()))
            gi2 = _np(idx2[b, j])
            check_selection(gi2, re["idx"], lambda t: np.array([key[int(x)] for x in t]),
                            what=f"reindex ({b},{j})")
            o, l = _attn_ref(d, b, j, gi2)
            check_attention(out[b, j], lse[b, j], o, l, what=f"attention ({b},{j})")


@pytest.mark.parametrize("rows", [3, 256])
def test_attention_sink(rows):
    # Per-head sink logits (no sink, small, comparable to the logits, and one
    # that takes nearly all the mass), through the split merge (3 rows) and
    # the single-workgroup rows (256).
    T = 4000
    if rows == 3:
        d = synth.decode_workload(B=3, T=T, kdtype="bf16", seed=71)
    else:
        d = synth.prefill_workload(n_q=256, prefix_tokens=T, seed=72)
    B, n_q = d["q"].shape[0], d["q"].shape[1]
    rng = np.random.default_rng(73)
    sink = rng.uniform(-4.0, 6.0, 64)
    sink[:8] = -np.inf
    sink[8] = 40.0
    sink_t = torch.from_numpy(sink.astype(np.float32))
    nkv = d["kv_fp4"].shape[1]
    idx = np.stack([np.sort(rng.choice(nkv, size=512, replace=False)) for _ in range(B * n_q)])
    print(f"attention sink rows={rows}", flush=True)
    out, lse = _attn_gpu(d, torch.from_numpy(idx.astype(np.int32)).reshape(B, n_q, 512), sink=sink_t)
    for r in (range(B * n_q) if rows == 3 else (0, 97, 255)):
        b, j = divmod(r, n_q)
        o, l = _attn_ref(d, b, j, idx[r], sink=sink.astype(np.float32).astype(np.float64))
        check_attention(out[b, j], lse[b, j], o, l, what=f"sink row {r}")
