"""Parity at the full sizes of the workloads, in the launch configuration
the benchmark times, on query rows the oracle computes one by one.

Inputs are generated on the GPU by the seeded synthetic generator; the oracle
reads the same bytes (copied to the host) for the sampled rows.
"""
import numpy as np
import pytest
import torch

from _helpers import check_attention, check_selection, u16
from oracle import formats, pipeline
from oracle import topk as otopk
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


def _kraw(d, b):
    k = _np(d["k_idx"][b])
    return (k.view(np.uint16), "bf16") if d["kdtype"] == "bf16" else (k, "fp8")


def _attn_ref(d, b, j, idx_row, q, swa):
    idx_row = np.asarray(idx_row, dtype=np.int64)
    sel = torch.as_tensor(idx_row[idx_row >= 0], device="cuda")
    return pipeline.attention(u16(q[b, j]), _np(d["kv_fp4"][b][sel]), _np(d["kv_scale"][b][sel]),
                              np.arange(len(sel)), _np(swa[b]), int(d["swa_pos0"][b]),
                              int(d["q_pos"][b, j]), d["sm_scale"],
                              kv_fmt=d.get("kv_fmt", "e8m0_32"))


def _attention(d, q, swa, idx, reuse=False):
    B, n_q = q.shape[0], q.shape[1]
    out = torch.empty(B, n_q, 64, 512, dtype=torch.int16, device="cuda")
    lse = torch.empty(B, n_q, 64, device="cuda")
    fn = csa.reuse_attn if reuse else csa.sparse_attn_decode
    kv_fmt = csa.KV_FP4_E4M3_16 if d.get("kv_fmt") == "e4m3_16" else csa.KV_MXFP4_E8M0_32
    fn(q, d["kv_fp4"], d["kv_scale"], idx, swa, d["swa_pos0"], d["q_pos"], d["sm_scale"], out,
       lse=lse, kv_fmt=kv_fmt)
    return out, lse


def _full_layer(d):
    B, N = d["B"], d["kv_fp4"].shape[1]
    bm = torch.empty(B, 1, (N + 7) // 8, device="cuda")
    csa.index_score(d["q_idx"], d["w_idx"], d["k_idx"], d["vis_len"], block_max=bm)
    pool = torch.empty(B, 1, 2048, dtype=torch.int32, device="cuda")
    csa.block_topk(bm, d["vis_len"], N, 2048, pool)
    idx = torch.empty(B, 1, 512, dtype=torch.int32, device="cuda")
    csa.reindex_topk(csa.MODE_FULL, d["vis_len"], N, 512, idx, q_idx=d["q_idx"], w_idx=d["w_idx"],
                     k_idx=d["k_idx"], pool_blocks=pool)
    out, lse = _attention(d, d["q"], d["swa"], idx)
    torch.cuda.synchronize()
    return pool, idx, out, lse


def _check_full(d, b, pool, idx, out, lse):
    T = int(d["vis_len"][b, 0])
    kr, kd = _kraw(d, b)
    ref = pipeline.full_layer(u16(d["q_idx"][b, 0]), _np(d["w_idx"][b, 0]), kr, kd, T)
    gp = _np(pool[b, 0])
    check_selection(gp, ref["pool"], lambda j: ref["block_max"][j], what=f"pool row {b}")
    pos = otopk.pool_positions(gp, T)
    ri = otopk.pool_topk(ref["scores"][pos], pos, 512)
    gi = _np(idx[b, 0])
    check_selection(gi, ri, lambda t: ref["scores"][t], what=f"idx row {b}")
    # The Full layer's Top-512 is defined over every visible entry: the
    # GPU's in-pool selection must equal the flat Top-512 over [0, T) (up to
    # ties).
    glob = otopk.flat_topk(ref["scores"], T, 512)
    check_selection(gi, glob, lambda t: ref["scores"][t], what=f"global idx row {b}")
    o, l = _attn_ref(d, b, 0, gi, d["q"], d["swa"])
    check_attention(u16(out[b, 0]), _np(lse[b, 0]), o, l, what=f"attention row {b}")
    return gp


def test_tiny_2k():
    d = synth.make("tiny_2k", device="cuda")
    print("workload tiny_2k", flush=True)
    pool, idx, out, lse = _full_layer(d)
    assert np.all(_np(pool[0, 0])[:256] == np.arange(256))   # 256 blocks: all kept
    _check_full(d, 0, pool, idx, out, lse)


def test_full_64k():
    d = synth.make("full_64k", device="cuda")
    print("workload full_64k", flush=True)
    pool, idx, out, lse = _full_layer(d)
    for b in range(d["B"]):
        _check_full(d, b, pool, idx, out, lse)


@pytest.mark.parametrize("name", ["reuse_128k", "reuse_128k_e4m3"])
def test_reuse_128k(name):
    d = synth.make(name, device="cuda")
    print(f"workload {name}", flush=True)
    out, lse = _attention(d, d["q"], d["swa"], d["idx"], reuse=True)
    torch.cuda.synchronize()
    for b in (0, 21, 42, 63):
        o, l = _attn_ref(d, b, 0, _np(d["idx"][b, 0]), d["q"], d["swa"])
        check_attention(u16(out[b, 0]), _np(lse[b, 0]), o, l, what=f"{name} row {b}")


def test_maximum_context():
    # The largest context the boundary accepts: 2^22 entries per sequence,
    # i.e. 524,288 block maxima per row for the block Top-K (whose selection
    # bitmap in LDS is sized for that), and sequence 2's main KV starting
    # 2 GiB into its buffer.  Row 2 is ragged (its last 5 entries not yet
    # visible, the current token the last visible one).
    T = 1 << 22
    d = synth.make("full_reindex_1m", device="cuda", B=3, T=T)
    d["vis_len"][2, 0] = T - 5
    d["q_pos"][2, 0] = T - 6
    print("workload full and reindex layers at 2^22 entries, B=3", flush=True)
    pool, idx, out, lse = _full_layer(d)
    idx2 = torch.empty(d["B"], 1, 512, dtype=torch.int32, device="cuda")
    csa.reindex_topk(csa.MODE_REINDEX, d["vis_len"], T, 512, idx2, q_idx=d["q_idx2"],
                     w_idx=d["w_idx2"], k_idx=d["k_idx"], pool_blocks=pool)
    torch.cuda.synchronize()
    for b in (0, 2):
        gp = _check_full(d, b, pool, idx, out, lse)
        kr, kd = _kraw(d, b)
        re = pipeline.reindex_layer(u16(d["q_idx2"][b, 0]), _np(d["w_idx2"][b, 0]), kr, kd, gp,
                                    int(d["vis_len"][b, 0]))
        key = dict(zip(re["positions"].tolist(), re["scores"].tolist()))
        check_selection(_np(idx2[b, 0]), re["idx"], lambda t: np.array([key[int(x)] for x in t]),
                        what=f"reindex row {b}")


def test_full_reindex_1m():
    d = synth.make("full_reindex_1m", device="cuda")
    print("workload full_reindex_1m", flush=True)
    pool, idx, out, lse = _full_layer(d)
    N = d["kv_fp4"].shape[1]
    idx2 = torch.empty(d["B"], 1, 512, dtype=torch.int32, device="cuda")
    csa.reindex_topk(csa.MODE_REINDEX, d["vis_len"], N, 512, idx2, q_idx=d["q_idx2"],
                     w_idx=d["w_idx2"], k_idx=d["k_idx"], pool_blocks=pool)
    out2, lse2 = _attention(d, d["q2"], d["swa2"], idx2)
    torch.cuda.synchronize()
    for b in (0, 5):
        gp = _check_full(d, b, pool, idx, out, lse)
        kr, kd = _kraw(d, b)
        re = pipeline.reindex_layer(u16(d["q_idx2"][b, 0]), _np(d["w_idx2"][b, 0]), kr, kd, gp, N)
        key = dict(zip(re["positions"].tolist(), re["scores"].tolist()))
        gi2 = _np(idx2[b, 0])
        check_selection(gi2, re["idx"], lambda t: np.array([key[int(x)] for x in t]),
                        what=f"reindex row {b}")
        o, l = _attn_ref(d, b, 0, gi2, d["q2"], d["swa2"])
        check_attention(u16(out2[b, 0]), _np(lse2[b, 0]), o, l, what=f"reindex attention row {b}")


def test_prefill_128k():
    d = synth.make("prefill_128k", device="cuda")
    print("workload prefill_128k", flush=True)
    n_q, N = d["n_q"], d["kv_fp4"].shape[1]
    scores = torch.empty(1, n_q, N, device="cuda")
    csa.index_score(d["q_idx"], d["w_idx"], d["k_idx"], d["vis_len"], scores=scores)
    idx = torch.empty(1, n_q, 512, dtype=torch.int32, device="cuda")
    csa.reindex_topk(csa.MODE_FULL, d["vis_len"], N, 512, idx, scores=scores)
    out, lse = _attention(d, d["q"], d["swa"], idx)
    torch.cuda.synchronize()
    kr, kd = _kraw(d, 0)
    for j in (0, 1, 2047, 4095):
        vis = int(d["vis_len"][0, j])
        ref = pipeline.prefill_topk(u16(d["q_idx"][0, j]), _np(d["w_idx"][0, j]), kr, kd, vis)
        g = _np(scores[0, j, :vis]).astype(np.float64)
        s = ref["scores"]
        assert np.all(np.abs(g - s) <= 1e-5 * np.abs(s) + 1e-6 * np.abs(s).max()), f"scores row {j}"
        gi = _np(idx[0, j])
        check_selection(gi, ref["idx"], lambda t: s[t], what=f"prefill idx row {j}")
        o, l = _attn_ref(d, 0, j, gi, d["q"], d["swa"])
        check_attention(u16(out[0, j]), _np(lse[0, j]), o, l, what=f"prefill attention row {j}")


def test_prefill_past_2g_scores():
    # A prefill call whose score matrix has more than 2^31 elements: 520
    # query rows over the largest accepted context (4,194,304 entries), so
    # the scoring GEMM stores, and the long-row flat Top-k reads, past the
    # 32-bit element range.
    n_q = 520
    d = synth.make("prefill_128k", device="cuda", n_q=n_q, prefix_tokens=2 * ((1 << 22) - n_q // 2))
    N = d["kv_fp4"].shape[1]
    assert N == 1 << 22 and n_q * N > 2 ** 31
    print(f"prefill {n_q} rows x {N} entries", flush=True)
    scores = torch.empty(1, n_q, N, device="cuda")
    csa.index_score(d["q_idx"], d["w_idx"], d["k_idx"], d["vis_len"], scores=scores)
    idx = torch.empty(1, n_q, 512, dtype=torch.int32, device="cuda")
    csa.reindex_topk(csa.MODE_FULL, d["vis_len"], N, 512, idx, scores=scores)
    out, lse = _attention(d, d["q"], d["swa"], idx)
    torch.cuda.synchronize()
    kr, kd = _kraw(d, 0)
    for j in (0, n_q - 1):
        vis = int(d["vis_len"][0, j])
        ref = pipeline.prefill_topk(u16(d["q_idx"][0, j]), _np(d["w_idx"][0, j]), kr, kd, vis)
        g = _np(scores[0, j, :vis]).astype(np.float64)
        s = ref["scores"]
        assert np.all(np.abs(g - s) <= 1e-5 * np.abs(s) + 1e-6 * np.abs(s).max()), f"scores row {j}"
        gi = _np(idx[0, j])
        check_selection(gi, ref["idx"], lambda t: s[t], what=f"prefill idx row {j}")
        o, l = _attn_ref(d, 0, j, gi, d["q"], d["swa"])
        check_attention(u16(out[0, j]), _np(lse[0, j]), o, l, what=f"prefill attention row {j}")


def test_kv_append_past_2g():
    # Appends at the end of the largest accepted context (positions up to
    # 2^22 - 1) in three sequences: the third one's rows sit past 2 GiB into
    # the main-KV buffer.
    N, n_new = 1 << 22, 8
    d = synth.make("kv_append_64k", device="cuda", B=3, n_new=n_new)
    kv_fp4 = torch.zeros(3, N, 256, dtype=torch.uint8, device="cuda")
    kv_scale = torch.zeros(3, N, 16, dtype=torch.uint8, device="cuda")
    pos = torch.full((3,), N - n_new, dtype=torch.int32, device="cuda")
    print("kv append at 2^22 - 8, B=3", flush=True)
    csa.kv_append(d["kv_new"], pos, kv_fp4, kv_scale)
    torch.cuda.synchronize()
    for b in range(3):
        kv = formats.bf16_to_f64(_np(d["kv_new"][b]).view(np.uint16))
        fp4, sc = formats.f64_to_mxfp4(kv)
        assert np.array_equal(_np(kv_fp4[b, N - n_new:]), fp4), f"E2M1 rows of sequence {b}"
        assert np.array_equal(_np(kv_scale[b, N - n_new:]), sc), f"scales of sequence {b}"
        assert not bool(kv_fp4[b, :N - n_new].any()), f"rows outside the append, sequence {b}"


@pytest.mark.parametrize("kv_fmt", ["e8m0_32", "e4m3_16"])
def test_kv_append_64k(kv_fmt):
    # The benchmark's append (4 x 65,536 tokens, window of the last 128), run
    # once on the device; sampled main rows and every window row are checked
    # against the oracle's encoding (placement is covered at small size).
    d = synth.make("kv_append_64k", device="cuda", kv_fmt=kv_fmt)
    print(f"kv_append_64k {kv_fmt}", flush=True)
    fmt = csa.KV_FP4_E4M3_16 if kv_fmt == "e4m3_16" else csa.KV_MXFP4_E8M0_32
    csa.kv_append(d["kv_new"], d["pos"], d["kv_fp4"], d["kv_scale"], swa_new=d["swa_new"],
                  swa_kv=d["swa"], swa_pos0=d["swa_pos0"], kv_fmt=fmt)
    torch.cuda.synchronize()
    rng = np.random.default_rng(53)
    n_new, s_cap = d["n_new"], d["swa"].shape[1]
    for b in range(d["B"]):
        rows = torch.from_numpy(
            np.unique(np.concatenate([rng.integers(0, n_new, 96), [0, n_new - 1]]))).cuda()
        kv = formats.bf16_to_f64(_np(d["kv_new"][b][rows]).view(np.uint16))
        fp4, sc = (formats.f64_to_fp4e4 if kv_fmt == "e4m3_16" else formats.f64_to_mxfp4)(kv)
        assert np.array_equal(_np(d["kv_fp4"][b][rows]), fp4)
        assert np.array_equal(_np(d["kv_scale"][b][rows]), sc)
        sw = formats.bf16_to_f64(_np(d["swa_new"][b, n_new - s_cap:]).view(np.uint16))
        assert np.array_equal(_np(d["swa"][b]), formats.f64_to_e4m3(sw))
