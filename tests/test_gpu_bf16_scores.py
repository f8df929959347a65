"""The BF16-score variant (DeepSeek-V4 essay §10.2): index scores stored as
bf16 and the flat Top-k taken over those values.

Parity of the parts that have a definition: each stored score is the
kernel's fp32 score rounded to the nearest bf16 (ties to even), so it equals
torch's cast of the fp32 path's score bit for bit, and lies within one bf16
step of the oracle's bf16 rounding of the fp64 score; the selection over the
stored bf16 values equals the oracle's Top-k over the same values exactly
(ties by position).  The set's recall against the fp32 selection is a
property of the data, checked here only to be high on a small case and
reported by the benchmark.
"""
import numpy as np
import pytest
import torch

from _helpers import u16
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


SENTINEL = 0x7FC1   # a NaN pattern no score produces


def _both(d, vis_t):
    """GPU scores of every row: fp32, and bf16 from the BF16-score scan."""
    B, n_q, N = d["B"], d["n_q"], d["k_idx"].shape[1]
    f32 = torch.full((B, n_q, N), float("nan"), device="cuda")
    b16 = torch.full((B, n_q, N), SENTINEL, dtype=torch.int16, device="cuda")
    q, w, k = d["q_idx"].cuda(), d["w_idx"].cuda(), d["k_idx"].cuda()
    csa.index_score(q, w, k, vis_t, scores=f32)
    csa.index_score_bf16(q, w, k, vis_t, b16)
    torch.cuda.synchronize()
    return f32, b16


def _check_row(f32_row, b16_row, ref, v, what):
    # Bit for bit the rounding of the kernel's own fp32 score ...
    want = _np(f32_row[:v].to(torch.bfloat16).view(torch.int16)).view(np.uint16)
    got = _np(b16_row).view(np.uint16)
    assert np.array_equal(got[:v], want), f"{what}: bf16 != rounding of the fp32 score"
    assert np.all(got[v:] == SENTINEL), f"{what}: scores past vis_len written"
    # ... and within one bf16 step of the oracle's rounding of the fp64 score.
    o = formats.bf16_to_f64(formats.f64_to_bf16(ref))
    g = formats.bf16_to_f64(got[:v])
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(o), 2.0 ** -126))) - 7)
    assert np.all(np.abs(g - o) <= step), f"{what}: more than one bf16 step from the oracle"


@pytest.mark.parametrize("kdtype,T", [("bf16", 2048), ("fp8", 4133)])
def test_scan_bf16_scores_ragged(kdtype, T):
    vis = [0, 1, 7, 33, 513, T - 1, T]
    B = len(vis)
    d = synth.decode_workload(B=B, T=T, kdtype=kdtype, seed=501)
    vis_t = torch.tensor(vis, dtype=torch.int32).reshape(B, 1).cuda()
    print(f"scan bf16 scores {kdtype} T={T}", flush=True)
    f32, b16 = _both(d, vis_t)
    for b, v in enumerate(vis):
        kr, kd = _kraw(d, b)
        ref = pipeline.scores_prefix(u16(d["q_idx"][b, 0]), _np(d["w_idx"][b, 0]), kr, kd, v)
        _check_row(f32[b, 0], b16[b, 0], ref, v, f"row {b}")


@pytest.mark.parametrize("kdtype", ["bf16", "fp8"])
def test_gemm_bf16_scores_prefill_rows(kdtype):
    # 70 prefill rows (several row groups and a ragged one) over 5,000 entries.
    d = synth.prefill_workload(n_q=70, prefix_tokens=5000, seed=502, kdtype=kdtype)
    vis_t = d["vis_len"].cuda()
    print(f"prefill bf16 scores {kdtype}", flush=True)
    f32, b16 = _both(d, vis_t)
    vis = _np(vis_t)[0]
    kr, kd = _kraw(d, 0)
    for j in range(0, 70, 7):
        ref = pipeline.scores_prefix(u16(d["q_idx"][0, j]), _np(d["w_idx"][0, j]), kr, kd, vis[j])
        _check_row(f32[0, j], b16[0, j], ref, vis[j], f"row {j}")


def _flat_case(rows_bits, vis_rows, k):
    """GPU flat Top-k over given bf16 patterns vs the oracle on the same values."""
    R = len(rows_bits)
    N = max(len(x) for x in rows_bits)
    arr = np.zeros((R, 1, N), dtype=np.uint16)
    for i, x in enumerate(rows_bits):
        arr[i, 0, :len(x)] = x
    sc = torch.from_numpy(arr.view(np.int16)).cuda()
    vis = torch.tensor(vis_rows, dtype=torch.int32).reshape(R, 1).cuda()
    out = torch.full((R, 1, k), -7, dtype=torch.int32, device="cuda")
    ks = torch.zeros(R, 1, k, device="cuda")
    csa.flat_topk_bf16(sc, vis, k, out, idx_score=ks)
    torch.cuda.synchronize()
    out, ks = _np(out), _np(ks)
    for i in range(R):
        vals = formats.bf16_to_f64(arr[i, 0])
        want = otopk.flat_topk(vals, vis_rows[i], k)
        assert out[i, 0].tolist() == want.tolist(), f"row {i} vis={vis_rows[i]} k={k}"
        sel = want[want >= 0]
        assert np.array_equal(ks[i, 0, :len(sel)].astype(np.float64), vals[sel])
        assert np.all(np.isneginf(ks[i, 0, len(sel):]))


def _finite_bf16(rng, n, spread):
    # Scores as they come from the scan: bf16 of N(0, spread) values, with
    # many exact repeats once rounded.
    v = rng.standard_normal(n) * spread
    return formats.f64_to_bf16(v)


@pytest.mark.parametrize("n", [5000, 73728, 80000])
def test_flat_topk_bf16_exact_on_the_stored_values(n):
    # Up to 73,728 items the row is held in registers; 80,000 streams.
    rng = np.random.default_rng(503)
    rows = [_finite_bf16(rng, n, 1.0), _finite_bf16(rng, n, 1e-3) ,
            np.full(n, formats.f64_to_bf16(np.array([2.5]))[0], dtype=np.uint16),
            formats.f64_to_bf16(np.round(rng.standard_normal(n) * 4) / 4),
            _finite_bf16(rng, n, 30.0)]
    vis = [n, n - 3, n, 0, 300]
    print(f"flat top-k bf16 n={n}", flush=True)
    for k in (1, 512):
        _flat_case(rows, vis, k)


def test_prefill_bf16_path_against_the_oracle():
    # Scores by the BF16 scan, then the flat Top-k over them: the selection
    # is the oracle's Top-k over the same stored values, and its recall
    # against the oracle's fp32-score selection is high.
    d = synth.prefill_workload(n_q=32, prefix_tokens=6000, seed=504, kdtype="bf16")
    B, n_q, N = d["B"], d["n_q"], d["k_idx"].shape[1]
    vis_t = d["vis_len"].cuda()
    b16 = torch.zeros(B, n_q, N, dtype=torch.int16, device="cuda")
    csa.index_score_bf16(d["q_idx"].cuda(), d["w_idx"].cuda(), d["k_idx"].cuda(), vis_t, b16)
    idx = torch.full((B, n_q, 512), -7, dtype=torch.int32, device="cuda")
    print("prefill bf16 path", flush=True)
    csa.flat_topk_bf16(b16, vis_t, 512, idx)
    torch.cuda.synchronize()
    b16, idx, vis = _np(b16).view(np.uint16), _np(idx), _np(vis_t)[0]
    kr, kd = _kraw(d, 0)
    recalls = []
    for j in range(0, n_q, 5):
        v = vis[j]
        want = otopk.flat_topk(formats.bf16_to_f64(b16[0, j]), v, 512)
        assert idx[0, j].tolist() == want.tolist(), f"row {j}"
        ref = pipeline.prefill_topk(u16(d["q_idx"][0, j]), _np(d["w_idx"][0, j]), kr, kd, v)["idx"]
        r = ref[ref >= 0]
        recalls.append(len(np.intersect1d(r, want[want >= 0])) / max(len(r), 1))
    assert min(recalls) > 0.9, recalls
