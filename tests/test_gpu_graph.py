"""Graph replay of whole hot-path steps.

A decode step (KV append, scan, block Top-K, Full and Reindex selections,
both attentions) and a prefill step (matrix-core scoring, flat Top-K, attention)
are captured into a HIP graph through torch.cuda.CUDAGraph and replayed
several times.  Before the eager reference run and before every replay the
outputs are overwritten with a sentinel, and unrelated eager work runs on
the device between replays; every replay must reproduce the eager result
bit for bit (every kernel is deterministic).
"""
import pytest
import torch

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


def _ws(op, B, n_q, N, top_k, kb):
    n = csa.workspace_size(op, B, n_q, N, top_k, kb)
    return torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")


def _decode_step(d):
    B, N = d["B"], d["k_idx"].shape[1]
    z = lambda *s, dt=torch.int32: torch.empty(*s, dtype=dt, device="cuda")
    o = {
        "bm": z(B, 1, (N + 7) // 8, dt=torch.float32), "pool": z(B, 1, 2048),
        "idx": z(B, 1, 512), "out": z(B, 1, 64, 512, dt=torch.int16),
        "lse": z(B, 1, 64, dt=torch.float32), "idx2": z(B, 1, 512),
        "out2": z(B, 1, 64, 512, dt=torch.int16), "lse2": z(B, 1, 64, dt=torch.float32),
    }
    ws_bt = _ws(csa.OP_BLOCK_TOPK, B, 1, N, 512, 2048)
    ws_re = _ws(csa.OP_REINDEX_TOPK, B, 1, N, 512, 2048)
    ws_at = _ws(csa.OP_SPARSE_ATTN, B, 1, N, 512, 0)
    # The step starts by appending the current token's entries (position
    # N - 1, main and window caches), as a decode step of an engine would.
    g = torch.Generator(device="cuda").manual_seed(23)
    kv_new = synth.to_bf16_bits(torch.randn(B, 1, 512, device="cuda", generator=g))
    swa_new = synth.to_bf16_bits(torch.randn(B, 1, 512, device="cuda", generator=g))
    pos = torch.full((B,), N - 1, dtype=torch.int32, device="cuda")

    def run():
        csa.kv_append(kv_new, pos, d["kv_fp4"], d["kv_scale"], swa_new=swa_new, swa_kv=d["swa"],
                      swa_pos0=d["swa_pos0"])
        csa.index_score(d["q_idx"], d["w_idx"], d["k_idx"], d["vis_len"], block_max=o["bm"])
        csa.block_topk(o["bm"], d["vis_len"], N, 2048, o["pool"], ws=ws_bt)
        csa.reindex_topk(csa.MODE_FULL, d["vis_len"], N, 512, o["idx"], q_idx=d["q_idx"],
                         w_idx=d["w_idx"], k_idx=d["k_idx"], pool_blocks=o["pool"], ws=ws_re)
        csa.sparse_attn_decode(d["q"], d["kv_fp4"], d["kv_scale"], o["idx"], d["swa"],
                               d["swa_pos0"], d["q_pos"], d["sm_scale"], o["out"], lse=o["lse"],
                               ws=ws_at)
        csa.reindex_topk(csa.MODE_REINDEX, d["vis_len"], N, 512, o["idx2"], q_idx=d["q_idx2"],
                         w_idx=d["w_idx2"], k_idx=d["k_idx"], pool_blocks=o["pool"], ws=ws_re)
        csa.sparse_attn_decode(d["q2"], d["kv_fp4"], d["kv_scale"], o["idx2"], d["swa2"],
                               d["swa_pos0"], d["q_pos"], d["sm_scale"], o["out2"],
                               lse=o["lse2"], ws=ws_at)
    return run, o


def _prefill_step(d):
    B, n_q, N = d["B"], d["n_q"], d["k_idx"].shape[1]
    z = lambda *s, dt=torch.int32: torch.empty(*s, dtype=dt, device="cuda")
    o = {
        "scores": z(B, n_q, N, dt=torch.float32), "idx": z(B, n_q, 512),
        "out": z(B, n_q, 64, 512, dt=torch.int16), "lse": z(B, n_q, 64, dt=torch.float32),
    }
    ws_re = _ws(csa.OP_REINDEX_TOPK, B, n_q, N, 512, 0)
    ws_at = _ws(csa.OP_SPARSE_ATTN, B, n_q, N, 512, 0)

    def run():
        csa.index_score(d["q_idx"], d["w_idx"], d["k_idx"], d["vis_len"], scores=o["scores"])
        csa.reindex_topk(csa.MODE_FULL, d["vis_len"], N, 512, o["idx"], scores=o["scores"],
                         ws=ws_re)
        csa.sparse_attn_decode(d["q"], d["kv_fp4"], d["kv_scale"], o["idx"], d["swa"],
                               d["swa_pos0"], d["q_pos"], d["sm_scale"], o["out"], lse=o["lse"],
                               ws=ws_at)
    return run, o


def _poison(o):
    for t in o.values():
        if t.dtype == torch.float32:
            t.fill_(float("nan"))
        else:
            t.fill_(-12345)


def _check_replays(run, o, replays=3):
    # Entries a call leaves unwritten by contract (scores past a row's
    # visible length) keep the sentinel in the reference as in the replays.
    _poison(o)
    run()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in o.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    a = torch.randn(1024, 1024, device="cuda")
    for rep in range(replays):
        # Unrelated eager work between replays, then a sentinel in every output.
        a = torch.tanh(a @ a.T / 1024.0)
        torch.cuda.synchronize()
        _poison(o)
        g.replay()
        torch.cuda.synchronize()
        for k, v in o.items():
            same = torch.equal(v, ref[k]) if v.dtype != torch.float32 else bool(
                (v.view(torch.int32) == ref[k].view(torch.int32)).all())
            assert same, f"replay {rep}: {k} differs from the eager result"


def test_graph_replay_decode_full_reindex():
    d = synth.decode_workload(B=2, T=40000, kdtype="fp8", seed=21, reindex=True, device="cuda")
    print("graph decode B=2 T=40000 fp8 Full+Reindex", flush=True)
    _check_replays(*_decode_step(d))


def test_graph_replay_prefill():
    d = synth.prefill_workload(n_q=64, prefix_tokens=8192, seed=22, device="cuda")
    print("graph prefill n_q=64 prefix=8192 bf16", flush=True)
    _check_replays(*_prefill_step(d))
