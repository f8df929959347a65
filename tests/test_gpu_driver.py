"""The layer driver (csa2_run_layer) over the model's schedule.

The decoder's 20 layers (Full + 3 Reuse, then 4 x (Reindex + 3 Reuse)) and
the encoder's 20 (2 pure-SWA layers, then 3 x (Full + 5 Reuse), prefill
rows) run through the driver; every layer's output must be bit-identical to
the same layer made of the individual calls, which are checked against the
oracle elsewhere; one layer of each mode is also checked against the oracle
directly.
"""
import numpy as np
import pytest
import torch

from _helpers import check_attention, check_selection, u16
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


def _layer_inputs(B, n_q, gen, with_indexer):
    q = synth.to_bf16_bits(gen.normal(B, n_q, 64, 512))
    swa = synth.to_fp8_bytes(gen.normal(B, 128 + n_q - 1, 512))
    qi = synth.to_bf16_bits(gen.normal(B, n_q, 32, 128)) if with_indexer else None
    w = gen.uniform(B, n_q, 32) if with_indexer else None
    return q, swa, qi, w


def test_decoder_layers_through_the_driver():
    B, T = 2, 4096
    d = synth.decode_workload(B=B, T=T, kdtype="fp8", seed=301)
    gen = synth.Gen(302, "cuda")
    cuda = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in d.items()}
    state = csa.LayerState(B, 1, T, k_blocks=256, top_k=512)
    pool_ref = torch.empty(B, 1, 256, dtype=torch.int32, device="cuda")
    idx_ref = torch.empty(B, 1, 512, dtype=torch.int32, device="cuda")
    bm = torch.empty(B, 1, T // 8, device="cuda")
    checked = set()
    for layer in range(20, 40):
        mode = csa.layer_mode(layer)
        q, swa, qi, w = _layer_inputs(B, 1, gen, mode in (csa.MODE_FULL, csa.MODE_REINDEX))
        out = torch.zeros(B, 1, 64, 512, dtype=torch.int16, device="cuda")
        lse = torch.zeros(B, 1, 64, device="cuda")
        print(f"driver decoder layer {layer} mode {mode}", flush=True)
        csa.run_layer(mode, state, cuda["k_idx"], cuda["kv_fp4"], cuda["kv_scale"],
                      cuda["vis_len"], q, swa, cuda["swa_pos0"], cuda["q_pos"], d["sm_scale"], out,
                      lse=lse, q_idx=qi, w_idx=w)
        # The same layer from the individual calls.
        if mode == csa.MODE_FULL:
            csa.index_score(qi, w, cuda["k_idx"], cuda["vis_len"], block_max=bm)
            csa.block_topk(bm, cuda["vis_len"], T, 256, pool_ref)
            csa.reindex_topk(csa.MODE_FULL, cuda["vis_len"], T, 512, idx_ref, q_idx=qi, w_idx=w,
                             k_idx=cuda["k_idx"], pool_blocks=pool_ref)
        elif mode == csa.MODE_REINDEX:
            csa.reindex_topk(csa.MODE_REINDEX, cuda["vis_len"], T, 512, idx_ref, q_idx=qi,
                             w_idx=w, k_idx=cuda["k_idx"], pool_blocks=pool_ref)
        o2 = torch.zeros_like(out)
        l2 = torch.zeros_like(lse)
        csa.sparse_attn_decode(q, cuda["kv_fp4"], cuda["kv_scale"], idx_ref, swa, cuda["swa_pos0"],
                               cuda["q_pos"], d["sm_scale"], o2, lse=l2)
        torch.cuda.synchronize()
        assert np.array_equal(_np(state.idx), _np(idx_ref)), layer
        assert np.array_equal(u16(out), u16(o2)) and np.array_equal(_np(lse), _np(l2)), layer
        if mode in checked:
            continue
        checked.add(mode)
        # Oracle: the layer's selection and attention for row 0.
        k0 = _np(d["k_idx"][0])
        if mode == csa.MODE_FULL:
            ref = pipeline.full_layer(u16(qi[0, 0]), _np(w[0, 0]), k0, "fp8", T, k_blocks=256)
            check_selection(_np(state.idx[0, 0]), ref["idx"], lambda t: ref["scores"][t],
                            what=f"layer {layer} Top-k")
            full_pool = _np(state.pool_blocks[0, 0])
        elif mode == csa.MODE_REINDEX:
            ref = pipeline.reindex_layer(u16(qi[0, 0]), _np(w[0, 0]), k0, "fp8", full_pool, T)
            check_selection(_np(state.idx[0, 0]), ref["idx"],
                            lambda t: pipeline.scores_at(u16(qi[0, 0]), _np(w[0, 0]), k0, "fp8", t),
                            what=f"layer {layer} Top-k")
        sel = _np(state.idx[0, 0])
        sel = sel[sel >= 0]
        o, l = pipeline.attention(u16(q[0, 0]), _np(d["kv_fp4"][0])[sel], _np(d["kv_scale"][0])[sel],
                                  np.arange(len(sel)), _np(swa[0]), int(d["swa_pos0"][0]),
                                  int(d["q_pos"][0, 0]), d["sm_scale"])
        check_attention(u16(out[0, 0]), _np(lse[0, 0]), o, l, what=f"layer {layer}")
    assert checked == {csa.MODE_FULL, csa.MODE_REINDEX, csa.MODE_REUSE}


def test_encoder_layers_through_the_driver():
    # A prefill chunk of 32 query tokens through the encoder's schedule: two
    # window-only layers, then Full (flat Top-k over every visible entry) and
    # Reuse layers.
    n_q = 32
    d = synth.prefill_workload(n_q=n_q, prefix_tokens=4096, seed=303)
    N = d["kv_fp4"].shape[1]
    gen = synth.Gen(304, "cuda")
    cuda = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in d.items()}
    state = csa.LayerState(1, n_q, N, top_k=512)
    scores = torch.empty(1, n_q, N, device="cuda")
    idx_ref = torch.empty(1, n_q, 512, dtype=torch.int32, device="cuda")
    for layer in range(0, 20):
        mode = csa.layer_mode(layer)
        q, _, qi, w = _layer_inputs(1, n_q, gen, mode == csa.MODE_FULL)
        swa = cuda["swa"]
        out = torch.zeros(1, n_q, 64, 512, dtype=torch.int16, device="cuda")
        lse = torch.zeros(1, n_q, 64, device="cuda")
        print(f"driver encoder layer {layer} mode {mode}", flush=True)
        csa.run_layer(mode, state, cuda["k_idx"], cuda["kv_fp4"], cuda["kv_scale"],
                      cuda["vis_len"], q, swa, cuda["swa_pos0"], cuda["q_pos"], d["sm_scale"], out,
                      lse=lse, q_idx=qi, w_idx=w)
        if mode == csa.MODE_FULL:
            csa.index_score(qi, w, cuda["k_idx"], cuda["vis_len"], scores=scores)
            csa.reindex_topk(csa.MODE_FULL, cuda["vis_len"], N, 512, idx_ref, scores=scores)
        o2 = torch.zeros_like(out)
        l2 = torch.zeros_like(lse)
        if mode == csa.MODE_SWA:
            csa.sparse_attn_decode(q, cuda["kv_fp4"], cuda["kv_scale"], None, swa,
                                   cuda["swa_pos0"], cuda["q_pos"], d["sm_scale"], o2, lse=l2)
        else:
            csa.sparse_attn_decode(q, cuda["kv_fp4"], cuda["kv_scale"], idx_ref, swa,
                                   cuda["swa_pos0"], cuda["q_pos"], d["sm_scale"], o2, lse=l2)
        torch.cuda.synchronize()
        assert np.array_equal(u16(out), u16(o2)) and np.array_equal(_np(lse), _np(l2)), layer
        if mode == csa.MODE_SWA and layer == 0:
            # Window-only attention against the oracle with no selected entry.
            j = n_q - 1
            o, l = pipeline.attention(u16(q[0, j]), _np(d["kv_fp4"][0])[:0],
                                      _np(d["kv_scale"][0])[:0], np.arange(0), _np(swa[0]),
                                      int(d["swa_pos0"][0]), int(d["q_pos"][0, j]), d["sm_scale"])
            check_attention(u16(out[0, j]), _np(lse[0, j]), o, l, what="window-only layer")


def test_driver_state_errors():
    B, T = 1, 1024
    d = synth.decode_workload(B=B, T=T, kdtype="fp8", seed=305)
    cuda = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in d.items()}
    state = csa.LayerState(B, 1, T, k_blocks=128, top_k=512)
    out = torch.zeros(B, 1, 64, 512, dtype=torch.int16, device="cuda")
    for mode in (csa.MODE_REUSE, csa.MODE_REINDEX):
        with pytest.raises(csa.Csa2Error) as e:
            csa.run_layer(mode, state, cuda["k_idx"], cuda["kv_fp4"], cuda["kv_scale"],
                          cuda["vis_len"], cuda["q"], cuda["swa"], cuda["swa_pos0"], cuda["q_pos"],
                          d["sm_scale"], out, q_idx=cuda["q_idx"], w_idx=cuda["w_idx"])
        assert e.value.status == 7
