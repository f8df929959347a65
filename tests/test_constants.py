"""Constants of the path against the pages' configuration table (CPU only).

[架构详解 §1 config table]: query heads / head dim 64 / 512; CSA2 top-k 512;
indexer heads / dim 32 / 128; hierarchical pool at most 2048 blocks of 8
positions (16384 candidates); SWA window 128; compression encoder 2, decoder
1; maximum context 1,048,576 tokens.
"""
from oracle import attention, indexer, topk
import synth


def test_constants_match_config_table():
    assert (synth.HEADS, synth.DIM) == (64, 512)
    assert (synth.HEADS_IDX, synth.DIM_IDX) == (32, 128)
    assert synth.TOP_K == topk.TOP_K == 512
    assert synth.K_BLOCKS == topk.MAX_POOL_BLOCKS == 2048
    assert indexer.BLOCK == 8 and topk.MAX_POOL_BLOCKS * indexer.BLOCK == 16384
    assert synth.WINDOW == attention.WINDOW == 128


def test_workload_shapes():
    # Decode at the maximum context and the prefill chunk's m=2 entry count.
    assert synth.WORKLOADS["full_reindex_1m"][1]["T"] == 1048576
    n_q, prefix = 4096, 131072
    assert prefix // 2 + n_q // 2 == 67584
