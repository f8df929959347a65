"""The allocation-free block Top-K (csa2_block_topk_noalloc, through the C
ABI) gives the same pools as csa2_block_topk on two calls in a row, the
second smaller, on the library's shared scratch array."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _rows(B, nb, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, 1, nb, generator=g)
    x[0, 0, : nb // 3] = torch.round(x[0, 0, : nb // 3] * 2) / 2    # heavy ties in row 0
    return x.cuda()


@pytest.mark.parametrize("first,second", [((8, 1 << 20), (3, 40000)), ((64, 1 << 17), (2, 9000))])
def test_block_topk_noalloc_matches_workspace_version(first, second):
    assert torch.cuda.is_available()
    import compressed_sparse_attention_index_amd as csa
    csa.lib()
    for i, (B, N) in enumerate((first, second)):
        nb = (N + 7) // 8
        bm = _rows(B, nb, 100 + i)
        vis = torch.tensor([N - 37 * j for j in range(B)], dtype=torch.int32).reshape(B, 1).cuda()
        want = torch.full((B, 1, 2048), -7, dtype=torch.int32, device="cuda")
        got = torch.full((B, 1, 2048), -7, dtype=torch.int32, device="cuda")
        print(f"block_topk_noalloc call {i}: B={B} N_cap={N}", flush=True)
        csa.block_topk(bm, vis, N, 2048, want)
        csa.block_topk_noalloc(bm, vis, N, 2048, got)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"call {i}"
        # and the pool is the exact top set of each row (ties by block id)
        for b in (0, B - 1):
            n = (int(vis[b, 0]) + 7) // 8
            keys = bm[b, 0, :n].double().cpu().numpy()
            order = np.lexsort((np.arange(n), -keys))[:2048]
            assert np.array_equal(np.sort(order), got[b, 0].cpu().numpy()[: min(2048, n)])
