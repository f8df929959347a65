"""Comparison helpers shared by the parity tests (no arithmetic of the method)."""
import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

ATTN_ATOL, ATTN_RTOL = 2e-3, 1e-2      # attention output tolerance
TIE_REL = 1e-6                         # selections: ties within 1e-6 of the k-th key


def ensure_built():
    """Builds libcsa2.so if it is missing (the CPU suite may run before a build)."""
    from compressed_sparse_attention_index_amd import LIB_PATH, build
    if not os.path.exists(LIB_PATH):
        build.build()
    return LIB_PATH


def u16(t):
    """torch int16 tensor of bf16 bits -> numpy uint16."""
    return t.detach().cpu().numpy().view(np.uint16)


def check_selection(gpu_ids, oracle_ids, key_of, rel=TIE_REL, what="selection"):
    """Index sets agree except for items within rel of the k-th oracle key.

    gpu_ids / oracle_ids: 1-D int arrays, ascending, -1 padded.  key_of(ids)
    returns the oracle's fp64 keys of the given ids.
    """
    g = np.asarray(gpu_ids, dtype=np.int64)
    o = np.asarray(oracle_ids, dtype=np.int64)
    assert g.shape == o.shape, what
    gv, ov = g[g >= 0], o[o >= 0]
    assert np.all(g[len(gv):] == -1), f"{what}: -1 padding must be at the end"
    assert len(gv) == len(ov), f"{what}: {len(gv)} selected, oracle {len(ov)}"
    assert len(np.unique(gv)) == len(gv), f"{what}: duplicate ids"
    assert np.all(np.diff(gv) > 0), f"{what}: not ascending"
    if np.array_equal(gv, ov):
        return 0
    kth = key_of(ov).min()
    diff = np.setxor1d(gv, ov)
    dk = key_of(diff)
    bad = diff[np.abs(dk - kth) > rel * abs(kth)]
    assert len(bad) == 0, (f"{what}: {len(diff)} ids differ, {len(bad)} outside the tie band; "
                           f"e.g. id {bad[0]} key {key_of(bad[:1])[0]!r} vs k-th {kth!r}")
    return len(diff)


BF16_MIN_SUBNORMAL = 2.0 ** -133


def check_attention(out_bits, lse, o_ref, lse_ref, what="attention", dim_scale=None):
    """|g - o| <= 2e-3 + 1e-2 |o| elementwise; lse within 1e-4 (absolute, relative above 1).

    dim_scale: optional [512] power-of-two scale per output dim (values whose
    entries all carry that scale are compared in units of it; one bf16
    subnormal step, the output's resolution there, is allowed on top)."""
    g = (out_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    floor = 0.0
    if dim_scale is not None:
        g, o_ref = g / dim_scale, o_ref / dim_scale
        floor = BF16_MIN_SUBNORMAL / dim_scale
    err = np.abs(g - o_ref)
    lim = ATTN_ATOL + floor + ATTN_RTOL * np.abs(o_ref)
    worst = np.unravel_index(np.argmax(err - lim), err.shape)
    assert np.all(err <= lim), (f"{what}: max err {err.max():.3e}; worst at {worst}: "
                                f"got {g[worst]:.6f} want {o_ref[worst]:.6f}")
    if lse is not None:
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lse), fin), f"{what}: lse finiteness differs"
        le = np.abs(lse[fin] - lse_ref[fin])
        assert np.all(le <= 1e-4 * np.maximum(1.0, np.abs(lse_ref[fin]))), \
            f"{what}: lse max err {le.max():.3e}"
    return float(err.max())
