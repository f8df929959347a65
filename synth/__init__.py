"""Seeded synthetic inputs for the CSA2 decode hot path.

This module only draws random tensors and stores them in the formats the
cache holds (bf16, FP8 E4M3FN, MXFP4 = E2M1 + E8M0/32).  It computes none of
the method's arithmetic (no scoring, selection or attention) and is shared by
the tests, the smoke check and the benchmark; neither the oracle nor the HIP
library imports it.

Draws use one torch.Generator per workload on the requested device, in a
fixed order (indexer query, indexer weights, indexer K, K row scaling,
attention query, main KV, SWA KV, supplied indices).  Values from a CPU
generator and a GPU generator differ; each test feeds the same bytes to both
sides.

Quantisation recipes (input preparation, not the method):
  bf16   : round to nearest even (torch cast).
  FP8    : clamp to +-448, then round to nearest even (torch cast to
           float8_e4m3fn).
  MXFP4  : per 32 elements, X = floor(log2(amax)) - 2 (E8M0 code X + 127,
           clamped to [0, 254]; code 0 for an all-zero block); each element
           v / 2^X rounded to nearest even on the E2M1 grid, saturating at 6;
           element 2j in the low nibble of byte j.
"""
import math

import torch

HEADS_IDX, DIM_IDX = 32, 128
HEADS, DIM = 64, 512
WINDOW = 128
TOP_K = 512
K_BLOCKS = 2048
SM_SCALE = 1.0 / math.sqrt(DIM)

# E2M1 rounding thresholds between consecutive magnitudes
# {0, .5, 1, 1.5, 2, 3, 4, 6}; a tie goes to the even code.
_E2M1_MID = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
_E2M1_TIE_UP = (0, 1, 0, 1, 0, 1, 0)


def to_bf16_bits(x):
    """float tensor -> int16 tensor holding the bf16 bit patterns (RNE)."""
    return x.to(torch.bfloat16).view(torch.int16)


def to_fp8_bytes(x):
    """float tensor -> uint8 FP8 E4M3FN codes (saturating at +-448, RNE)."""
    return x.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


def to_mxfp4(x):
    """float tensor [..., D] -> (uint8 [..., D/2] packed E2M1, uint8 [..., D/32] E8M0)."""
    shp = x.shape
    d = shp[-1]
    xb = x.reshape(*shp[:-1], d // 32, 32).to(torch.float32)
    amax = xb.abs().amax(dim=-1, keepdim=True)
    _, ex = torch.frexp(amax)                      # amax = m * 2^ex, m in [0.5, 1)
    xexp = (ex - 1 - 2).clamp(-127, 127)           # floor(log2 amax) - emax(E2M1)
    xexp = torch.where(amax > 0, xexp, torch.full_like(xexp, -127))
    code = (xexp + 127).to(torch.uint8)
    a = (xb.abs() / torch.ldexp(torch.ones_like(amax), xexp.to(torch.float32))).clamp(max=6.0)
    mag = torch.zeros_like(a, dtype=torch.uint8)
    for t, up in zip(_E2M1_MID, _E2M1_TIE_UP):
        mag += (a > t).to(torch.uint8)
        if up:
            mag += (a == t).to(torch.uint8)
    nib = mag | ((xb < 0) & (mag > 0)).to(torch.uint8) << 3
    nib = nib.reshape(*shp[:-1], d)
    packed = nib[..., 0::2] | (nib[..., 1::2] << 4)
    return packed.contiguous(), code.reshape(*shp[:-1], d // 32).contiguous()


def to_fp4_e4m3(x):
    """float tensor [..., D] -> (uint8 [..., D/2] packed E2M1, uint8 [..., D/16]
    E4M3FN scale codes): per 16 elements the scale is amax / 6 cast to
    float8_e4m3fn (round to nearest even, clamped to 448); each element
    |v| / s rounded to nearest even on the E2M1 grid (threshold compares
    against t * s, exact in float32), saturating at 6; element 2j in the low
    nibble of byte j; a block whose scale is 0 stores +0."""
    shp = x.shape
    d = shp[-1]
    xb = x.reshape(*shp[:-1], d // 16, 16).to(torch.float32)
    amax = xb.abs().amax(dim=-1, keepdim=True)
    code = (amax / 6.0).clamp(max=448.0).to(torch.float8_e4m3fn)
    s = code.to(torch.float32)
    a = xb.abs()
    mag = torch.zeros_like(a, dtype=torch.uint8)
    for t, up in zip(_E2M1_MID, _E2M1_TIE_UP):
        thr = t * s
        mag += (a > thr).to(torch.uint8)
        if up:
            mag += (a == thr).to(torch.uint8)
    mag = torch.where(s > 0, mag, torch.zeros_like(mag))
    nib = mag | ((xb < 0) & (mag > 0)).to(torch.uint8) << 3
    nib = nib.reshape(*shp[:-1], d)
    packed = nib[..., 0::2] | (nib[..., 1::2] << 4)
    return packed.contiguous(), code.view(torch.uint8).reshape(*shp[:-1], d // 16).contiguous()


class Gen:
    """A seeded generator bound to one device."""

    def __init__(self, seed, device="cpu"):
        self.device = torch.device(device)
        self.g = torch.Generator(device=self.device)
        self.g.manual_seed(int(seed))

    def normal(self, *shape):
        return torch.randn(*shape, generator=self.g, device=self.device, dtype=torch.float32)

    def uniform(self, *shape):
        return torch.rand(*shape, generator=self.g, device=self.device, dtype=torch.float32)

    def perm(self, n):
        return torch.randperm(n, generator=self.g, device=self.device)


def _normal_mxfp4(gen, b, n, chunk=1 << 18, kv_fmt="e8m0_32"):
    """Main KV [b, n, 512] ~ N(0,1) stored as E2M1 with E8M0 scales per 32
    ("e8m0_32") or E4M3 scales per 16 ("e4m3_16"), drawn in row chunks."""
    enc, per = {"e8m0_32": (to_mxfp4, 32), "e4m3_16": (to_fp4_e4m3, 16)}[kv_fmt]
    fp4 = torch.empty(b, n, DIM // 2, dtype=torch.uint8, device=gen.device)
    sc = torch.empty(b, n, DIM // per, dtype=torch.uint8, device=gen.device)
    for bi in range(b):
        for lo in range(0, n, chunk):
            hi = min(n, lo + chunk)
            p, s = enc(gen.normal(hi - lo, DIM))
            fp4[bi, lo:hi] = p
            sc[bi, lo:hi] = s
    return fp4, sc


def _index_keys(gen, b, n, kdtype, heavy_rows=0, heavy_scale=4.0, lognormal_sigma=None,
                chunk=1 << 18):
    """Indexer K [b, n, 128] ~ N(0,1), optionally with row scaling, stored bf16
    or FP8 ([b, n, 128]), or MXFP4: (a uint8 buffer of b * n * 68 bytes, the
    rows' 64 bytes of E2M1 first, then their 4 E8M0 scales; and the same keys
    as bf16 bits [b, n, 128], the unquantised reference)."""
    if kdtype == "mxfp4":
        ref = _index_keys(gen, b, n, "bf16", heavy_rows, heavy_scale, lognormal_sigma, chunk)
        rows = b * n
        buf = torch.empty(rows * 68, dtype=torch.uint8, device=gen.device)
        e2m1 = buf[:rows * 64].view(rows, 64)
        sc = buf[rows * 64:].view(rows, 4)
        flat = ref.view(rows, DIM_IDX)
        for lo in range(0, rows, chunk):
            hi = min(rows, lo + chunk)
            p, s = to_mxfp4(flat[lo:hi].view(torch.bfloat16).float())
            e2m1[lo:hi] = p
            sc[lo:hi] = s
        return buf, ref
    out_dtype = torch.int16 if kdtype == "bf16" else torch.uint8
    k = torch.empty(b, n, DIM_IDX, dtype=out_dtype, device=gen.device)
    for bi in range(b):
        rowscale = None
        if heavy_rows:
            rowscale = torch.ones(n, device=gen.device)
            rowscale[gen.perm(n)[:heavy_rows]] = heavy_scale
        elif lognormal_sigma is not None:
            rowscale = torch.exp(lognormal_sigma * gen.normal(n))
        for lo in range(0, n, chunk):
            hi = min(n, lo + chunk)
            x = gen.normal(hi - lo, DIM_IDX)
            if rowscale is not None:
                x = x * rowscale[lo:hi, None]
            k[bi, lo:hi] = to_bf16_bits(x) if kdtype == "bf16" else to_fp8_bytes(x)
    return k


def indexer_query(gen, b, n_q=1):
    """(qI int16 bf16-bits [b, n_q, 32, 128], w float32 [b, n_q, 32] ~ U(0,1))."""
    return to_bf16_bits(gen.normal(b, n_q, HEADS_IDX, DIM_IDX)), gen.uniform(b, n_q, HEADS_IDX)


def attn_query(gen, b, n_q=1):
    return to_bf16_bits(gen.normal(b, n_q, HEADS, DIM))


def swa_kv(gen, b, s):
    return to_fp8_bytes(gen.normal(b, s, DIM))


def decode_workload(B, T, kdtype="fp8", seed=0, device="cpu", heavy_frac=0.0,
                    lognormal_sigma=None, reindex=False, supplied_idx=False, kv_fmt="e8m0_32"):
    """Decode step inputs: one query token per sequence at position T-1;
    main KV in scale format kv_fmt ("e8m0_32" or "e4m3_16").

    Full (and optional Reindex) layers share indexer K and main KV; each layer
    has its own indexer query, attention query and SWA KV.
    """
    gen = Gen(seed, device)
    d = {"B": B, "T": T, "n_q": 1, "kdtype": kdtype, "sm_scale": SM_SCALE, "kv_fmt": kv_fmt}
    if not supplied_idx:
        d["q_idx"], d["w_idx"] = indexer_query(gen, B)
        heavy = int(round(heavy_frac * T)) if heavy_frac else 0
        d["k_idx"] = _index_keys(gen, B, T, kdtype, heavy_rows=heavy,
                                 lognormal_sigma=lognormal_sigma)
        if kdtype == "mxfp4":
            # The MXFP4 buffer, and the unquantised keys the recall of the
            # FP4 path is measured against.
            d["k_idx"], d["k_idx_ref"] = d["k_idx"]
        if reindex:
            d["q_idx2"], d["w_idx2"] = indexer_query(gen, B)
    d["q"] = attn_query(gen, B)
    d["kv_fp4"], d["kv_scale"] = _normal_mxfp4(gen, B, T, kv_fmt=kv_fmt)
    s = min(WINDOW, T)
    d["swa"] = swa_kv(gen, B, s)
    if reindex:
        d["q2"] = attn_query(gen, B)
        d["swa2"] = swa_kv(gen, B, s)
    if supplied_idx:
        k = min(TOP_K, T)
        idx = torch.stack([torch.sort(gen.perm(T)[:k]).values for _ in range(B)])
        d["idx"] = idx.to(torch.int32).reshape(B, 1, k)
    d["vis_len"] = torch.full((B, 1), T, dtype=torch.int32, device=gen.device)
    d["swa_pos0"] = torch.full((B,), T - s, dtype=torch.int32, device=gen.device)
    d["q_pos"] = torch.full((B, 1), T - 1, dtype=torch.int32, device=gen.device)
    return d


def decoder_workload(B, T, kdtype="fp8", seed=6, device="cpu", lognormal_sigma=0.5):
    """One decode step through the decoder's 20 layers (layers 20..39): the
    shared indexer K and main KV of `decode_workload`, and per layer its own
    attention query and SWA KV, plus its own indexer query and weights for
    the Full and Reindex layers (layers 20, 24, 28, 32, 36)."""
    d = decode_workload(B=B, T=T, kdtype=kdtype, seed=seed, device=device,
                        lognormal_sigma=lognormal_sigma)
    gen = Gen(seed + 1000, device)
    s = d["swa"].shape[1]
    layers = []
    for layer in range(20, 40):
        e = {"layer": layer, "q": attn_query(gen, B), "swa": swa_kv(gen, B, s)}
        if (layer - 20) % 4 == 0:
            e["q_idx"], e["w_idx"] = indexer_query(gen, B)
        layers.append(e)
    d["layers"] = layers
    return d


def prefill_workload(n_q=4096, prefix_tokens=131072, seed=4, device="cpu", kdtype="bf16",
                     kv_fmt="e8m0_32"):
    """Encoder prefill chunk (m=2): n_q new tokens after a prefix of prefix_tokens.

    Entries: prefix_tokens/2 prefix entries plus n_q/2 chunk entries; token p
    of the chunk (j = p - prefix_tokens) sees entries [0, prefix/2 + (j+1)//2).
    Window: tokens [prefix - W + 1, prefix + n_q - 1].
    """
    gen = Gen(seed, device)
    n_ent = prefix_tokens // 2 + n_q // 2
    d = {"B": 1, "n_q": n_q, "T": n_ent, "kdtype": kdtype, "sm_scale": SM_SCALE,
         "kv_fmt": kv_fmt}
    d["q_idx"], d["w_idx"] = indexer_query(gen, 1, n_q)
    d["k_idx"] = _index_keys(gen, 1, n_ent, kdtype)
    d["q"] = attn_query(gen, 1, n_q)
    d["kv_fp4"], d["kv_scale"] = _normal_mxfp4(gen, 1, n_ent, kv_fmt=kv_fmt)
    swa_lo = prefix_tokens - WINDOW + 1
    s = prefix_tokens + n_q - swa_lo
    d["swa"] = swa_kv(gen, 1, s)
    j = torch.arange(n_q, device=gen.device, dtype=torch.int32)
    d["vis_len"] = (prefix_tokens // 2 + (j + 1) // 2).reshape(1, n_q).to(torch.int32)
    d["swa_pos0"] = torch.full((1,), swa_lo, dtype=torch.int32, device=gen.device)
    d["q_pos"] = (prefix_tokens + j).reshape(1, n_q).to(torch.int32)
    return d


# The workloads, by name: (builder, kwargs).
def kv_append_workload(B, n_new, seed=0, device="cpu", kv_fmt="e8m0_32"):
    """KV append inputs: n_new new tokens per sequence at positions 0 ..
    n_new - 1 (bf16 entries ~N(0,1)), empty caches of n_new main entries and
    a window of the last 128 tokens."""
    gen = Gen(seed, device)
    s = min(WINDOW, n_new)
    d = {"B": B, "n_q": 1, "n_new": n_new, "kv_fmt": kv_fmt}
    d["kv_new"] = to_bf16_bits(gen.normal(B, n_new, DIM))
    d["swa_new"] = to_bf16_bits(gen.normal(B, n_new, DIM))
    d["pos"] = torch.zeros(B, dtype=torch.int32, device=gen.device)
    d["swa_pos0"] = torch.full((B,), n_new - s, dtype=torch.int32, device=gen.device)
    d["kv_fp4"] = torch.zeros(B, n_new, DIM // 2, dtype=torch.uint8, device=gen.device)
    per = {"e8m0_32": 32, "e4m3_16": 16}[kv_fmt]
    d["kv_scale"] = torch.zeros(B, n_new, DIM // per, dtype=torch.uint8, device=gen.device)
    d["swa"] = torch.zeros(B, s, DIM, dtype=torch.uint8, device=gen.device)
    return d


WORKLOADS = {
    "tiny_2k": (decode_workload, dict(B=1, T=2048, kdtype="bf16", seed=0)),
    "full_64k": (decode_workload, dict(B=4, T=65536, kdtype="fp8", seed=1, heavy_frac=0.01)),
    "reuse_128k": (decode_workload, dict(B=64, T=131072, seed=2, supplied_idx=True)),
    "reuse_128k_e4m3": (decode_workload, dict(B=64, T=131072, seed=2, supplied_idx=True,
                                              kv_fmt="e4m3_16")),
    "full_reindex_1m": (decode_workload, dict(B=8, T=1048576, kdtype="fp8", seed=3,
                                              lognormal_sigma=0.5, reindex=True)),
    "prefill_128k": (prefill_workload, dict(n_q=4096, prefix_tokens=131072, seed=4)),
    "kv_append_64k": (kv_append_workload, dict(B=4, n_new=65536, seed=5)),
    "full_reindex_1m_fp4": (decode_workload, dict(B=8, T=1048576, kdtype="mxfp4", seed=3,
                                                  lognormal_sigma=0.5, reindex=True)),
    # The same inputs; the query goes on the FP4 path too (a library option).
    "full_reindex_1m_fp4qk": (decode_workload, dict(B=8, T=1048576, kdtype="mxfp4", seed=3,
                                                    lognormal_sigma=0.5, reindex=True)),
    "decoder_1m": (decoder_workload, dict(B=8, T=1048576, kdtype="fp8", seed=6)),
}


def make(name, device="cpu", **override):
    fn, kw = WORKLOADS[name]
    kw = dict(kw)
    kw.update(override)
    return fn(device=device, **kw)
