#!/usr/bin/env python3
"""Benchmark of the CSA2 decode hot path on one MI355X (gfx950).

One step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM.  Default workload (full_reindex_1m): 8 sequences at
1,048,576 positions of context decode one token each through a decoder Full
layer (indexer scan with fused block maximum -> Top-2048 blocks -> Top-512 in
the 16,384-position pool -> sparse attention over 512 MXFP4 entries plus the
128-token FP8 window) and then a Reindex layer (re-score the pool with the
layer's own indexer query -> Top-512 -> attention with its own query and
window).  Throughput is decode query-tokens per second: B per step.

Prints ONE JSON line on stdout; diagnostics go to stderr.
"""
import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

APPEND_METRIC = "KV append tokens/s (MXFP4 main KV + FP8 window); % of HBM GB/s roofline"
METRIC = "CSA2 decode query-tokens/s at 128K and 1M ctx; % of HBM GB/s roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
# Sources of each dominant kernel: a stored traffic measurement is used only
# while their hash is unchanged.
KERNEL_SOURCES = {
    "index_scan": ["index_score.hip", "index_core.h", "csa2_device.h"],
    "sparse_attn": ["attention.hip", "attention_rows.hip", "csa2_device.h"],
    "index_gemm": ["index_gemm.hip", "index_core.h", "csa2_device.h"],
    "kv_append": ["kv_append.hip", "csa2_device.h"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="full_reindex_1m",
                   choices=["tiny_2k", "full_64k", "reuse_128k", "reuse_128k_e4m3",
                            "full_reindex_1m", "full_reindex_1m_fp4", "full_reindex_1m_fp4qk",
                            "prefill_128k",
                            "kv_append_64k", "decoder_1m"])
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="CPU time budget of the oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true", help="skip the graph-replay measurement")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the 128K points (Reuse decode, prefill chunk) of the default line")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run a 1 GiB device copy (reference for the traffic counters)")
    p.add_argument("--calibrate-mfma", action="store_true",
                   help="also time library bf16 GEMMs (torch.matmul): a square one, the "
                        "practical matrix-core rate, and the indexer contraction unfused")
    return p.parse_args()


def source_hash(kernel):
    """Hash of the code of a kernel's sources: comments and layout are left out,
    since they do not change what the counters measured."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "compressed_sparse_attention_index_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(l.strip() for l in text.splitlines() if l.strip()).encode())
    return h.hexdigest()[:16]


# Per-step inputs read whole by a step, by workload: extra input sets replace
# these (large shared tensors such as the main-KV cache, of which a step
# gathers only the selected rows, are kept).
ROTATED = {
    "tiny_2k": (),
    "full_64k": ("q_idx", "w_idx", "k_idx", "q", "swa"),
    "reuse_128k": ("q", "swa", "idx"),
    "reuse_128k_e4m3": ("q", "swa", "idx"),
    "full_reindex_1m": (),
    "full_reindex_1m_fp4": (),
    "full_reindex_1m_fp4qk": (),
    "prefill_128k": (),
    "kv_append_64k": ("kv_new", "swa_new"),
    "decoder_1m": (),
}
CACHE_BYTES = 256 << 20        # MI355X last-level (Infinity) cache


def rotation_sets(name, d, step_bytes, torch, synth, max_sets=64):
    """Input sets cycled through by consecutive steps so that the bytes the
    steps read between two uses of one set exceed twice the 256 MB
    last-level cache: each timed step then reads its inputs from HBM, not
    from the cache.  Workloads whose step alone reads more (the 1M scan reads
    1 GiB; the prefill chunk reads 0.6 GB) use one set; so does the tiny
    latency-bound configuration."""
    keys = ROTATED[name]
    n = 1 if not keys else min(max_sets, -(-2 * CACHE_BYTES // max(step_bytes, 1)) + 1)
    sets = [d]
    for s in range(1, n):
        if name == "full_64k":
            # Same recipe (heavy-tail keys included), another seed.
            sets.append(synth.make(name, device="cuda", seed=1000 + s))
            continue
        g = synth.Gen(1000 + s, "cuda")
        e = dict(d)
        for k in keys:
            t = d[k]
            if k == "idx":
                T = d["kv_fp4"].shape[1]
                e[k] = torch.stack([torch.sort(g.perm(T)[:t.shape[-1]]).values
                                    for _ in range(t.shape[0])]).to(torch.int32).reshape(t.shape)
            elif t.dtype == torch.uint8:            # FP8 window entries
                e[k] = synth.to_fp8_bytes(g.normal(*t.shape))
            else:                                   # bf16 bits, N(0,1)
                e[k] = synth.to_bf16_bits(g.normal(*t.shape))
        sets.append(e)
    return sets


class Step:
    """Buffers and the launch sequence of one hot-path step (all on one stream)."""

    def __init__(self, name, d, csa, torch, sets=None):
        self.name, self.d, self.csa, self.torch = name, d, csa, torch
        self.sets = sets or [d]
        self.turn = 0
        self._calls = {}
        dev = "cuda"
        B, n_q = d["B"], d["n_q"]
        self.B, self.n_q = B, n_q
        self.rows = B * n_q
        self.N = d["kv_fp4"].shape[1]
        if name == "kv_append_64k":
            self.rows = B * d["n_new"]   # tokens appended per step
            return
        if name == "decoder_1m":
            # The decoder's 20 layers through the layer driver.
            self.state = csa.LayerState(B, n_q, self.N, k_blocks=2048, top_k=512)
            self.out = torch.empty(B, n_q, 64, 512, dtype=torch.int16, device=dev)
            self.lse = torch.empty(B, n_q, 64, dtype=torch.float32, device=dev)
            self.bm = torch.empty(B, n_q, (self.N + 7) // 8, dtype=torch.float32, device=dev)
            return
        z = lambda *s, dt=torch.int32: torch.empty(*s, dtype=dt, device=dev)
        self.out = z(B, n_q, 64, 512, dt=torch.int16)
        self.lse = z(B, n_q, 64, dt=torch.float32)
        self.idx = z(B, n_q, 512)
        self.ws_attn = self._ws(csa.OP_SPARSE_ATTN, 512, 0)
        if name.startswith("reuse_128k"):
            return
        if name == "prefill_128k":
            # The flat Top-512 reads the scores; no block maxima are needed.
            self.bm = None
            self.scores = z(B, n_q, self.N, dt=torch.float32)
            return
        # Full (and Reindex) decode layers through the layer driver; the
        # block maxima of the dominant-kernel loop get their own buffer.
        self.bm = z(B, n_q, (self.N + 7) // 8, dt=torch.float32)
        self.state = csa.LayerState(B, n_q, self.N, k_blocks=2048, top_k=512)
        if "q_idx2" in d:
            self.out2 = z(B, n_q, 64, 512, dt=torch.int16)
            self.lse2 = z(B, n_q, 64, dt=torch.float32)

    def _ws(self, op, top_k, kb):
        n = self.csa.workspace_size(op, self.B, self.n_q, self.N, top_k, kb)
        # Zero-filled once, as the block Top-K workspace expects.
        return self.torch.zeros(max(n, 16), dtype=self.torch.uint8, device="cuda")

    def _next(self):
        d = self.sets[self.turn % len(self.sets)]
        self.turn += 1
        return d

    def _scan(self, d):
        """The scan of input set d (prepared once per set)."""
        key = ("scan", id(d))
        if key not in self._calls:
            self._calls[key] = self.csa.index_score_call(
                d["q_idx"], d["w_idx"], d["k_idx"], d["vis_len"], block_max=self.bm,
                scores=getattr(self, "scores", None))
        self._calls[key].run()

    def dominant(self):
        """Launch only the kernel the roofline figure is about."""
        if self.name == "decoder_1m":
            d = self._next()
            key = ("scan", id(d))
            if key not in self._calls:
                self._calls[key] = self.csa.index_score_call(
                    d["layers"][0]["q_idx"], d["layers"][0]["w_idx"], d["k_idx"], d["vis_len"],
                    block_max=self.bm)
            self._calls[key].run()
        elif self.name == "kv_append_64k":
            self.run()
        elif self.name.startswith("reuse_128k"):
            d = self._next()
            self._attn(d, "reuse", d["q"], d["swa"], d["idx"], self.out, self.lse)
        else:
            self._scan(self._next())

    def _attn(self, d, kind, q, swa, idx, out, lse):
        """An attention call of input set d (prepared once per set and kind)."""
        key = (kind, id(d))
        if key not in self._calls:
            csa = self.csa
            fmt = csa.KV_FP4_E4M3_16 if d.get("kv_fmt") == "e4m3_16" else csa.KV_MXFP4_E8M0_32
            mk = csa.reuse_attn_call if kind == "reuse" else csa.sparse_attn_call
            self._calls[key] = mk(q, d["kv_fp4"], d["kv_scale"], idx, swa, d["swa_pos0"],
                                  d["q_pos"], d["sm_scale"], out, lse=lse, kv_fmt=fmt,
                                  ws=self.ws_attn)
        self._calls[key].run()

    def run(self, full_only=False):
        d, csa = self._next(), self.csa
        if self.name == "decoder_1m":
            if id(d) not in self._calls:
                self._calls[id(d)] = [
                    (csa.layer_mode(e["layer"]),
                     csa.layer_call(self.state, d["k_idx"], d["kv_fp4"], d["kv_scale"],
                                    d["vis_len"], e["q"], e["swa"], d["swa_pos0"], d["q_pos"],
                                    d["sm_scale"], self.out, lse=self.lse, q_idx=e.get("q_idx"),
                                    w_idx=e.get("w_idx")))
                    for e in d["layers"]]
            self.state.struct.has_pool = self.state.struct.has_idx = 0
            for mode, call in self._calls[id(d)]:
                call.run(mode)
            return
        if self.name == "kv_append_64k":
            csa.kv_append(d["kv_new"], d["pos"], d["kv_fp4"], d["kv_scale"], swa_new=d["swa_new"],
                          swa_kv=d["swa"], swa_pos0=d["swa_pos0"])
            return
        if self.name.startswith("reuse_128k"):
            self._attn(d, "reuse", d["q"], d["swa"], d["idx"], self.out, self.lse)
            return
        if self.name == "prefill_128k":
            self._scan(d)
            csa.reindex_topk(csa.MODE_FULL, d["vis_len"], self.N, 512, self.idx, scores=self.scores)
            self._attn(d, "decode", d["q"], d["swa"], self.idx, self.out, self.lse)
            return
        full, reindex = self._layer_calls(d)
        full.run(csa.MODE_FULL)
        if reindex is not None and not full_only:
            reindex.run(csa.MODE_REINDEX)

    def _layer_calls(self, d):
        """The Full (and Reindex) layer calls of an input set, prepared once."""
        key = id(d)
        if key not in self._calls:
            csa = self.csa
            fmt = csa.KV_FP4_E4M3_16 if d.get("kv_fmt") == "e4m3_16" else csa.KV_MXFP4_E8M0_32
            mk = lambda q_idx, w_idx, q, swa, out, lse: csa.layer_call(
                self.state, d["k_idx"], d["kv_fp4"], d["kv_scale"], d["vis_len"], q, swa,
                d["swa_pos0"], d["q_pos"], d["sm_scale"], out, lse=lse, q_idx=q_idx, w_idx=w_idx,
                kv_fmt=fmt)
            full = mk(d["q_idx"], d["w_idx"], d["q"], d["swa"], self.out, self.lse)
            reindex = (mk(d["q_idx2"], d["w_idx2"], d["q2"], d["swa2"], self.out2, self.lse2)
                       if "q_idx2" in d else None)
            self._calls[key] = (full, reindex)
        return self._calls[key]


def algorithmic(name, d):
    """(dominant kernel, its bytes or flops per launch, bound, step bytes) by definition."""
    B, n_q = d["B"], d["n_q"]
    if name == "kv_append_64k":
        # Per token: the bf16 main entry read, its MXFP4 row written; per
        # window row: the bf16 entry read, its FP8 row written; pos, swa_pos0.
        per = B * (d["n_new"] * (1024 + 256 + 16) + d["swa"].shape[1] * (1024 + 512) + 8)
        return "kv_append", per, "hbm", per
    # Per query row: 512 selected entries (256 B of E2M1 plus 16 B of E8M0
    # or 32 B of E4M3 scales), 128 FP8 window entries, q in and out (bf16),
    # the indices and lse.
    entry = 256 + (32 if d.get("kv_fmt") == "e4m3_16" else 16)
    attn_bytes = 512 * entry + 128 * 512 + 64 * 512 * 2 * 2 + 512 * 4 + 64 * 4
    if name.startswith("reuse_128k"):
        per = B * attn_bytes
        return "sparse_attn", per, "hbm", per
    T = d["T"]
    krow = {"fp8": 128, "bf16": 256, "mxfp4": 68}[d["kdtype"]]
    nb = (T + 7) // 8
    if name == "decoder_1m":
        # One scan (Full layer 20), four pool re-scores (Reindex layers), 20
        # attention calls.
        scan = B * (T * krow + 32 * 128 * 2 + 32 * 4 + nb * 4)
        step = (B * (T * krow + 32 * 128 * 2 + 32 * 4) + 4 * B * (16384 * krow + 32 * 128 * 2 + 32 * 4)
                + 20 * B * attn_bytes)
        return "index_scan", scan, "hbm", step
    if name == "prefill_128k":
        vis = d["vis_len"].double().sum().item()
        flops = 2.0 * 32 * 128 * vis
        return "index_gemm", flops, "mfma", None
    scan = B * (T * krow + 32 * 128 * 2 + 32 * 4 + nb * 4)
    step = B * (T * krow + 32 * 128 * 2 + 32 * 4) + B * attn_bytes
    if "q_idx2" in d:
        step += B * (16384 * krow + 32 * 128 * 2 + 32 * 4) + B * attn_bytes
    return "index_scan", scan, "hbm", step


def mxfp4_rows(d, b):
    """Sequence b's MXFP4 indexer keys in the oracle's row layout [T, 68]."""
    import numpy as np
    T, rows = d["T"], d["B"] * d["T"]
    buf = d["k_idx_buf"]
    e2m1 = buf[b * T * 64:(b + 1) * T * 64].view(T, 64)
    sc = buf[rows * 64 + b * T * 4:rows * 64 + (b + 1) * T * 4].view(T, 4)
    return np.concatenate([e2m1.cpu().numpy(), sc.cpu().numpy()], axis=1)


def fp4_recall(d, step):
    """Recall of the FP4 indexer path: the GPU Full layer's Top-512 on MXFP4
    keys (and, with the FP4 query, an MXFP4 query) against the oracle's
    Top-512 on the same keys unquantised (bf16) with the bf16 query, per
    query row; the mean and the minimum over the rows."""
    import numpy as np
    from oracle import pipeline
    step.run(full_only=True)   # the Full layer's Top-512 stays in the layer state
    import torch
    torch.cuda.synchronize()
    rec = []
    for b in range(d["B"]):
        vis = int(d["vis_len"][b, 0])
        ref = pipeline.full_layer(d["q_idx"][b, 0].cpu().numpy().view(np.uint16),
                                  d["w_idx"][b, 0].cpu().numpy(),
                                  d["k_idx_ref"][b].cpu().numpy().view(np.uint16), "bf16", vis)
        want = ref["idx"][ref["idx"] >= 0]
        got = step.state.idx[b, 0].cpu().numpy()
        got = got[got >= 0]
        rec.append(len(np.intersect1d(want, got)) / max(len(want), 1))
    return {"mean": round(float(np.mean(rec)), 5), "min": round(float(np.min(rec)), 5),
            "rows": len(rec),
            "against": "oracle Top-512 over the same keys unquantised (bf16) with the bf16 query, "
                       "fp64 scores"}


def bf16_scores_report(d, csa, torch, steps):
    """The BF16-score variant on the prefill chunk (V4 essay §10.2): the
    scoring call and the flat Top-512 timed with fp32 and with bf16 scores
    (HIP events, back-to-back launches), and the recall of the bf16 path's
    Top-512 against the oracle's fp64 Top-512 on sampled query rows."""
    import numpy as np
    from oracle import pipeline
    B, n_q, N = d["B"], d["n_q"], d["kv_fp4"].shape[1]
    vis = d["vis_len"]
    f32 = torch.empty(B, n_q, N, dtype=torch.float32, device="cuda")
    b16 = torch.empty(B, n_q, N, dtype=torch.int16, device="cuda")
    idx = torch.empty(B, n_q, 512, dtype=torch.int32, device="cuda")
    calls = {
        "scores_fp32": lambda: csa.index_score(d["q_idx"], d["w_idx"], d["k_idx"], vis, scores=f32),
        "scores_bf16": lambda: csa.index_score_bf16(d["q_idx"], d["w_idx"], d["k_idx"], vis, b16),
        "select_fp32": lambda: csa.reindex_topk(csa.MODE_FULL, vis, N, 512, idx, scores=f32),
        "select_bf16": lambda: csa.flat_topk_bf16(b16, vis, 512, idx),
    }
    us = {}
    for key, fn in calls.items():
        fn()
        us[key] = round(timed(torch, fn, max(3, steps // 4))[0] * 1e3, 1)
    calls["scores_bf16"]()
    calls["select_bf16"]()
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    rows = list(range(0, n_q, max(1, n_q // 8)))[:8]
    kr = d["k_idx"][0].cpu().numpy()
    kr = kr.view(np.uint16) if d["kdtype"] == "bf16" else kr
    rec = []
    for j in rows:
        v = int(vis[0, j])
        ref = pipeline.prefill_topk(d["q_idx"][0, j].cpu().numpy().view(np.uint16),
                                    d["w_idx"][0, j].cpu().numpy(), kr, d["kdtype"], v)["idx"]
        r = ref[ref >= 0]
        g = got[0, j][got[0, j] >= 0]
        rec.append(len(np.intersect1d(r, g)) / max(len(r), 1))
    return {"us": us,
            "select_speedup": round(us["select_fp32"] / us["select_bf16"], 3),
            "scores_speedup": round(us["scores_fp32"] / us["scores_bf16"], 3),
            "recall": {"mean": round(float(np.mean(rec)), 5), "min": round(float(np.min(rec)), 5),
                       "rows": len(rec),
                       "against": "oracle Top-512 over fp64 scores (the fp32 path's definition)"}}


def cpu_baseline(name, d, budget_s):
    """The fp64 oracle as it stands, on a bounded sample of the same workload's rows."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info
    from oracle import pipeline

    def npy(t):
        return t.detach().cpu().numpy()

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    B, n_q = d["B"], d["n_q"]
    if name == "kv_append_64k":
        # Chunks of the first sequence's tokens through the oracle's append.
        kv, sw = npy(d["kv_new"][0]).view(np.uint16), npy(d["swa_new"][0]).view(np.uint16)
        n_new, s_cap, chunk = d["n_new"], d["swa"].shape[1], 1024
        done, t_total = 0, 0.0
        while done < n_new and t_total < budget_s:
            m = min(chunk, n_new - done)
            fp4 = np.zeros((1, n_new, 256), np.uint8)
            sc = np.zeros((1, n_new, 16), np.uint8)
            swa = np.zeros((1, s_cap, 512), np.uint8)
            t0 = time.perf_counter()
            pipeline.kv_append(fp4, sc, swa, kv[None, done:done + m], sw[None, done:done + m],
                               np.array([done]), np.array([n_new - s_cap]))
            t_total += time.perf_counter() - t0
            done += m
        return {"value": done / t_total, "unit": "tokens/s", "cores": int(threads),
                "kind": "oracle",
                "sample": f"the first {done} of {B * n_new} appended tokens (sequence 0), "
                          f"{chunk} per call (fp64 numpy, {t_total:.1f} s)"}
    rows = [(b, j) for b in range(B) for j in range(n_q)]
    done, t_total = 0, 0.0
    for b, j in rows:
        kr = None
        if "k_idx" in d:
            kd = d["kdtype"]
            if kd == "mxfp4":
                kr = mxfp4_rows(d, b)
            else:
                kr = npy(d["k_idx"][b])
                if kd == "bf16":
                    kr = kr.view(np.uint16)
        swa = npy(d["swa"][b])
        t0 = time.perf_counter()
        if name == "decoder_1m":
            # The 20 decoder layers of one row: Full, Reindex re-scoring its
            # pool, and every layer's attention over the latest Top-k.
            vis = int(d["vis_len"][b, j])
            kvd = d["kv_fp4"].device
            for e in d["layers"]:
                mode = pipeline.layer_mode(e["layer"])
                if mode == "full":
                    full = pipeline.full_layer(npy(e["q_idx"][b, j]).view(np.uint16),
                                               npy(e["w_idx"][b, j]), kr, kd, vis)
                    idx = full["idx"]
                elif mode == "reindex":
                    idx = pipeline.reindex_layer(npy(e["q_idx"][b, j]).view(np.uint16),
                                                 npy(e["w_idx"][b, j]), kr, kd, full["pool"],
                                                 vis)["idx"]
                sel = torch.from_numpy(idx[idx >= 0]).to(kvd)
                pipeline.attention(npy(e["q"][b, j]).view(np.uint16), npy(d["kv_fp4"][b][sel]),
                                   npy(d["kv_scale"][b][sel]), np.arange(len(sel)),
                                   npy(e["swa"][b]), int(d["swa_pos0"][b]), int(d["q_pos"][b, j]),
                                   d["sm_scale"])
        elif name.startswith("reuse_128k"):
            idx = npy(d["idx"][b, j])
            fp4, sc = npy(d["kv_fp4"][b][d["idx"][b, j].long()]), npy(d["kv_scale"][b][d["idx"][b, j].long()])
            pipeline.attention(npy(d["q"][b, j]).view(np.uint16), fp4, sc, np.arange(len(idx)), swa,
                               int(d["swa_pos0"][b]), int(d["q_pos"][b, j]), d["sm_scale"],
                               kv_fmt=d.get("kv_fmt", "e8m0_32"))
        else:
            vis = int(d["vis_len"][b, j])
            qi, w = npy(d["q_idx"][b, j]).view(np.uint16), npy(d["w_idx"][b, j])
            if name == "prefill_128k":
                idx = pipeline.prefill_topk(qi, w, kr, kd, vis)["idx"]
            else:
                full = pipeline.full_layer(qi, w, kr, kd, vis)
                idx = full["idx"]
            sel = torch.from_numpy(idx[idx >= 0])
            kvd = d["kv_fp4"].device
            fp4 = npy(d["kv_fp4"][b][sel.to(kvd)])
            sc = npy(d["kv_scale"][b][sel.to(kvd)])
            pipeline.attention(npy(d["q"][b, j]).view(np.uint16), fp4, sc, np.arange(len(sel)), swa,
                               int(d["swa_pos0"][b]), int(d["q_pos"][b, j]), d["sm_scale"])
            if "q_idx2" in d:
                re = pipeline.reindex_layer(npy(d["q_idx2"][b, j]).view(np.uint16),
                                            npy(d["w_idx2"][b, j]), kr, kd, full["pool"], vis)
                i2 = re["idx"]
                s2 = torch.from_numpy(i2[i2 >= 0]).to(kvd)
                pipeline.attention(npy(d["q2"][b, j]).view(np.uint16), npy(d["kv_fp4"][b][s2]),
                                   npy(d["kv_scale"][b][s2]), np.arange(len(s2)), npy(d["swa2"][b]),
                                   int(d["swa_pos0"][b]), int(d["q_pos"][b, j]), d["sm_scale"])
        t_total += time.perf_counter() - t0
        done += 1
        if t_total >= budget_s:
            break
    return {"value": done / t_total, "unit": "query-tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} of {len(rows)} query rows of the same workload, all of each row's "
                      f"steps (fp64 numpy, {t_total:.1f} s)"}


def traffic_from_profile(dominant, src_hash, workload):
    # Counters are per launch of one workload's dominant call: they apply only
    # to that workload and only while the kernel's sources are unchanged.
    pdir = os.path.join(ROOT, "profiles")
    for fname in sorted(os.listdir(pdir)):
        if not (fname.startswith(dominant) and fname.endswith("_traffic.json")):
            continue
        with open(os.path.join(pdir, fname)) as f:
            rec = json.load(f)
        if rec.get("source_hash") == src_hash and rec.get("workload") == workload:
            return rec.get("bytes_per_launch")
    return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def timed(torch, fn, steps):
    """`steps` back-to-back calls of fn on the current stream, an event after
    each: (mean ms, p10 ms, p90 ms) of the per-call intervals."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(steps):
        fn()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    q = lambda f: per[min(len(per) - 1, int(round(f * (len(per) - 1))))]
    return evs[0].elapsed_time(evs[steps]) / steps, q(0.1), q(0.9)


def measure(name, args, torch, synth, csa, cpu=True, graph=True, later=None):
    """One workload: input generation, rotated input sets, eager steps, the
    dominant kernel alone, optional graph replay and oracle baseline."""
    t0 = time.time()
    d = synth.make(name, device="cuda")
    if d.get("kdtype") == "mxfp4":
        # The FP4 indexer keys go to the library as one buffer (E2M1 rows,
        # then their scales); the oracle reads them row by row.
        d["k_idx_buf"] = d["k_idx"]
        d["k_idx"] = csa.Mxfp4Keys(d["k_idx"], d["B"] * d["T"], d["T"],
                                   fp4_query=name == "full_reindex_1m_fp4qk")
    dominant, per_launch, bound, step_bytes = algorithmic(name, d)
    sets = rotation_sets(name, d, step_bytes or per_launch, torch, synth)
    torch.cuda.synchronize()
    log(f"[bench] generated {name} on the GPU ({len(sets)} input set(s)) in "
        f"{time.time() - t0:.1f} s")
    step = Step(name, d, csa, torch, sets)

    for _ in range(args.warmup):
        step.run()
    ms, p10, p90 = timed(torch, step.run, args.steps)
    # The dominant call alone: `steps` back-to-back launches on the same
    # stream (rotating input sets like the steps).
    for _ in range(args.warmup):
        step.dominant()
    dom_ms, dom_p10, dom_p90 = timed(torch, step.dominant, args.steps)
    log(f"[bench] {name}: eager {ms * 1e3:.1f} us/step (p10 {p10 * 1e3:.1f}, p90 {p90 * 1e3:.1f}), "
        f"dominant call {dom_ms * 1e3:.1f} us/launch")

    graph_ms = None
    if graph:
        try:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                step.run()
            torch.cuda.current_stream().wait_stream(s)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step.run()
            for _ in range(args.warmup):
                g.replay()
            graph_ms = timed(torch, g.replay, args.steps)[0]
            log(f"[bench] {name}: graph replay {graph_ms * 1e3:.1f} us/step")
        except Exception as exc:  # graph capture is an extra measurement only
            log(f"[bench] graph replay skipped: {exc!r}")

    if args.calibrate_copy:
        # A plain 1 GiB device-to-device copy: rocprofv3's FETCH_SIZE / WRITE_SIZE
        # for it scale the counters of the dominant kernel to bytes.
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    mfma_cal = mfma_calibration(torch, args.steps) if args.calibrate_mfma else None

    append = name == "kv_append_64k"
    rows = step.rows
    unit = "tokens/s" if append else "query-tokens/s"
    if bound == "hbm":
        achieved = per_launch / (dom_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = per_launch / (dom_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
    roof["traffic"] = traffic_from_profile(dominant, source_hash(dominant), name)
    roof["kernel"] = dominant
    roof["per_launch"] = per_launch
    roof["launch_us"] = round(dom_ms * 1e3, 2)
    roof["launch_us_p10_p90"] = [round(dom_p10 * 1e3, 2), round(dom_p90 * 1e3, 2)]

    cpu_rec = None

    def baseline(d=d):   # bound now: the workload's name `d` is deleted below
        t0 = time.time()
        r = cpu_baseline(name, d, args.cpu_seconds)
        r["cpu_model"] = cpu_model()
        log(f"[bench] oracle baseline: {r['value']:.4f} {r['unit']} ({time.time() - t0:.1f} s)")
        return r

    if cpu and later is None:
        cpu_rec = baseline()
    elif cpu:
        # Run after every GPU measurement of the process: the host's BLAS
        # threads stay busy for a while after the oracle and would slow the
        # launching thread of the measurements that follow.
        later.append(baseline)

    T = d["kv_fp4"].shape[1]
    if append:
        cfg = {"workload": name, "batch": d["B"], "tokens_per_sequence": d["n_new"],
               "window": d["swa"].shape[1], "main_kv": "MXFP4 (E2M1 + E8M0/32)", "swa_kv": "FP8 E4M3FN"}
    else:
        reuse = name.startswith("reuse_128k")
        cfg = {"workload": name, "batch": d["B"], "query_rows": rows, "context": T,
               "indexer_k": None if reuse else ("mxfp4 (query mxfp4)" if name == "full_reindex_1m_fp4qk"
                                                else d.get("kdtype")), "top_k": 512,
               "pool_blocks": None if reuse or name == "prefill_128k" else 2048, "window": 128,
               "layers": {"full_64k": "Full", "tiny_2k": "Full", "reuse_128k": "Reuse",
                          "reuse_128k_e4m3": "Reuse", "full_reindex_1m": "Full+Reindex",
                          "full_reindex_1m_fp4": "Full+Reindex (FP4 indexer keys)",
                          "full_reindex_1m_fp4qk": "Full+Reindex (FP4 indexer keys and query)",
                          "prefill_128k": "prefill (m=2)",
                          "decoder_1m": "decoder layers 20-39 (Full + 3 Reuse, "
                                        "4 x (Reindex + 3 Reuse))"}[name],
               "main_kv": ("E2M1 + E4M3/16" if d.get("kv_fmt") == "e4m3_16"
                           else "MXFP4 (E2M1 + E8M0/32)")}
    cfg["input_sets"] = len(sets)
    if step_bytes:
        cfg["step_algorithmic_bytes"] = step_bytes
        cfg["step_hbm_frac"] = round(step_bytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)
    rec = {"value": round(rows / (ms / 1e3), 2), "unit": unit, "ms_per_step": round(ms, 5),
           "ms_per_step_p10": round(p10, 5), "ms_per_step_p90": round(p90, 5),
           "config": cfg, "roofline": roof, "cpu_baseline": cpu_rec}
    if mfma_cal is not None:
        rec["mfma_calibration"] = mfma_cal
    if graph_ms is not None:
        rec["graph_ms_per_step"] = round(graph_ms, 5)
        rec["graph_value"] = round(rows / (graph_ms / 1e3), 2)
    if name == "prefill_128k":
        t0 = time.time()
        rec["bf16_scores"] = bf16_scores_report(d, csa, torch, args.steps)
        log(f"[bench] BF16 scores {rec['bf16_scores']} ({time.time() - t0:.1f} s)")
    if d.get("kdtype") == "mxfp4":
        t0 = time.time()
        key = "recall_fp4_qk" if name == "full_reindex_1m_fp4qk" else "recall_fp4_keys"
        rec[key] = fp4_recall(d, step)
        log(f"[bench] FP4 indexer recall {rec[key]} ({time.time() - t0:.1f} s)")
    del step, sets, d
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def mfma_calibration(torch, steps):
    """Library bf16 GEMMs (torch.matmul, hipBLASLt) timed like the dominant
    calls: an 8192^3 square product, the matrix-core rate a tuned dense GEMM
    reaches here, and the prefill indexer's contraction without its fused
    epilogue (4096 rows x 32 heads against 67,584 keys over 128 dims, bf16
    head scores written out), the unfused alternative's first step."""
    out = {"kernel": "torch.matmul bf16 (hipBLASLt)", "peak_tflops": BF16_PEAK_TFLOPS}
    g = torch.Generator(device="cuda").manual_seed(7)
    for tag, m, k, n in (("square_8192", 8192, 8192, 8192),
                         ("indexer_heads_unfused", 4096 * 32, 128, 67584)):
        a = torch.randn(m, k, device="cuda", generator=g).to(torch.bfloat16)
        b = torch.randn(n, k, device="cuda", generator=g).to(torch.bfloat16)
        bt = b.t().contiguous()   # (k, n)
        c = torch.empty(m, n, device="cuda", dtype=torch.bfloat16)
        fn = lambda: torch.matmul(a, bt, out=c)
        for _ in range(3):
            fn()
        ms = timed(torch, fn, max(3, min(steps, 10)))[0]
        flops = 2.0 * m * k * n
        tf = flops / (ms / 1e3) / 1e12
        out[tag] = {"m": m, "k": k, "n": n, "ms": round(ms, 4), "tflops": round(tf, 1),
                    "frac": round(tf / BF16_PEAK_TFLOPS, 4), "out_bytes": m * n * 2}
        log(f"[bench] calibration {tag}: {ms * 1e3:.1f} us, {tf:.1f} TFLOP/s")
        del a, b, bt, c
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the hot path has no "
              "multi-GPU mode in this build.", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import compressed_sparse_attention_index_amd as csa
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    csa.lib()
    torch.cuda.set_device(0)

    later = []
    head = measure(args.workload, args, torch, synth, csa, cpu=not args.no_cpu_baseline,
                   graph=not args.no_graph, later=later)
    append = args.workload == "kv_append_64k"
    rec = {"metric": APPEND_METRIC if append else METRIC, "value": head["value"],
           "unit": head["unit"], "n_gpus": 1, "steps": args.steps, "warmup": args.warmup}
    rec.update({k: v for k, v in head.items() if k not in ("value", "unit")})
    rec.update({"higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                "dtype": "fp32" if append else "bf16", "data": "synthetic"})
    if args.workload == "full_reindex_1m" and not args.no_extra:
        # The 128K points of the metric: the Reuse-layer decode (B=64) with
        # either main-KV scale format and the encoder prefill chunk, each with
        # its own dominant call's roofline.
        # A Reuse step is about 25 us, so those points time at least 200
        # steps (5 ms): with 20, one slow host launch moved the mean by a
        # third.
        rec["points_128k"] = []
        for w in ("reuse_128k", "reuse_128k_e4m3", "prefill_128k"):
            pa = args
            if w.startswith("reuse"):
                pa = argparse.Namespace(**{**vars(args), "steps": max(args.steps, 200),
                                           "warmup": max(args.warmup, 20)})
            pt = measure(w, pa, torch, synth, csa, cpu=False, graph=False)
            pt["steps"], pt["warmup"] = pa.steps, pa.warmup
            rec["points_128k"].append(pt)
    for job in later:
        rec["cpu_baseline"] = job()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
