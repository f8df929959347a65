"""Builds libcsa2.so (the C-ABI HIP library) in this package directory for gfx950.

Run as `python -m compressed_sparse_attention_index_amd.build`.  Every source
is compiled with hipcc for gfx950 only, then linked into one shared library.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["api.hip", "index_score.hip", "index_gemm.hip", "topk.hip", "attention.hip",
           "attention_rows.hip", "kv_append.hip", "driver.hip"]
LIB = os.path.join(HERE, "libcsa2.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# Per-source extra flags.  The prefill-scoring and whole-row attention
# kernels work on their MFMA accumulators with vector ALU code; keeping MFMA
# results in ordinary VGPRs (not accumulation registers) avoids copying them
# around.
EXTRA = {"index_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "attention_rows.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{err}")
    return err


def build(verbose=False):
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, *EXTRA.get(s, []), "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        for msg in ex.map(_run, cmds):
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
