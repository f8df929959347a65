"""Plain fp64 CPU oracle of the CSA2 decode hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this package: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library, its headers or
its binding, and imports nothing from them.

Sources cited in this package (titles of the web pages that describe the
method, with the section on that page):

* "DeepSeek-V4.1-Flash 架构详解：CED、CSA2 与 890 字节 KV Cache"
  (gentlecold.top) -- cited as [架构详解 §n].
* "DeepSeek-V4.1-Flash" research digest (vibe-research.pages.dev) -- cited as
  [研究摘要 §n].
* The DeepSeek-V4 essay at mlqm.cn (news 871487) -- cited as [V4 essay §n].
* "How DeepSeek V4.1 Flash beats 1.6T models" (blog.4sapi.com) -- cited as
  [4sapi, <heading>].

The bit-level number formats (OCP MX v1.0 E2M1 / E8M0, OCP FP8 E4M3FN) are
the public OCP definitions; the pages only name the formats.

Modules:
  formats    -- decoding of bf16, FP8 E4M3FN, E2M1, E8M0 and MXFP4 entries, and
                encoding into FP8 E4M3FN and MXFP4 (the KV append step)
  indexer    -- indexer score and block maximum
  topk       -- block Top-K, pool Top-K (Full / Reindex), flat Top-K
  attention  -- sparse multi-query attention with the SWA window, one softmax,
                optional per-head sink
  pipeline   -- one query's Full / Reindex / Reuse / prefill step from raw bytes,
                and the KV append of new tokens

Every function here is pinned by a CPU test (closed forms, invariants, brute
force, library routines, hand-worked examples); none is marked
"parity unpinned".
"""
from . import formats, indexer, topk, attention, pipeline  # noqa: F401
